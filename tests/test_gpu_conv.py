"""GPU parity of the short convolution (gdn_conv_* through the C ABI) with the
fp64 oracle of oracle/conv.py, plus its bitwise invariants: carried states,
the decode update against the forward, paged against gathered states, and
repeatable weight gradients. Every output, the token sums of the weight and bias
gradients included, is held to the pages' elementwise bar atol = rtol = 1e-2
(cake_gdn page, 'Tests')."""
import sys

import numpy as np
import pytest
import torch

from chunked_gated_delta_04_amd import synth
from tests.gpu_helpers import assert_bar, f64, to_dev
from oracle import conv as CV

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn
else:
    gdn = None

LENS = [1, 2, 3, 63, 64, 65, 130, 0, 7]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _act(a):
    return "silu" if a else None


def run_fwd(inp, act="silu", state=True):
    d = to_dev(inp)
    return gdn.conv_fwd(d["x"], d["weight"], d["bias"], d["cu_seqlens"],
                        state_in=d["state_in"], activation=act,
                        cu_seqlens_host=inp["cu_seqlens"], want_state=state)


def oracle_fwd(inp, act="silu"):
    return CV.conv_forward(f64(inp["x"]), f64(inp["weight"]),
                           None if inp["bias"] is None else f64(inp["bias"]),
                           inp["cu_seqlens"].tolist(),
                           None if inp["state_in"] is None else f64(inp["state_in"]), act)


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("act", ["silu", None])
@pytest.mark.parametrize("extras", [(True, True), (False, False)])
def test_forward_matches_the_oracle(W, act, extras):
    bias, state = extras
    _say(f"conv fwd W={W} act={act} bias={bias} state={state}")
    inp = synth.conv_inputs(LENS, 64, W, seed=91 + W, bias=bias, state=state)
    y, so = run_fwd(inp, act)
    y_ref, so_ref = oracle_fwd(inp, act)
    assert_bar("y", f64(y), y_ref)
    assert np.array_equal(f64(so), so_ref)  # end states are copies of inputs


@pytest.mark.parametrize("W", [2, 4])
@pytest.mark.parametrize("act", ["silu", None])
def test_backward_matches_the_oracle_and_repeats_bitwise(W, act):
    _say(f"conv bwd W={W} act={act}")
    inp = synth.conv_inputs(LENS, 64, W, seed=95 + W, bias=True, state=True, with_dy=True)
    d = to_dev(inp)

    def run():
        return gdn.conv_bwd(d["x"], d["weight"], d["bias"], d["cu_seqlens"], d["dy"],
                            state_in=d["state_in"], activation=act,
                            cu_seqlens_host=inp["cu_seqlens"])
    g = run()
    dx, dw, db, ds = CV.conv_backward(f64(inp["x"]), f64(inp["weight"]), f64(inp["bias"]),
                                      inp["cu_seqlens"].tolist(), f64(inp["dy"]),
                                      f64(inp["state_in"]), act)
    assert_bar("dx", f64(g["dx"]), dx)
    assert_bar("dweight", f64(g["dweight"]), dw)
    assert_bar("dbias", f64(g["dbias"]), db)
    assert_bar("dstate", f64(g["dstate"]), ds)
    for _ in range(3):
        g2 = run()
        for k in g:
            assert torch.equal(g[k], g2[k]), k


def test_one_call_equals_two_calls_with_the_state_carried_bitwise():
    inp = synth.conv_inputs([300], 128, 4, seed=97, bias=True, state=True)
    y, so = run_fwd(inp)
    for p in (1, 2, 3, 64, 65, 299):
        a = dict(inp, x=inp["x"][:p], cu_seqlens=torch.tensor([0, p], dtype=torch.int32))
        ya, sa = run_fwd(a)
        b = dict(inp, x=inp["x"][p:], cu_seqlens=torch.tensor([0, 300 - p], dtype=torch.int32),
                 state_in=sa.cpu())
        yb, sb = run_fwd(b)
        assert torch.equal(torch.cat([ya, yb]), y) and torch.equal(sb, so), p


def test_update_steps_equal_the_forward_bitwise_and_skip_the_null_block():
    _say("conv update")
    C, W, T = 256, 4, 9
    inp = synth.conv_inputs([T], C, W, seed=98, bias=True, state=True)
    y, so = run_fwd(inp)
    pool, _ = synth.conv_pool_inputs(3, C, W, slots=6, n_null=0, seed=99)
    pool[4] = inp["state_in"][0]
    pool_d = pool.cuda()
    d = to_dev(inp)
    idx = torch.tensor([0, 4, 0], dtype=torch.int32)
    for t in range(T):
        x3 = torch.stack([d["x"][t], d["x"][t], d["x"][t]])
        yt = gdn.conv_update(x3, d["weight"], d["bias"], pool_d, idx.cuda(), indices_host=idx)
        assert torch.equal(yt[1], y[t]), t
        assert torch.equal(yt[0], torch.zeros_like(yt[0])) and torch.equal(yt[2], yt[0])
    p = pool_d.cpu()
    assert torch.equal(p[4], so[0].cpu())
    keep = [0, 1, 2, 3, 5]
    assert torch.equal(p[keep], pool[keep])


def test_update_matches_the_oracle_at_decode_size():
    _say("conv update 256 rows")
    N, C, W = 256, 8192, 4
    pool, idx = synth.conv_pool_inputs(N, C, W, slots=512, n_null=16, seed=100)
    inp = synth.conv_inputs([N], C, W, seed=101)
    pd = pool.cuda()
    y = gdn.conv_update(inp["x"].cuda(), inp["weight"].cuda(), None, pd, idx.cuda(),
                        indices_host=idx)
    y_ref, pool_ref = CV.conv_update(f64(inp["x"]), f64(inp["weight"]), None, f64(pool), idx.numpy())
    assert_bar("y", f64(y), y_ref)
    assert np.array_equal(f64(pd), pool_ref)


def test_paged_forward_equals_gathered_states_bitwise_and_continues():
    _say("conv paged")
    C, W = 128, 4
    lens = [30, 2, 1, 45, 0, 70]
    inp = synth.conv_inputs(lens, C, W, seed=102, bias=True)
    pool, idx = synth.conv_pool_inputs(len(lens), C, W, slots=12, n_null=1, seed=103)
    init = torch.tensor([1, 0, 1, 1, 0, 1], dtype=torch.int32)
    d = to_dev(inp)
    pd = pool.cuda()
    y = gdn.conv_fwd_paged(d["x"], d["weight"], d["bias"], d["cu_seqlens"], pd, idx.cuda(),
                           has_initial_state=init.cuda(), indices_host=idx,
                           cu_seqlens_host=inp["cu_seqlens"])
    start = torch.zeros(len(lens), C, W - 1, dtype=torch.bfloat16)
    for n, (s, f) in enumerate(zip(idx.tolist(), init.tolist())):
        if s != 0 and f:
            start[n] = pool[s]
    y2, so = run_fwd(dict(inp, state_in=start))
    assert torch.equal(y, y2)
    p = pd.cpu()
    touched = set()
    for n, s in enumerate(idx.tolist()):
        if s != 0:
            assert torch.equal(p[s], so[n].cpu()), n
            touched.add(s)
    for s in range(12):
        if s not in touched:
            assert torch.equal(p[s], pool[s]), s
    y_ref, pool_ref = CV.conv_forward_paged(f64(inp["x"]), f64(inp["weight"]), f64(inp["bias"]),
                                            inp["cu_seqlens"].tolist(), f64(pool), idx.numpy(),
                                            init.numpy())
    assert_bar("y", f64(y), y_ref)
    assert np.array_equal(f64(p), pool_ref)


def test_device_only_boundaries_match_the_host_route_bitwise():
    _say("conv device-only boundaries")
    inp = synth.conv_inputs(LENS, 64, 4, seed=104, bias=True, state=True, with_dy=True)
    d = to_dev(inp)

    def run(hc):
        y, so = gdn.conv_fwd(d["x"], d["weight"], d["bias"], d["cu_seqlens"], state_in=d["state_in"],
                             cu_seqlens_host=hc)
        gr = gdn.conv_bwd(d["x"], d["weight"], d["bias"], d["cu_seqlens"], d["dy"],
                          state_in=d["state_in"], cu_seqlens_host=hc)
        return y, so, gr
    y1, s1, g1 = run(inp["cu_seqlens"])
    y2, s2, g2 = run(None)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_no_tokens():
    C, W = 64, 4
    e = torch.empty(0, C, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(C, W, device="cuda").to(torch.bfloat16)
    cu = torch.zeros(3, dtype=torch.int32)
    st = torch.randn(2, C, W - 1, device="cuda").to(torch.bfloat16)
    y, so = gdn.conv_fwd(e, w, None, cu.cuda(), state_in=st, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(so, st)
    g = gdn.conv_bwd(e, w, None, cu.cuda(), e, state_in=st, cu_seqlens_host=cu)
    assert torch.equal(g["dweight"], torch.zeros_like(g["dweight"]))
    assert torch.equal(g["dstate"], torch.zeros_like(g["dstate"]))


def test_full_size_sampled_channels_and_bitwise_repeat():
    """The training shape (2 x 8192 tokens, 8192 channels, width 4, SiLU):
    sampled channels against the oracle, the whole backward twice."""
    _say("conv full size")
    inp = synth.workload_inputs("conv_2x8192_c8192_w4")
    d = to_dev(inp)
    y, _ = gdn.conv_fwd(d["x"], d["weight"], None, d["cu_seqlens"],
                        cu_seqlens_host=inp["cu_seqlens"], want_state=False)
    g = gdn.conv_bwd(d["x"], d["weight"], None, d["cu_seqlens"], d["dy"],
                     cu_seqlens_host=inp["cu_seqlens"], want_dstate=False)
    g2 = gdn.conv_bwd(d["x"], d["weight"], None, d["cu_seqlens"], d["dy"],
                      cu_seqlens_host=inp["cu_seqlens"], want_dstate=False)
    for k in ("dx", "dweight"):
        assert torch.equal(g[k], g2[k]), k
    cols = [0, 1, 2, 3, 4095, 4096, 8188, 8191] + \
        np.random.default_rng(3).integers(0, 8192, 8).tolist()
    sub = lambda t: f64(t[:, cols])  # noqa: E731
    y_ref, _ = CV.conv_forward(sub(inp["x"]), f64(inp["weight"][cols]), None,
                               inp["cu_seqlens"].tolist())
    assert_bar("y", sub(y.cpu()), y_ref)
    dx, dw, _, _ = CV.conv_backward(sub(inp["x"]), f64(inp["weight"][cols]), None,
                                    inp["cu_seqlens"].tolist(), sub(inp["dy"]))
    assert_bar("dx", sub(g["dx"].cpu()), dx)
    assert_bar("dweight", f64(g["dweight"].cpu()[cols]), dw)
