"""GPU parity of the chunk forward/backward (HIP path through the C ABI) with the
fp64 oracle, plus the bitwise invariants the method implies."""
import os
import sys

import numpy as np
import pytest
import torch

from chunked_gated_delta_04_amd import synth
from tests.gpu_helpers import (assert_bar, assert_dg_bar, f64, oracle_backward,
                               oracle_backward_all_heads, oracle_forward,
                               oracle_forward_all_heads, oracle_workers, to_dev)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn
else:
    gdn = None


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def run_fwd(inp, save=False, host_cu=True, stream=None):
    d = to_dev(inp)
    host = inp["cu_seqlens"].to(torch.int32) if host_cu else None
    return gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], h0=d["h0"],
                         cu_seqlens_host=host, save_for_backward=save, stream=stream)


def run_fwd_bwd(inp, dhT=None, stream=None):
    d = to_dev(inp)
    host = inp["cu_seqlens"].to(torch.int32)
    o, hT, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 h0=d["h0"], cu_seqlens_host=host, save_for_backward=True,
                                 stream=stream)
    grads = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved,
                          d["do"], dhT=None if dhT is None else dhT.cuda(), cu_seqlens_host=host,
                          want_dh0=True, stream=stream)
    return o, hT, grads


SMALL_LENS = [1, 63, 64, 65, 200, 130]


def small_inputs(lens=SMALL_LENS, H=2, HV=4, seed=7, h0=True, with_do=False):
    return synth.chunk_inputs(lens, H, HV, seed, h0_std=0.1 if h0 else None, with_do=with_do)


# ------------------------------------------------------------------ forward parity
@pytest.mark.parametrize("h0", [True, False])
def test_forward_matches_oracle_small_varlen(h0):
    _say(f"fwd small varlen h0={h0}")
    inp = small_inputs(h0=h0)
    o, hT, _ = run_fwd(inp)
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)


@pytest.mark.parametrize("H,HV,lens", [(1, 1, [200]), (2, 2, [70, 1]), (3, 9, [130, 64]),
                                        (1, 4, [65, 128, 3])])
def test_forward_matches_oracle_for_head_groups(H, HV, lens):
    """One to four value heads per key head, including chain counts that leave
    part of the scan grid's last cycle over the XCDs empty: the value heads of a key
    head share its normalised q, k tiles, and each applies its own decays."""
    _say(f"fwd head groups H={H} HV={HV} lens={lens}")
    inp = small_inputs(lens=lens, H=H, HV=HV, seed=13)
    o, hT, _ = run_fwd(inp)
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)


def test_forward_matches_oracle_single_head_workload():
    _say("fwd 1x256 h1")
    inp = synth.workload_inputs("fwd_1x256_h1")
    o, hT, _ = run_fwd(inp)
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)


@pytest.mark.parametrize("name", ["fwd_4x4096_h16_hv32", "fwd_varlen12_32768_h16_hv32"])
def test_forward_full_size_all_heads(name):
    """Every (sequence, value head) of the 4 x 4096 pack and of the 12-sequence
    varlen pack against the oracle (run over key-head slices in worker processes;
    about 10-40 s of host time on 16 cores)."""
    _say(f"fwd full {name}: oracle over {oracle_workers()} worker processes")
    inp = synth.workload_inputs(name)
    o, hT, _ = run_fwd(inp)
    o, hT = o.cpu(), hT.cpu()
    import time
    t = time.time()
    o_ref, hT_ref = oracle_forward_all_heads(inp)
    _say(f"  oracle {time.time() - t:.1f} s")
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)


def test_forward_device_only_boundaries_match_host_route_bitwise():
    inp = small_inputs()
    o1, h1, _ = run_fwd(inp, host_cu=True)
    o2, h2, _ = run_fwd(inp, host_cu=False)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("H,HV", [(2, 4), (2, 6)])
def test_forward_saving_for_the_backward_gives_the_same_bits(H, HV):
    """A forward that saves for a backward writes the WY pass's tiles into the
    saved buffer instead of the workspace (and adds T, T^T, gamma, beta); the
    same arithmetic, so o and hT equal the forward without saving bit for bit."""
    inp = small_inputs(H=H, HV=HV)
    o1, h1, _ = run_fwd(inp, save=False)
    o2, h2, saved = run_fwd(inp, save=True)
    assert saved is not None
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_forward_strong_decay_is_finite():
    inp = small_inputs()
    inp["g"] = torch.full_like(inp["g"], -60.0)
    o, hT, _ = run_fwd(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(hT).all()
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)


def test_backward_strong_decay_matches_oracle():
    """g = -60 everywhere (the forget-all case): every decay factor underflows to
    zero, and the gradients stay finite and inside the bar."""
    _say("bwd g=-60")
    inp = small_inputs(with_do=True)
    inp["g"] = torch.full_like(inp["g"], -60.0)
    dhT = 0.1 * torch.randn(len(SMALL_LENS), 4, 128, 128, generator=torch.Generator().manual_seed(4))
    o, hT, grads = run_fwd_bwd(inp, dhT=dhT)
    for name, t in grads.items():
        assert torch.isfinite(t.float()).all(), name
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)
    _check_grads(grads, oracle_backward(inp, dhT=dhT), "g=-60")


def test_backward_with_all_zero_q_and_k_rows_matches_oracle():
    """Rows of q and k that are all zero: the norm then divides by sqrt(1e-6), so
    those rows' gradients are scaled by 1e3 through the norm backward; the
    zero keys write nothing into the state."""
    _say("bwd zero q/k rows")
    inp = small_inputs(with_do=True)
    for t in (0, 5, 64, 127, 200, 450):
        inp["q"][t] = 0
    for t in (3, 63, 64, 130, 201, 520):
        inp["k"][t] = 0
    inp["q"][300, 1] = 0
    inp["k"][301, 0] = 0
    o, hT, grads = run_fwd_bwd(inp)
    for name, t in grads.items():
        assert torch.isfinite(t.float()).all(), name
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)
    ref = oracle_backward(inp)
    for name in ("dv", "dbeta", "dh0"):
        assert_bar(f"zero rows {name}", f64(grads[name]), ref[name])
    assert_dg_bar("zero rows dg", f64(grads["dg"]), ref["dg"])
    # dq, dk: a zero row's norm is sqrt(1e-6) = 1e-3, and the norm backward
    # multiplies that row's gradient by its inverse, 1e3 - the fp32-accumulated
    # bf16-operand error of the normalised gradient with it. Such rows are compared
    # in the normalised coordinates (both sides times the row's norm, which undoes
    # exactly that factor); every other row against the plain bar.
    for name, x in (("dq", "q"), ("dk", "k")):
        xv = f64(inp[x])
        norm = np.sqrt((xv * xv).sum(-1, keepdims=True) + 1e-6)
        zero = (xv == 0).all(-1)
        got, want = f64(grads[name]), ref[name]
        assert zero.sum() > 0
        assert_bar(f"zero rows {name} (nonzero rows)", got[~zero], want[~zero])
        assert_bar(f"zero rows {name} (zero rows, times the row norm)",
                   (got * norm)[zero], (want * norm)[zero])


def test_zero_beta_matches_oracle():
    """beta = 0 writes nothing: U = T diag(beta) V and W vanish on those tokens,
    so the corrected values D are zero there (a whole value head, a whole chunk
    of every head, and single tokens), while dbeta still receives the
    gradient of the write that did not happen."""
    _say("fwd+bwd zero beta")
    inp = small_inputs(with_do=True)
    inp["beta"][:, 1] = 0
    inp["beta"][64:128] = 0
    for t in (0, 5, 63, 200, 450):
        inp["beta"][t] = 0
    o, hT, grads = run_fwd_bwd(inp)
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)
    ref = oracle_backward(inp)
    for name in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert_bar(f"zero beta {name}", f64(grads[name]), ref[name])
    assert_dg_bar("zero beta dg", f64(grads["dg"]), ref["dg"])
    # the head without writes: dv is zero (v never enters the state)
    assert (grads["dv"][:, 1] == 0).all()


# ------------------------------------------------------------------ edge cases
def test_no_tokens_passes_the_state_through():
    H, HV, N = 2, 4, 3
    h0 = 0.1 * torch.randn(N, HV, 128, 128, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    e = torch.empty(0, H, 128, dtype=torch.bfloat16, device="cuda")
    ev = torch.empty(0, HV, 128, dtype=torch.bfloat16, device="cuda")
    eg = torch.empty(0, HV, dtype=torch.float32, device="cuda")
    o, hT, _ = gdn.chunk_fwd(e, e, ev, eg, eg, cu, h0=h0, cu_seqlens_host=cu.cpu())
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(hT, h0)
    o, hT, _ = gdn.chunk_fwd(e, e, ev, eg, eg, cu, h0=None, cu_seqlens_host=cu.cpu())
    assert torch.equal(hT, torch.zeros_like(hT))


def test_zero_length_sequence_inside_a_pack():
    inp = small_inputs(lens=[70, 0, 33])
    o, hT, _ = run_fwd(inp)
    assert torch.equal(hT[1].cpu(), inp["h0"][1])
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)


# ------------------------------------------------------------------ invariants (bitwise)
def test_a_sequence_alone_equals_it_inside_a_pack_bitwise():
    inp = small_inputs(lens=[100, 150, 77])
    o, hT, _ = run_fwd(inp)
    cu = inp["cu_seqlens"].tolist()
    s0, s1 = cu[1], cu[2]
    alone = dict(q=inp["q"][s0:s1], k=inp["k"][s0:s1], v=inp["v"][s0:s1], g=inp["g"][s0:s1],
                 beta=inp["beta"][s0:s1], cu_seqlens=torch.tensor([0, s1 - s0], dtype=torch.int32),
                 h0=inp["h0"][1:2].contiguous())
    o1, h1, _ = run_fwd(alone)
    assert torch.equal(o1, o[s0:s1]) and torch.equal(h1[0], hT[1])


def test_linearity_in_state_and_values_bitwise():
    inp = small_inputs()
    o, hT, _ = run_fwd(inp)
    inp2 = dict(inp, v=(2 * inp["v"].float()).to(torch.bfloat16), h0=2 * inp["h0"])
    o2, h2, _ = run_fwd(inp2)
    assert torch.equal(o2.float(), 2 * o.float()) and torch.equal(h2, 2 * hT)


def test_value_heads_of_one_key_head_with_equal_inputs_agree_bitwise():
    inp = small_inputs(H=1, HV=2)
    for key in ("v", "g", "beta"):
        inp[key][:, 1] = inp[key][:, 0]
    inp["h0"][:, 1] = inp["h0"][:, 0]
    o, hT, _ = run_fwd(inp)
    assert torch.equal(o[:, 0], o[:, 1]) and torch.equal(hT[:, 0], hT[:, 1])


def test_state_carry_across_two_calls():
    """One call equals two calls with the end state carried, at the split points
    of the pages' continuity sweep (AttnGym, 'Paged-state continuity') and
    around chunk edges."""
    TOT = 1700
    lens = [TOT]
    inp = small_inputs(lens=lens, H=1, HV=2)
    o, hT, _ = run_fwd(inp)
    for p in (1, 63, 64, 65, 527, 528, 1056, 1584):
        a = dict(q=inp["q"][:p], k=inp["k"][:p], v=inp["v"][:p], g=inp["g"][:p],
                 beta=inp["beta"][:p], cu_seqlens=torch.tensor([0, p], dtype=torch.int32),
                 h0=inp["h0"])
        oa, ha, _ = run_fwd(a)
        b = dict(q=inp["q"][p:], k=inp["k"][p:], v=inp["v"][p:], g=inp["g"][p:],
                 beta=inp["beta"][p:], cu_seqlens=torch.tensor([0, TOT - p], dtype=torch.int32),
                 h0=ha.cpu())
        ob, hb, _ = run_fwd(b)
        assert_bar(f"o split {p}", f64(torch.cat([oa, ob])), f64(o))
        assert_bar(f"hT split {p}", f64(hb), f64(hT))


# ------------------------------------------------------------------ backward parity
def _check_grads(grads, ref, tag):
    for name in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert_bar(f"{tag} {name}", f64(grads[name]), ref[name])
    assert_dg_bar(f"{tag} dg", f64(grads["dg"]), ref["dg"])


@pytest.mark.parametrize("with_dhT", [False, True])
def test_backward_matches_oracle_small_varlen(with_dhT):
    _say(f"bwd small varlen dhT={with_dhT}")
    inp = small_inputs(with_do=True)
    dhT = 0.1 * torch.randn(len(SMALL_LENS), 4, 128, 128, generator=torch.Generator().manual_seed(3)) \
        if with_dhT else None
    o, hT, grads = run_fwd_bwd(inp, dhT=dhT)
    ref = oracle_backward(inp, dhT=dhT)
    o_ref, _ = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    _check_grads(grads, ref, "small")


@pytest.mark.parametrize("H,HV", [(2, 2), (1, 3), (1, 4)])
def test_backward_matches_oracle_for_other_head_groups(H, HV):
    """One, three and four value heads per key head: the gradient kernel
    walks the value heads of a key head in order, copying the next one's
    states in while it finishes the current one."""
    _say(f"bwd head groups H={H} HV={HV}")
    lens = [1, 64, 130]
    inp = small_inputs(lens=lens, H=H, HV=HV, seed=11, with_do=True)
    dhT = 0.1 * torch.randn(len(lens), HV, 128, 128, generator=torch.Generator().manual_seed(5))
    o, hT, grads = run_fwd_bwd(inp, dhT=dhT)
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)
    ref = oracle_backward(inp, dhT=dhT)
    _check_grads(grads, ref, f"H{H}HV{HV}")


def test_backward_full_size_whole_sequence_and_determinism():
    """The 2 x 8192 pack: run twice (bitwise equal), then every head of its second
    sequence (tokens 8192 .. 16383, all 16 key / 32 value heads) against the
    oracle, over key-head slices in worker processes."""
    _say(f"bwd full 2x8192: oracle over {oracle_workers()} worker processes")
    inp = synth.workload_inputs("fwdbwd_2x8192_h16_hv32")
    o, hT, grads = run_fwd_bwd(inp)
    # bitwise repeat
    o2, hT2, grads2 = run_fwd_bwd(inp)
    assert torch.equal(o, o2) and torch.equal(hT, hT2)
    for kname in grads:
        assert torch.equal(grads[kname], grads2[kname]), kname
    del o2, hT2, grads2
    grads = {kk: vv.cpu() for kk, vv in grads.items()}
    import time
    t = time.time()
    seq = 1
    ref = oracle_backward_all_heads(inp, seq)
    _say(f"  oracle {time.time() - t:.1f} s")
    t0, t1 = inp["cu_seqlens"].tolist()[seq:seq + 2]
    for name in ("dq", "dk", "dv", "dbeta"):
        assert_bar(f"{name}[seq {seq}]", f64(grads[name][t0:t1]), ref[name])
    assert_bar(f"dh0[seq {seq}]", f64(grads["dh0"][seq]), ref["dh0"])
    for hv in range(inp["v"].shape[1]):
        assert_dg_bar(f"dg[seq {seq}, hv {hv}]", f64(grads["dg"][t0:t1, hv]), ref["dg"][:, hv])


def test_backward_with_device_only_boundaries_matches_host_route_bitwise():
    """Without a host copy of cu_seqlens the chunk count is the bound T/64 + N,
    so the table holds unused slots that every backward kernel must skip; the
    results equal those of the exactly sized call bit for bit."""
    _say("bwd device-only boundaries")
    lens = [1, 63, 64, 65, 0, 130]
    inp = small_inputs(lens=lens, seed=13, with_do=True)
    d = to_dev(inp)
    host = inp["cu_seqlens"].to(torch.int32)

    def run(hc):
        o, hT, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                     h0=d["h0"], cu_seqlens_host=hc, save_for_backward=True)
        gr = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved,
                           d["do"], cu_seqlens_host=hc)
        rc = gdn.chunk_bwd_recompute(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                     d["do"], h0=d["h0"], cu_seqlens_host=hc)
        return o, hT, gr, rc
    o1, h1, g1, r1 = run(host)
    o2, h2, g2, r2 = run(None)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for name in g1:
        assert torch.equal(g1[name], g2[name]), name
        assert torch.equal(r1[name], r2[name]), name
        assert torch.equal(g1[name], r1[name]), name


def test_backward_gate_gradients_at_4_byte_aligned_outputs_give_the_same_bits():
    """With an even number of value heads per key head and dg, dbeta 8-byte
    aligned, the gradient pass writes two heads' gate gradients in one store;
    outputs that are only 4-byte aligned take one store per head and must hold
    the same bits."""
    _say("bwd gate gradients at 4-byte aligned outputs")
    inp = small_inputs(H=2, HV=4, with_do=True)
    d = to_dev(inp)
    host = inp["cu_seqlens"].to(torch.int32)
    o, hT, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 h0=d["h0"], cu_seqlens_host=host, save_for_backward=True)
    ref = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved,
                        d["do"], cu_seqlens_host=host)
    T, HV = d["v"].shape[0], d["v"].shape[1]
    N = host.numel() - 1
    dev = d["q"].device
    p = gdn.make_problem(N, T, 2, HV, d["cu_seqlens"], host, 0.0)
    dg = torch.full((T * HV + 1,), float("nan"), dtype=torch.float32, device=dev)[1:].view(T, HV)
    db = torch.full((T * HV + 1,), float("nan"), dtype=torch.float32, device=dev)[1:].view(T, HV)
    assert dg.data_ptr() % 8 == 4 and db.data_ptr() % 8 == 4
    out = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]),
               dv=torch.empty_like(d["v"]), dg=dg, dbeta=db,
               dh0=torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev))
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_size(p), dtype=torch.uint8, device=dev)
    gdn.gdn_chunk_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], saved, d["do"], None,
                      out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], out["dh0"], ws)
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(ref[name], out[name]), name


def test_backward_repeats_bitwise_many_times_and_on_a_side_stream():
    inp = small_inputs(with_do=True)
    o, hT, g0 = run_fwd_bwd(inp)
    side = torch.cuda.Stream()
    for i in range(20):
        if i % 2:
            with torch.cuda.stream(side):
                o2, hT2, g2 = run_fwd_bwd(inp)
        else:
            o2, hT2, g2 = run_fwd_bwd(inp)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(hT, hT2)
        for kname in g0:
            assert torch.equal(g0[kname], g2[kname]), (i, kname)


_CHILD = r"""
import hashlib, sys, torch
sys.path.insert(0, {root!r})
from tests.test_gpu_chunk import small_inputs, run_fwd_bwd
inp = small_inputs(with_do=True)
o, hT, grads = run_fwd_bwd(inp)
h = hashlib.sha256()
for t in [o, hT] + [grads[k] for k in sorted(grads)]:
    h.update(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
print(h.hexdigest())
"""


def test_backward_repeats_bitwise_in_a_fresh_process():
    """The same inputs in a new process (a fresh context, fresh allocations)
    give the same bits (cake_gdn, 'Tests': bit-identical across processes)."""
    import hashlib
    import subprocess
    _say("bwd fresh process")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inp = small_inputs(with_do=True)
    o, hT, grads = run_fwd_bwd(inp)
    h = hashlib.sha256()
    for t in [o, hT] + [grads[k] for k in sorted(grads)]:
        h.update(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    r = subprocess.run([sys.executable, "-c", _CHILD.format(root=root)], capture_output=True,
                       text=True, timeout=240, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == h.hexdigest()
