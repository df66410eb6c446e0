"""GPU parity of the two forms that split the work differently: the local
transition (gdn_chunk_transition, one GPU's share of a context-parallel
forward) with the context-parallel forward and backward assembled from it on
one GPU, and the backward that recomputes the per-chunk states
(gdn_chunk_bwd_recompute)."""
import sys

import numpy as np
import pytest
import torch

from chunked_gated_delta_04_amd import synth
from tests.gpu_helpers import assert_bar, assert_dg_bar, f64, oracle_backward, oracle_forward, to_dev
from oracle import recurrence as R

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn
else:
    gdn = None


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


SMALL_LENS = [1, 63, 64, 65, 200, 0, 130]


def oracle_transition(inp):
    return R.transition(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                        f64(inp["beta"]), inp["cu_seqlens"].tolist())


def run_transition(inp):
    d = to_dev(inp)
    return gdn.chunk_transition(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                cu_seqlens_host=inp["cu_seqlens"])


# ------------------------------------------------------------------ transition
def test_transition_matches_the_oracle_small_varlen():
    _say("transition small varlen")
    inp = synth.chunk_inputs(SMALL_LENS, 2, 4, seed=81, h0_std=None)
    M, s = run_transition(inp)
    M_ref, s_ref = oracle_transition(inp)
    assert_bar("M", f64(M), M_ref)
    assert_bar("s", f64(s), s_ref)
    eye = torch.eye(128, device="cuda").expand(4, 128, 128)
    assert torch.equal(M[5], eye) and torch.equal(s[5], torch.zeros_like(s[5]))


def test_transition_matches_the_oracle_three_value_heads_per_key_head():
    """Three value heads per key head: the scan grid's last cycle over the XCDs is only
    partly filled, and M's and s's columns run as separate blocks."""
    _say("transition H=3 HV=9")
    inp = synth.chunk_inputs([130, 64, 1], 3, 9, seed=87, h0_std=None)
    M, s = run_transition(inp)
    M_ref, s_ref = oracle_transition(inp)
    assert_bar("M", f64(M), M_ref)
    assert_bar("s", f64(s), s_ref)


def test_transition_end_state_is_the_forward_from_zero_bitwise():
    inp = synth.chunk_inputs(SMALL_LENS, 2, 4, seed=82, h0_std=None)
    _, s = run_transition(inp)
    d = to_dev(inp)
    _, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                             cu_seqlens_host=inp["cu_seqlens"])
    assert torch.equal(s, hT)


def test_transition_maps_any_start_state_to_the_forward_end_state():
    inp = synth.chunk_inputs([300, 64, 129], 1, 2, seed=83, h0_std=0.1)
    M, s = run_transition(inp)
    d = to_dev(inp)
    _, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                             h0=d["h0"], cu_seqlens_host=inp["cu_seqlens"])
    pred = torch.matmul(d["h0"], M) + s
    assert_bar("S0 M + s", f64(pred), f64(hT))


# ------------------------------------------------------------------ context parallel on one GPU
def _shards(inp, cuts):
    """Split one sequence at the given token offsets: the shards become the
    sequences of one pack, in order."""
    T = inp["q"].shape[0]
    bounds = [0] + list(cuts) + [T]
    return dict(q=inp["q"], k=inp["k"], v=inp["v"], g=inp["g"], beta=inp["beta"],
                cu_seqlens=torch.tensor(bounds, dtype=torch.int32)), len(bounds) - 1


def cp_forward(inp, cuts):
    """Context-parallel forward of one sequence, each shard standing for a rank:
    local transitions, the exclusive prefix of the start states (what the
    ranks' exchange computes), then each shard's forward from its start state."""
    sh, R_ = _shards(inp, cuts)
    d = to_dev(sh)
    M, s = gdn.chunk_transition(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                cu_seqlens_host=sh["cu_seqlens"])
    starts = [inp["h0"][0].cuda()]
    for r in range(R_ - 1):
        starts.append(torch.matmul(starts[-1], M[r]) + s[r])
    h_in = torch.stack(starts)
    o, hT, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 h0=h_in, cu_seqlens_host=sh["cu_seqlens"], save_for_backward=True)
    return o, hT[-1], (sh, d, M, h_in, saved)


@pytest.mark.parametrize("cuts", [(512, 1024, 1536), (300, 1000, 1548)])
def test_context_parallel_forward_assembled_from_transitions(cuts):
    _say(f"cp forward cuts={cuts}")
    inp = synth.chunk_inputs([2048], 1, 2, seed=84, h0_std=0.1)
    o, hT, _ = cp_forward(inp, cuts)
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref[0])


def test_context_parallel_backward_assembled_from_transitions():
    """The backward of the same split: each shard's dh0 at zero incoming state
    gradient, the reverse prefix dS_in = dS_out M^T + dh0(0), then each shard's
    backward with its true incoming gradient."""
    _say("cp backward")
    inp = synth.chunk_inputs([2048], 1, 2, seed=85, h0_std=0.1, with_do=True)
    cuts = (300, 1000, 1548)
    o, hT, (sh, d, M, h_in, saved) = cp_forward(inp, cuts)
    Rn = len(cuts) + 1
    do = inp["do"].cuda()
    local = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved, do,
                          cu_seqlens_host=sh["cu_seqlens"])
    dS_out = [None] * Rn
    dS_out[Rn - 1] = torch.zeros(2, 128, 128, device="cuda")
    for r in range(Rn - 1, 0, -1):
        dS_out[r - 1] = torch.matmul(dS_out[r], M[r].transpose(-1, -2)) + local["dh0"][r]
    grads = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved, do,
                          dhT=torch.stack(dS_out).contiguous(), cu_seqlens_host=sh["cu_seqlens"])
    ref = oracle_backward(inp)
    for name in ("dq", "dk", "dv", "dbeta"):
        assert_bar(name, f64(grads[name]), ref[name])
    assert_dg_bar("dg", f64(grads["dg"]), ref["dg"])
    assert_bar("dh0", f64(grads["dh0"][0:1]), ref["dh0"])


def test_transition_full_size_sampled_heads():
    """The bench pack (2 x 8192 tokens, 16 / 32 heads) cut into 8 shards of 2048
    tokens: sampled (shard, value head) pairs against the oracle."""
    _say("transition full size")
    inp = synth.workload_inputs("fwdbwd_2x8192_h16_hv32")
    sh = dict(inp, cu_seqlens=torch.arange(0, 16385, 2048, dtype=torch.int32))
    M, s = run_transition(sh)
    M, s = M.cpu(), s.cpu()
    rng = np.random.default_rng(2)
    for n, hv in [(0, 0), (7, 31)] + [(int(rng.integers(8)), int(rng.integers(32)))
                                      for _ in range(2)]:
        t0, t1 = 2048 * n, 2048 * (n + 1)
        h = hv // 2
        M_ref, s_ref = R.transition(f64(inp["q"][t0:t1, h:h + 1]), f64(inp["k"][t0:t1, h:h + 1]),
                                    f64(inp["v"][t0:t1, hv:hv + 1]), f64(inp["g"][t0:t1, hv:hv + 1]),
                                    f64(inp["beta"][t0:t1, hv:hv + 1]), [0, 2048])
        assert_bar(f"M[{n},{hv}]", f64(M[n, hv]), M_ref[0, 0])
        assert_bar(f"s[{n},{hv}]", f64(s[n, hv]), s_ref[0, 0])


# ------------------------------------------------------------------ recomputing backward
def _bwd_pair(inp, dhT=None):
    d = to_dev(inp)
    host = inp["cu_seqlens"]
    _, _, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                h0=d["h0"], cu_seqlens_host=host, save_for_backward=True)
    dh = None if dhT is None else dhT.cuda()
    a = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved, d["do"],
                      dhT=dh, cu_seqlens_host=host)
    b = gdn.chunk_bwd_recompute(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                d["do"], h0=d["h0"], dhT=dh, cu_seqlens_host=host)
    return a, b


@pytest.mark.parametrize("h0", [True, False])
def test_recomputing_backward_equals_the_saved_one_bitwise(h0):
    _say(f"recompute small h0={h0}")
    inp = synth.chunk_inputs(SMALL_LENS, 2, 4, seed=86, h0_std=0.1 if h0 else None, with_do=True)
    dhT = 0.1 * torch.randn(len(SMALL_LENS), 4, 128, 128, generator=torch.Generator().manual_seed(5))
    a, b = _bwd_pair(inp, dhT)
    for name in a:
        assert torch.equal(a[name], b[name]), name
    ref = oracle_backward(inp, dhT=dhT)
    for name in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert_bar(name, f64(b[name]), ref[name])
    assert_dg_bar("dg", f64(b["dg"]), ref["dg"])


def test_recomputing_backward_full_size_bitwise():
    _say("recompute full size")
    inp = synth.workload_inputs("fwdbwd_2x8192_h16_hv32")
    a, b = _bwd_pair(inp)
    for name in a:
        assert torch.equal(a[name], b[name]), name
