"""GPU parity of the recurrent decode step (HIP path through the C ABI) with the
fp64 oracle, and its bitwise null-index rules."""
import sys

import numpy as np
import pytest
import torch

from chunked_gated_delta_04_amd import synth
from tests.gpu_helpers import assert_bar, f64, to_dev
from oracle import recurrence as R

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn


def _oracle(inp, pool):
    return R.decode_step(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["a"]),
                         f64(inp["b"]), f64(inp["A_log"]), f64(inp["dt_bias"]), pool,
                         inp["ssm_state_indices"].numpy())


def _run(inp, pool_dev, host=True):
    d = to_dev({k: v for k, v in inp.items() if k != "state_pool"})
    return gdn.recurrent_step(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                              pool_dev, d["ssm_state_indices"],
                              indices_host=inp["ssm_state_indices"] if host else None)


def test_decode_small_matches_oracle_and_skip_rules(contract):
    print("decode small", file=sys.stderr, flush=True)
    inp = synth.decode_inputs(N=12, H=2, HV=4, slots=20, n_null=3, seed=5)
    idx = inp["ssm_state_indices"].clone()
    idx[0] = -3                      # a negative index also skips
    inp["ssm_state_indices"] = idx
    pool0 = inp["state_pool"]
    pool = pool0.cuda()
    o = _run(inp, pool)
    o_ref, pool_ref = _oracle(inp, f64(pool0))
    o, pool = o.cpu(), pool.cpu()
    assert_bar("o", f64(o), o_ref, atol=contract["decode_out_bar_fp32_state"]["value"], rtol=0.0)
    assert np.abs(f64(pool) - pool_ref).max() <= contract["decode_state_bar_fp32_state"]["value"]
    skipped = (idx <= 0).nonzero().flatten().tolist()
    for n in skipped:
        assert torch.equal(o[n], torch.zeros_like(o[n]))
    touched = set(i for i in idx.tolist() if i > 0)
    for s in range(pool.shape[0]):
        if s not in touched:
            assert torch.equal(pool[s], pool0[s]), s
    assert torch.equal(pool[0], pool0[0])


def test_decode_full_workload(contract):
    print("decode full 256 x pool 512", file=sys.stderr, flush=True)
    inp = synth.workload_inputs("decode_256_pool512_h16_hv32")
    pool0 = inp["state_pool"]
    pool = pool0.cuda()
    o = _run(inp, pool)
    o_ref, pool_ref = _oracle(inp, f64(pool0))
    o, pool = o.cpu(), pool.cpu()
    assert_bar("o", f64(o), o_ref, atol=contract["decode_out_bar_fp32_state"]["value"], rtol=0.0)
    dstate = float(np.abs(f64(pool) - pool_ref).max())
    assert dstate <= contract["decode_state_bar_fp32_state"]["value"], dstate
    idx = inp["ssm_state_indices"]
    for n in (idx <= 0).nonzero().flatten().tolist():
        assert torch.equal(o[n], torch.zeros_like(o[n]))
    untouched = sorted(set(range(512)) - set(i for i in idx.tolist() if i > 0))
    assert torch.equal(pool[untouched], pool0[untouched])


def test_decode_rejects_bad_host_indices():
    inp = synth.decode_inputs(N=4, H=1, HV=2, slots=6, n_null=0, seed=9)
    pool = inp["state_pool"].cuda()
    before = pool.clone()
    for bad in ([1, 2, 2, 3], [1, 6, 2, 3]):
        inp["ssm_state_indices"] = torch.tensor(bad, dtype=torch.int32)
        with pytest.raises(gdn.GdnError) as e:
            _run(inp, pool)
        assert e.value.status == 5
    torch.cuda.synchronize()
    assert torch.equal(pool, before)


def test_decode_row_is_batch_invariant_bitwise(contract):
    """A row's output and state block are the same bits alone or at any position
    of a batch of 64 (RL-Kernel PR #469, 'Results', L1)."""
    rows = contract["batch_invariance_rows"]["value"]
    B = contract["batch_invariance_rows"]["batch"]
    inp = synth.decode_inputs(N=B, H=2, HV=4, slots=B + 1, n_null=0, seed=11)
    inp["ssm_state_indices"] = torch.arange(1, B + 1, dtype=torch.int32)
    pool_b = inp["state_pool"].cuda()
    o_b = _run(inp, pool_b)
    for r in rows:
        one = {k: (v[r:r + 1] if k in ("q", "k", "v", "a", "b", "ssm_state_indices") else v)
               for k, v in inp.items()}
        pool_1 = inp["state_pool"].cuda()
        o_1 = _run(one, pool_1)
        slot = r + 1
        assert torch.equal(o_1[0], o_b[r]) and torch.equal(pool_1[slot], pool_b[slot])


def test_decode_steps_track_the_chunk_forward(contract):
    """T decode steps on one slot agree with one chunk forward over the same T tokens
    to about 1 % relative (RL-Kernel PR #469, 'Decode versus chunked prefill')."""
    for T in contract["decode_vs_chunk_T"]["value"]:
        H, HV = 2, 4
        gen = torch.Generator().manual_seed(T)
        q = torch.randn(T, H, 128, generator=gen).to(torch.bfloat16)
        k = torch.randn(T, H, 128, generator=gen).to(torch.bfloat16)
        v = torch.randn(T, HV, 128, generator=gen).to(torch.bfloat16)
        a = torch.randn(T, HV, generator=gen).to(torch.bfloat16)
        b = torch.randn(T, HV, generator=gen).to(torch.bfloat16)
        A_log = torch.empty(HV).uniform_(0, np.log(16), generator=gen)
        dt_bias = torch.zeros(HV)
        g, beta = R.decode_gating(f64(a), f64(b), f64(A_log), f64(dt_bias))
        pool = torch.zeros(2, HV, 128, 128, device="cuda")
        outs = []
        for t in range(T):
            outs.append(gdn.recurrent_step(q[t:t + 1].cuda(), k[t:t + 1].cuda(), v[t:t + 1].cuda(),
                                           a[t:t + 1].cuda(), b[t:t + 1].cuda(), A_log.cuda(),
                                           dt_bias.cuda(), pool,
                                           torch.tensor([1], dtype=torch.int32, device="cuda")))
        o_dec = torch.cat(outs).float()
        cu = torch.tensor([0, T], dtype=torch.int32)
        o_ch, hT, _ = gdn.chunk_fwd(q.cuda(), k.cuda(), v.cuda(),
                                    torch.tensor(g, dtype=torch.float32).cuda(),
                                    torch.tensor(beta, dtype=torch.float32).cuda(), cu.cuda(),
                                    cu_seqlens_host=cu)
        # the upper end of the pages' measured 0.5-1 % band
        bar = max(contract["decode_vs_chunk_rel"]["value"])
        rel = float((o_dec - o_ch.float()).abs().max() / o_ch.float().abs().max())
        assert rel < bar, (T, rel)
        srel = float((pool[1] - hT[0]).abs().max() / hT[0].abs().max())
        assert srel < bar, (T, srel)
