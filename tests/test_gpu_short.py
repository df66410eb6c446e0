"""GPU parity on packs of many short sequences: hundreds of sequences of 0 to 65
tokens (more sequences than one chunk-table pass of 256 threads covers, most of
them a single short chunk), forward and backward against the fp64 oracle."""
import sys

import numpy as np
import pytest
import torch

from chunked_gated_delta_04_amd import synth
from tests.gpu_helpers import assert_bar, assert_dg_bar, f64, oracle_backward, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn
else:
    gdn = None

SHORT = [0, 1, 2, 3, 5, 17, 33, 64, 65]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def short_pack(n, seed):
    gen = np.random.default_rng(seed)
    return [int(x) for x in gen.choice(SHORT, size=n)]


@pytest.mark.parametrize("n", [260])
def test_many_short_sequences_forward_and_backward(n):
    lens = short_pack(n, seed=n)
    _say(f"short pack: {n} sequences, {sum(lens)} tokens, H=2 HV=4")
    inp = synth.chunk_inputs(lens, 2, 4, seed=31, h0_std=0.1, with_do=True)
    d = to_dev(inp)
    host = inp["cu_seqlens"].to(torch.int32)
    o, hT, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 h0=d["h0"], cu_seqlens_host=host, save_for_backward=True)
    gr = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved,
                       d["do"], cu_seqlens_host=host, want_dh0=True)
    torch.cuda.synchronize()
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)
    ref = oracle_backward(inp)
    for name in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert_bar(name, f64(gr[name]), ref[name])
    assert_dg_bar("dg", f64(gr["dg"]), ref["dg"])
    # a sequence without tokens passes its start state through and gets zero gradients
    empty = [i for i, L in enumerate(lens) if L == 0]
    assert empty
    assert torch.equal(hT[empty].cpu(), inp["h0"][empty])
    assert torch.equal(gr["dh0"][empty].cpu(), torch.zeros_like(inp["h0"][empty]))


def test_three_value_heads_per_key_head_over_many_items():
    """An odd number of value heads per key head (2 key, 6 value heads) over
    more (chunk, key head) items than the gradient pass has workgroups, so that
    workgroups take several items in turn, against the fp64 oracle."""
    gen = np.random.default_rng(9)
    lens = [int(x) for x in gen.integers(0, 41, size=120)]
    H, HV = 2, 6
    items = (sum(lens) // 64 + len(lens)) * H
    _say(f"head groups of 3: {len(lens)} sequences, {sum(lens)} tokens, H={H} HV={HV}, "
         f"{items} items")
    assert items > 256
    inp = synth.chunk_inputs(lens, H, HV, seed=33, h0_std=0.1, with_do=True)
    d = to_dev(inp)
    host = inp["cu_seqlens"].to(torch.int32)
    o, hT, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 h0=d["h0"], cu_seqlens_host=host, save_for_backward=True)
    gr = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], saved,
                       d["do"], cu_seqlens_host=host, want_dh0=True)
    torch.cuda.synchronize()
    o_ref, hT_ref = oracle_forward(inp)
    assert_bar("o", f64(o), o_ref)
    assert_bar("hT", f64(hT), hT_ref)
    ref = oracle_backward(inp)
    for name in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert_bar(name, f64(gr[name]), ref[name])
    assert_dg_bar("dg", f64(gr["dg"]), ref["dg"])
