"""One long sequence (65,536 and 131,072 tokens, 16 key / 32 value heads): the
long-context rows of the Cake page's tests ("[Cake 1/13] gdn", miles-ext-kernels
PR #1, "Tests": single sequences of 32k to 128k tokens).

* Sampled heads against the oracle at 65,536 tokens: the forward of two key
  heads (four value heads) and the backward of one key head, each over the
  whole sequence, run in worker processes while the GPU computes.
* At both lengths and over every head, one call equals two calls split at a
  chunk boundary with the state carried (forward: hT -> h0; backward: the
  second half's dh0 -> the first half's dhT), bit for bit: the chunk grid and
  the fp32 running states at the split are the same, so the arithmetic is.
"""
import sys

import pytest
import torch

from chunked_gated_delta_04_amd import synth
from tests.gpu_helpers import (_pool, _slice_backward, _slice_forward, assert_bar, assert_dg_bar,
                               f64)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _fwd_bwd(d, lo, hi, h0, dhT):
    """gdn forward + backward over tokens [lo, hi) of the single sequence."""
    cu = torch.tensor([0, hi - lo], dtype=torch.int32)
    sl = slice(lo, hi)
    o, hT, saved = gdn.chunk_fwd(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl], d["beta"][sl],
                                 cu.cuda(), h0=h0, cu_seqlens_host=cu, save_for_backward=True)
    gr = gdn.chunk_bwd(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl], d["beta"][sl], cu.cuda(),
                       saved, d["do"][sl], dhT=dhT, cu_seqlens_host=cu)
    del saved
    return o, hT, gr


def test_long_sequence_sampled_heads_match_the_oracle():
    name = "fwdbwd_1x65536_h16_hv32"
    inp = synth.workload_inputs(name)
    T = inp["q"].shape[0]
    fwd_heads, bwd_head = (0, 15), 7       # key heads checked (value heads 2h, 2h + 1)
    _say(f"long {name}: oracle forward for key heads {fwd_heads}, backward for {bwd_head}, "
         "in worker processes")

    def sl(h, with_do):
        hvs = slice(2 * h, 2 * h + 2)
        a = [f64(inp["q"][:, h:h + 1]), f64(inp["k"][:, h:h + 1]), f64(inp["v"][:, hvs]),
             f64(inp["g"][:, hvs]), f64(inp["beta"][:, hvs]), [0, T]]
        if with_do:
            return tuple(a + [f64(inp["do"][:, hvs]), f64(inp["h0"][:, hvs]), None])
        return tuple(a + [f64(inp["h0"][:, hvs])])

    with _pool() as ex:
        fut_f = [ex.submit(_slice_forward, sl(h, False)) for h in fwd_heads]
        fut_b = ex.submit(_slice_backward, sl(bwd_head, True))
        d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        o, hT, gr = _fwd_bwd(d, 0, T, d["h0"], None)
        o, hT = o.cpu(), hT.cpu()
        gr = {k: v.cpu() for k, v in gr.items()}
        del d
        for h, fut in zip(fwd_heads, fut_f):
            o_ref, hT_ref = fut.result()
            hvs = slice(2 * h, 2 * h + 2)
            assert_bar(f"o[key head {h}]", f64(o[:, hvs]), o_ref)
            assert_bar(f"hT[key head {h}]", f64(hT[:, hvs]), hT_ref)
            _say(f"  forward key head {h} ok")
        ref = fut_b.result()
    h = bwd_head
    hvs = slice(2 * h, 2 * h + 2)
    assert_bar("dq", f64(gr["dq"][:, h]), ref["dq"][:, 0])
    assert_bar("dk", f64(gr["dk"][:, h]), ref["dk"][:, 0])
    assert_bar("dv", f64(gr["dv"][:, hvs]), ref["dv"])
    assert_bar("dbeta", f64(gr["dbeta"][:, hvs]), ref["dbeta"])
    assert_bar("dh0", f64(gr["dh0"][:, hvs]), ref["dh0"])
    for j in range(2):
        assert_dg_bar(f"dg[value head {2 * h + j}]", f64(gr["dg"][:, 2 * h + j]), ref["dg"][:, j])


@pytest.mark.parametrize("name", ["fwdbwd_1x65536_h16_hv32", "fwdbwd_1x131072_h16_hv32"])
def test_long_sequence_split_with_carried_state_is_bitwise_equal(name):
    inp = synth.workload_inputs(name)
    T = inp["q"].shape[0]
    split = T // 2 + 64 * 7                 # a chunk boundary off the middle
    _say(f"long {name}: one call vs two calls split at {split}")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, hT, gr = _fwd_bwd(d, 0, T, d["h0"], None)
    oa, ha, _ = gdn.chunk_fwd(d["q"][:split], d["k"][:split], d["v"][:split], d["g"][:split],
                              d["beta"][:split], torch.tensor([0, split], dtype=torch.int32).cuda(),
                              h0=d["h0"])
    ob, hb, grb = _fwd_bwd(d, split, T, ha, None)
    assert torch.equal(torch.cat([oa, ob]), o) and torch.equal(hb, hT)
    del oa, ob
    _, _, gra = _fwd_bwd(d, 0, split, d["h0"], grb["dh0"])
    for k in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(torch.cat([gra[k], grb[k]]), gr[k]), k
    assert torch.equal(gra["dh0"], gr["dh0"])
