"""The determinism gate: forward + backward repeated 100 times per shape row,
every repeat's outputs (o, hT, dq, dk, dv, dg, dbeta, dh0) bit-identical to the
first's, and the SHA-256 of the first and the last repeat equal.

The rows follow the shape table the cake_gdn page (miles PR #3597) runs its
gate on ("Validation of the round-13 kernels": fixed-length packs of 4, 8 and
16 x 4096 tokens, one 16384-token sequence, 32 x 512 and 128 x 128 short
sequences, a ragged pack, and the TP = 2 shard with 8 key / 16 value heads),
plus the pack of the fwd+bwd bench step (2 x 8192), the 12-sequence varlen pack
and one and two value heads per key head. Every output is compared on the
device after each repeat; nothing is copied to the host but the two hashed
repeats.
"""
import hashlib
import sys

import pytest
import torch

from chunked_gated_delta_04_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn

REPEATS = 100

ROWS = [
    # (name, lengths, H, HV)
    ("4x4096", [4096] * 4, 16, 32),
    ("8x4096", [4096] * 8, 16, 32),
    ("16x4096", [4096] * 16, 16, 32),
    ("1x16384", [16384], 16, 32),
    ("2x8192", [8192] * 2, 16, 32),
    ("32x512", [512] * 32, 16, 32),
    ("128x128", [128] * 128, 16, 32),
    ("varlen12_32768", synth.workload_lengths("fwd_varlen12_32768_h16_hv32"), 16, 32),
    ("ragged7", [4227, 4298, 4251, 4266, 4239, 4310, 4495], 16, 32),
    ("4x4096_h8_hv16", [4096] * 4, 8, 16),
    ("ragged_G1", [1, 63, 64, 65, 200, 130, 1000], 8, 8),
    ("ragged_G2", [1, 63, 64, 65, 200, 130, 1000], 4, 8),
]


def _hash(tensors):
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name,lens,H,HV", ROWS, ids=[r[0] for r in ROWS])
def test_forward_backward_repeat_bitwise(name, lens, H, HV):
    print(f"determinism {name}: {len(lens)} seqs, {sum(lens)} tokens, H={H} HV={HV}, "
          f"{REPEATS} repeats", file=sys.stderr, flush=True)
    inp = synth.chunk_inputs(lens, H, HV, seed=777 + len(lens), h0_std=0.1, with_do=True)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, N = sum(lens), len(lens)
    host = inp["cu_seqlens"]
    p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], host)
    dev = d["q"].device
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device=dev)
    hT = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev)
    saved = torch.empty(gdn.gdn_chunk_saved_size(p), dtype=torch.uint8, device=dev)
    wsf = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p), dtype=torch.uint8, device=dev)
    wsb = torch.empty(gdn.gdn_chunk_bwd_workspace_size(p), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    dg = torch.empty(T, HV, dtype=torch.float32, device=dev)
    dbeta = torch.empty_like(dg)
    dh0 = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev)
    outs = [o, hT, dq, dk, dv, dg, dbeta, dh0]

    def run():
        gdn.gdn_chunk_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o, hT, saved,
                          wsf, None)
        gdn.gdn_chunk_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], saved, d["do"], None,
                          dq, dk, dv, dg, dbeta, dh0, wsb, None)

    run()
    first = [t.clone() for t in outs]
    first_hash = _hash(first)
    for i in range(1, REPEATS):
        # scribble over the outputs so that a repeat that skipped a write would show
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        run()
        for j, (a, b) in enumerate(zip(first, outs)):
            assert torch.equal(a, b), (name, i, j)
    assert _hash(outs) == first_hash
