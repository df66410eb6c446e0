"""The per-stage timing entry points: the same bits as the untimed calls, with
events around every stage, around one stage only (the other handles NULL) or
none, and the recorded stages measure a positive time."""
import ctypes
import sys

import pytest
import torch

from chunked_gated_delta_04_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from chunked_gated_delta_04_amd import gdn


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _events(lib, idx):
    arr = (ctypes.c_void_p * (2 * gdn.GDN_MAX_STAGES))()
    for i in idx:
        ev = ctypes.c_void_p()
        assert lib.hipEventCreate(ctypes.byref(ev)) == 0
        arr[i] = ev
    return arr


def test_timed_calls_match_untimed():
    lens, H, HV = [200, 64, 1, 130], 2, 4
    print(f"timed calls: lens {lens}, H={H} HV={HV}", file=sys.stderr, flush=True)
    inp = synth.chunk_inputs(lens, H, HV, seed=41, h0_std=0.1, with_do=True)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, N = sum(lens), len(lens)
    p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], inp["cu_seqlens"])
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
    args_f = (p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o, hT, saved, wsf)
    args_b = (p, d["q"], d["k"], d["v"], d["g"], d["beta"], saved, d["do"], None,
              dq, dk, dv, dg, dbeta, dh0, wsb)

    gdn.gdn_chunk_fwd(*args_f, None)
    gdn.gdn_chunk_bwd(*args_b, None)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    lib = _hip()
    every = range(2 * gdn.GDN_MAX_STAGES)
    for name, idx_f, idx_b in (("every stage", every, every),
                               ("the last backward stage only", (), (4, 5)),
                               ("no stage", (), ())):
        ev_f, ev_b = _events(lib, idx_f), _events(lib, idx_b)
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        nf = gdn.gdn_chunk_fwd_timed(*args_f, ev_f, None)
        nb = gdn.gdn_chunk_bwd_timed(*args_b, ev_b, None)
        torch.cuda.synchronize()
        assert (nf, nb) == (3, 3), name
        assert [gdn.gdn_stage_name(1, j) for j in range(nb)][-1] == "bwd_chunk"
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), name
        for ev, idx, n in ((ev_f, idx_f, nf), (ev_b, idx_b, nb)):
            for j in range(n):
                if 2 * j in idx:
                    ms = ctypes.c_float()
                    assert lib.hipEventElapsedTime(ctypes.byref(ms), ev[2 * j], ev[2 * j + 1]) == 0
                    assert ms.value > 0, (name, j)
        for ev in (ev_f, ev_b):
            for h in ev:
                if h:
                    lib.hipEventDestroy(h)
