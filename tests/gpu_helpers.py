"""Shared helpers of the GPU tests: device transfer, oracle calls on sampled
heads, and the parity bar."""
import numpy as np
import torch

from oracle import recurrence as R

ATOL = 1e-2
RTOL = 1e-2


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def to_dev(d, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def within_bar(x, ref, atol=ATOL, rtol=RTOL):
    """|x - ref| <= atol + rtol |ref| elementwise. Returns (ok, max_abs_err, worst_ratio)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(x - ref)
    bound = atol + rtol * np.abs(ref)
    ratio = float((err / bound).max()) if err.size else 0.0
    return bool(np.all(err <= bound)), float(err.max()) if err.size else 0.0, ratio


def assert_bar(name, x, ref, atol=ATOL, rtol=RTOL):
    ok, mx, ratio = within_bar(x, ref, atol, rtol)
    assert ok, f"{name}: max|err| {mx:.3e}, worst err/bound {ratio:.3f}"
    return mx


def head_slice(inp, seq, hv, H, HV):
    """Oracle inputs for one sequence and the value heads of one key head."""
    cu = inp["cu_seqlens"].tolist()
    t0, t1 = cu[seq], cu[seq + 1]
    G = HV // H
    h = hv // G
    hvs = list(range(h * G, (h + 1) * G))
    out = dict(
        q=f64(inp["q"][t0:t1, h:h + 1]), k=f64(inp["k"][t0:t1, h:h + 1]),
        v=f64(inp["v"][t0:t1, hvs]), g=f64(inp["g"][t0:t1, hvs]),
        beta=f64(inp["beta"][t0:t1, hvs]), cu=[0, t1 - t0],
        h0=None if inp.get("h0") is None else f64(inp["h0"][seq:seq + 1, hvs]),
    )
    if "do" in inp:
        out["do"] = f64(inp["do"][t0:t1, hvs])
    return out, (t0, t1), h, hvs


def oracle_forward(inp):
    return R.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                     f64(inp["beta"]), inp["cu_seqlens"].tolist(),
                     None if inp.get("h0") is None else f64(inp["h0"]))


def oracle_backward(inp, dhT=None):
    return R.backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                      f64(inp["beta"]), inp["cu_seqlens"].tolist(), f64(inp["do"]),
                      None if inp.get("h0") is None else f64(inp["h0"]),
                      dhT=None if dhT is None else f64(dhT))


# ---------------------------------------------------------------- oracle over worker processes
# Full-size parity compares every (sequence, value head) with the oracle. The
# unchanged oracle runs on independent slices - one key head with its value
# heads, over the sequences asked for - in spawned worker processes (a fresh
# interpreter each: nothing GPU-related is inherited), then the pieces are put
# back in place. The pool size follows the host cores the process may use,
# capped at 16 (a GPU machine gives one GPU's share of its cores).
def oracle_workers():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _slice_forward(args):
    q, k, v, g, beta, cu, h0 = args
    return R.forward(q, k, v, g, beta, cu, h0)


def _slice_backward(args):
    q, k, v, g, beta, cu, do, h0, dhT = args
    return R.backward(q, k, v, g, beta, cu, do, h0, dhT=dhT)


def _pool():
    import concurrent.futures as cf
    import multiprocessing as mp
    return cf.ProcessPoolExecutor(max_workers=oracle_workers(), mp_context=mp.get_context("spawn"))


def oracle_forward_all_heads(inp):
    """Oracle o [T, HV, V] and hT [N, HV, V, K] of a whole pack, one task per key head."""
    T, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    G = HV // H
    N = inp["cu_seqlens"].numel() - 1
    cu = inp["cu_seqlens"].tolist()
    h0 = inp.get("h0")
    tasks = []
    for h in range(H):
        hvs = slice(h * G, (h + 1) * G)
        tasks.append((f64(inp["q"][:, h:h + 1]), f64(inp["k"][:, h:h + 1]), f64(inp["v"][:, hvs]),
                      f64(inp["g"][:, hvs]), f64(inp["beta"][:, hvs]), cu,
                      None if h0 is None else f64(h0[:, hvs])))
    o = np.zeros((T, HV, 128))
    hT = np.zeros((N, HV, 128, 128))
    with _pool() as ex:
        for h, (oh, hh) in enumerate(ex.map(_slice_forward, tasks)):
            o[:, h * G:(h + 1) * G] = oh
            hT[:, h * G:(h + 1) * G] = hh
    return o, hT


def oracle_backward_all_heads(inp, seq, dhT=None):
    """Oracle gradients of sequence `seq` of a pack over every head, one task per
    key head. Returns dq, dk [L, H, K], dv [L, HV, V], dg, dbeta [L, HV] (rows of
    the sequence) and dh0 [HV, V, K]."""
    T, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    G = HV // H
    cu = inp["cu_seqlens"].tolist()
    t0, t1 = cu[seq], cu[seq + 1]
    L = t1 - t0
    h0 = inp.get("h0")
    tasks = []
    for h in range(H):
        hvs = slice(h * G, (h + 1) * G)
        tasks.append((f64(inp["q"][t0:t1, h:h + 1]), f64(inp["k"][t0:t1, h:h + 1]),
                      f64(inp["v"][t0:t1, hvs]), f64(inp["g"][t0:t1, hvs]),
                      f64(inp["beta"][t0:t1, hvs]), [0, L], f64(inp["do"][t0:t1, hvs]),
                      None if h0 is None else f64(h0[seq:seq + 1, hvs]),
                      None if dhT is None else f64(dhT[seq:seq + 1, hvs])))
    out = dict(dq=np.zeros((L, H, 128)), dk=np.zeros((L, H, 128)), dv=np.zeros((L, HV, 128)),
               dg=np.zeros((L, HV)), dbeta=np.zeros((L, HV)), dh0=np.zeros((HV, 128, 128)))
    with _pool() as ex:
        for h, r in enumerate(ex.map(_slice_backward, tasks)):
            hvs = slice(h * G, (h + 1) * G)
            out["dq"][:, h] = r["dq"][:, 0]
            out["dk"][:, h] = r["dk"][:, 0]
            out["dv"][:, hvs] = r["dv"]
            out["dg"][:, hvs] = r["dg"]
            out["dbeta"][:, hvs] = r["dbeta"]
            out["dh0"][hvs] = r["dh0"][0]
    return out


def assert_dg_bar(name, x, ref):
    """The pages' bar for the decay gradient: atol scaled by the reference's
    largest magnitude, rtol 1e-2 (cake_gdn page, 'Tests'). The scaling loosens
    the bar for a gradient summed along the sequence; it never tightens it below
    the atol = 1e-2 that every other gradient gets (a reference that is ~0 -
    every decay underflowed - would otherwise ask for less than fp32 rounding)."""
    return assert_bar(name, x, ref, atol=ATOL * max(float(np.abs(ref).max()), 1.0))
