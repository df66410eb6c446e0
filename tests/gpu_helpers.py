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
