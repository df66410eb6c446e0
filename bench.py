#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule on one MI355X.

One step = one chunk forward (saving what the backward needs) plus one chunk
backward, over the 2 x 8192-token pack with 16 key / 32 value heads
(K = V = 128, chunk 64): every kernel of the chunk path, from the chunk table
to dq/dk/dv/dg/dbeta/dh0. Inputs are seeded synthetic tensors already resident
in HBM when timing starts. Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
                    [--no-secondary] [--fresh-processes 4] [--profile-step]

The headline is the mean of `steps` back-to-back steps between two events.
Beside it: the pages' operator protocol (each rep alone after a 512 MiB fill
that evicts the caches, median of the reps) in this process and in fresh
processes (median of their medians). Per-kernel durations come from HIP events
that the library records around each kernel it launches, on the stream it
launches on. Rooflines use the method's own bytes and flops (inputs, outputs
and the bf16 per-chunk states; no hand-off of this library), the roofline
object for the kernel with the largest average duration; the HBM bytes the
counters saw for it (committed profile summary) stand beside them. The CPU
baseline times the fp64 oracle on all host cores on a bounded sample of the
4 x 4096 and varlen forwards, the fwd+bwd step and the decode step.
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "fwdbwd_2x8192_h16_hv32"
METRIC = "GDN chunk fwd+bwd tokens/sec (H=16, HV=32, K=V=128); % bf16 MFMA peak"
PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12        # MI355X HBM3E, B/s

# Algorithmic work per chunk of 64 tokens and value head (K = V = 128). The
# masked triangles of the 64 x 64 products are not counted.
C, D = 64, 128
F_KKT = C * (C - 1) // 2 * 2 * D            # strictly lower K K^T
F_TSOLVE = C ** 3 // 3                      # (I + A)^-1
F_TRI = C * (C + 1) // 2 * 2 * D            # one lower-triangular 64x64 by 64x128 product
F_STATE = 2 * C * D * D                     # one 64x128 by 128x128 product
F_FWD = F_KKT + F_TSOLVE + 4 * F_TRI + 3 * F_STATE     # 9,024,853
F_FWDBWD = 3 * F_FWD
# per-kernel shares of the model (forward: WY pass vs scan; backward: its two kernels
# split the 2 * F_FWD gradient work as the gradient contractions are assigned to them)
KERNEL_FLOPS = {
    "chunk_prep": F_KKT + F_TSOLVE + 2 * F_TRI,                 # K K^T, T, W, Q K^T
    "fwd_scan": 2 * F_TRI + 3 * F_STATE,                        # U, attn D, W h, Q h, K^T D
    "bwd_dh_scan": F_TRI + 3 * F_STATE,                         # P^T dO, K dh, Q^T dO, W^T dD
    "bwd_chunk": 2 * F_FWD - (F_TRI + 3 * F_STATE),             # the remaining gradient work
}


def method_bytes(T, N, H, HV, n_chunks):
    """The method's own HBM bytes (nothing of this library's hand-offs): every
    input read once, every output written once, and the per-chunk states h_c
    (bf16) written by the forward and read by the backward. Per kernel, the part
    of those the kernel's job needs - what it could not avoid moving whatever
    the design: the WY pass reads q, k, g, beta; the forward scan reads v and
    h0 and writes o, hT, h_c; the dh scan reads q, k, g, beta and dO and writes
    dh0; the gradient pass reads q, k, v, g, beta, dO and h_c and writes dq, dk,
    dv, dg, dbeta. The step counts each tensor once per pass that must move it
    (the forward reads the inputs, the backward reads them again)."""
    qk = T * H * D * 2                   # q or k (or dq, dk), bf16
    vv = T * HV * D * 2                  # v, o, dO or dv, bf16
    gb = T * HV * 4                      # g, beta, dg or dbeta, fp32
    st = N * HV * D * D * 4              # h0, hT, dh0 (fp32 states)
    hc = n_chunks * HV * D * D * 2       # per-chunk start states, bf16
    per = {
        "chunk_prep": 2 * qk + 2 * gb,
        "fwd_scan": vv + st + vv + st + hc,
        "bwd_dh_scan": 2 * qk + 2 * gb + vv + st,
        "bwd_chunk": 2 * qk + vv + 2 * gb + vv + hc + 2 * qk + vv + 2 * gb,
    }
    fwd = 2 * qk + vv + 2 * gb + st + vv + st + hc
    bwd = 2 * qk + vv + 2 * gb + hc + vv + 2 * qk + vv + 2 * gb + st
    return per, {"fwd": fwd, "bwd": bwd, "step": fwd + bwd}


# stage name (gdn_stage_name) -> kernel symbol as the profiler names it
STAGE_KERNELS = {"chunk_table": "chunk_table_kernel", "chunk_prep": "chunk_prep_kernel<true>",
                 "fwd_scan": "fwd_scan_kernel<true, true, false>",
                 "bwd_dh_scan": "bwd_dh_scan_kernel", "bwd_chunk": "bwd_chunk_kernel<true>"}


def _code_tokens(text):
    """C/HIP source with comments removed and whitespace runs collapsed (string
    and character literals kept whole), so that editing a comment leaves the
    hash below unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the HIP sources' code (comments and layout ignored), to tie
    recorded counters to the code they measured."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "chunked_gated_delta_04_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8", errors="replace") as fh:
            h.update(_code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_counters():
    """Per-kernel counter figures of the committed summary of this workload (HBM
    bytes from FETCH_SIZE / WRITE_SIZE calibrated by a plain copy; MFMA busy
    fraction and bf16 MFMA work), or {} when that summary was taken on other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", WORKLOAD + ".md")
    try:
        text = open(path).read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return {}
    if blob.get("source") != kernel_source_hash():
        return {}
    return blob.get("kernels", {})


def hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def make_events(h, n):
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        ev = ctypes.c_void_p()
        if h.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        arr[i] = ev
    return arr


def sparse_events(h, n, idx):
    """A ctypes array of n event handles, created only at the indices in idx
    (the others NULL: the library records nothing there)."""
    arr = (ctypes.c_void_p * n)()
    for i in idx:
        ev = ctypes.c_void_p()
        if h.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        arr[i] = ev
    return arr


def elapsed_ms(h, a, b):
    ms = ctypes.c_float()
    if h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


# ---------------------------------------------------------------- CPU baseline
# The fp64 oracle as it stands, timed on the host cores: every (sequence, key
# head) slice of a workload is an independent task (its value heads read only
# that key head), run by a pool of spawned worker processes, one numpy thread
# each. The tasks are top-level functions so that the workers can import them.
def _oracle_fwd_task(a):
    from oracle import recurrence as R
    q, k, v, g, beta, cu, h0 = a
    R.forward(q, k, v, g, beta, cu, h0)
    return q.shape[0]


def _oracle_fwdbwd_task(a):
    from oracle import recurrence as R
    q, k, v, g, beta, cu, h0, do = a
    R.forward(q, k, v, g, beta, cu, h0)
    R.backward(q, k, v, g, beta, cu, do, h0)
    return q.shape[0]


def _oracle_decode_task(a):
    """One decode step over a group of rows; returns the seconds of the oracle
    call alone (the rows' pool blocks are large, and shipping them to the worker
    is not oracle work)."""
    from oracle import recurrence as R
    t = time.perf_counter()
    R.decode_step(*a)
    return time.perf_counter() - t


def _noop(_):
    return os.getpid()


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(target_s):
    """The oracle on the host's cores, on a bounded sample of each workload the
    pages' plan names: the forward of the 4 x 4096 pack and of the 12-sequence
    varlen pack, forward + backward of the 2 x 8192 pack (the headline's step)
    and one decode step of the 256-row batch. A sample is the first n tokens of
    every sequence over all heads; a 64-token probe of the same tasks sizes n
    to about `target_s` seconds. Returns the bench line's cpu_baseline object
    (value: the fwd+bwd tokens/s, the metric of the headline)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    from chunked_gated_delta_04_amd import synth

    os.environ.setdefault("OMP_NUM_THREADS", "1")
    workers = max(1, min(16, _host_cores()))

    def f64(t):
        return t.double().numpy()

    def slices(inp, n, with_do):
        H = inp["q"].shape[1]
        G = inp["v"].shape[1] // H
        cu = inp["cu_seqlens"].tolist()
        tasks, tokens = [], 0
        for s in range(len(cu) - 1):
            t0, t1 = cu[s], min(cu[s + 1], cu[s] + n)
            tokens += t1 - t0
            for h in range(H):
                hv = slice(h * G, (h + 1) * G)
                a = [f64(inp["q"][t0:t1, h:h + 1]), f64(inp["k"][t0:t1, h:h + 1]),
                     f64(inp["v"][t0:t1, hv]), f64(inp["g"][t0:t1, hv]),
                     f64(inp["beta"][t0:t1, hv]), [0, t1 - t0],
                     None if inp.get("h0") is None else f64(inp["h0"][s:s + 1, hv])]
                if with_do:
                    a.append(f64(inp["do"][t0:t1, hv]))
                tasks.append(tuple(a))
        return tasks, tokens

    def timed(ex, fn, tasks):
        t = time.perf_counter()
        list(ex.map(fn, tasks))
        return time.perf_counter() - t

    out = {}
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_noop, range(4 * workers)))           # workers up before any timing
        for name, fn, with_do in (("fwd_4x4096_h16_hv32", _oracle_fwd_task, False),
                                  ("fwd_varlen12_32768_h16_hv32", _oracle_fwd_task, False),
                                  (WORKLOAD, _oracle_fwdbwd_task, True)):
            inp = synth.workload_inputs(name)
            probe, ptok = slices(inp, 64, with_do)
            dt = timed(ex, fn, probe)
            longest = max(np.diff(inp["cu_seqlens"].numpy()))
            n = int(min(longest, max(64, 64 * target_s / max(dt, 1e-3))))
            tasks, tokens = slices(inp, n, with_do)
            dt = timed(ex, fn, tasks)
            out[name] = {"tokens_per_s": round(tokens / dt, 2), "tokens": tokens,
                         "first_tokens_per_sequence": n, "seconds": round(dt, 2),
                         "tasks": len(tasks), "what": "forward + backward" if with_do else "forward"}
            del inp, probe, tasks
        name = "decode_256_pool512_h16_hv32"
        inp = synth.workload_inputs(name)
        idx = inp["ssm_state_indices"].numpy()
        pool = inp["state_pool"]
        tasks = []
        for rows in np.array_split(np.arange(idx.size), workers):
            # the rows' own pool blocks, renumbered 1..n (0 stays the null block)
            act = [int(i) for i in idx[rows] if i > 0]
            sub = np.zeros((len(act) + 1,) + tuple(pool.shape[1:]))
            sub[1:] = f64(pool[act])
            ren = np.array([act.index(int(i)) + 1 if i > 0 else int(i) for i in idx[rows]],
                           dtype=np.int64)
            tasks.append((f64(inp["q"][rows]), f64(inp["k"][rows]), f64(inp["v"][rows]),
                          f64(inp["a"][rows]), f64(inp["b"][rows]), f64(inp["A_log"]),
                          f64(inp["dt_bias"]), sub, ren))
        # the groups run at once, one per worker: the step takes the slowest group's time
        dt = max(ex.map(_oracle_decode_task, tasks))
        out[name] = {"rows_per_s": round(idx.size / dt, 2), "rows": int(idx.size),
                     "seconds": round(dt, 3), "tasks": len(tasks),
                     "what": "one decode step (row groups in parallel, oracle time per group)"}
    head = out[WORKLOAD]
    return dict(
        value=head["tokens_per_s"], unit="tokens/s", cores=workers, kind="oracle",
        cpu_model=_cpu_model(), host_cores=_host_cores(),
        sample=(f"fp64 oracle forward + backward over the first "
                f"{head['first_tokens_per_sequence']} tokens of both sequences of {WORKLOAD} "
                f"(all 16 key / 32 value heads, {head['tasks']} (sequence, key head) tasks, "
                f"{head['seconds']} s) on {workers} worker processes of one thread each"),
        per_workload=out)


def copy_probe(mib):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiler run."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_dispatch": n * 4, "dispatches": 3}), flush=True)


def time_call(h, stream, fn, steps, warmup):
    """Average ms of fn() over `steps` calls, HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = make_events(h, 2)
    h.hipEventRecord(ev[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        fn()
    h.hipEventRecord(ev[1], ctypes.c_void_p(stream.cuda_stream))
    h.hipEventSynchronize(ev[1])
    return elapsed_ms(h, ev[0], ev[1]) / steps


def fwdbwd_step_ms(h, stream, name, steps, warmup):
    """Mean ms of a forward (saving for the backward) + backward step on a workload."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    inp = synth.workload_inputs(name)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    N = inp["cu_seqlens"].numel() - 1
    p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], inp["cu_seqlens"])
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device="cuda")
    hT = torch.empty(N, HV, 128, 128, dtype=torch.float32, device="cuda")
    saved = torch.empty(gdn.gdn_chunk_saved_size(p), dtype=torch.uint8, device="cuda")
    wsf = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(gdn.gdn_chunk_bwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    g_ = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
              dg=torch.empty_like(d["g"]), dbeta=torch.empty_like(d["beta"]),
              dh0=torch.empty(N, HV, 128, 128, dtype=torch.float32, device="cuda"))

    def step():
        gdn.gdn_chunk_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o, hT, saved,
                          wsf, stream)
        gdn.gdn_chunk_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], saved, d["do"], None,
                          g_["dq"], g_["dk"], g_["dv"], g_["dg"], g_["dbeta"], g_["dh0"], wsb,
                          stream)
    ms = time_call(h, stream, step, steps, warmup)
    return T, ms


def forward_packs(h, stream, names, steps, warmup):
    """Forward-only throughput (nothing saved for a backward) on varlen packs."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    out = {}
    for name in names:
        inp = synth.workload_inputs(name)
        d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        T, H, _ = inp["q"].shape
        HV = inp["v"].shape[1]
        N = inp["cu_seqlens"].numel() - 1
        p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], inp["cu_seqlens"])
        o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device="cuda")
        hT = torch.empty(N, HV, 128, 128, dtype=torch.float32, device="cuda")
        ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
        ms = time_call(h, stream, lambda: gdn.gdn_chunk_fwd(
            p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o, hT, None, ws, stream),
            steps, warmup)
        out[name] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1)}
        del d, o, hT, ws
    return out


def decode_step(h, stream, steps, warmup):
    """The decode step (256 rows, 16 of them on the null block, pool of 512
    states) against the HBM roofline."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    name = "decode_256_pool512_h16_hv32"
    inp = synth.workload_inputs(name)
    d = {k: v.cuda() for k, v in inp.items()}
    N, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    o = torch.empty(N, HV, 128, dtype=torch.bfloat16, device="cuda")
    slots = d["state_pool"].shape[0]
    ms = time_call(h, stream, lambda: gdn.gdn_recurrent_step(
        N, H, HV, 128, 128, 0.0, d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
        d["dt_bias"], d["state_pool"], slots, d["ssm_state_indices"], None, o, stream),
        steps, warmup)
    active = int((inp["ssm_state_indices"] > 0).sum())
    # algorithmic bytes: the active rows' fp32 state read and written once, their q, k, v,
    # a, b read once, every o row written, the index vector and the per-head A_log/dt_bias
    state = active * HV * 128 * 128 * 4 * 2
    io = active * (2 * H * 128 * 2 + HV * 128 * 2 + 2 * HV * 2) + N * HV * 128 * 2 + N * 4 + HV * 8
    bytes_ = state + io
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {name: {"ms": round(ms, 4), "rows_per_s": round(N / (ms * 1e-3), 1),
                   "algorithmic_bytes": bytes_, "achieved_GBps": round(gbs, 1),
                   "hbm_frac": round(gbs * 1e9 / PEAK_HBM, 4)}}


FWD_PACKS = ("fwd_4x4096_h16_hv32", "fwd_varlen12_32768_h16_hv32")
FWD_PACKS_TP2 = ("fwd_4x4096_h8_hv16", "fwd_varlen12_32768_h8_hv16")


def long_and_tp2_steps(h, stream, steps, warmup):
    """The fwd+bwd step at one GPU's share of a TP = 2 head split (8 key / 16
    value heads), on the same 16384 tokens as 32 x 512 and 128 x 128 short
    sequences, and on one long sequence of 65,536 and 131,072 tokens."""
    import torch
    out = {}
    for name, reps in (("fwdbwd_2x8192_h8_hv16", steps), ("fwdbwd_32x512_h16_hv32", steps),
                       ("fwdbwd_128x128_h16_hv32", steps), ("fwdbwd_1x65536_h16_hv32", steps),
                       ("fwdbwd_1x131072_h16_hv32", max(3, steps // 4))):
        T, ms = fwdbwd_step_ms(h, stream, name, reps, min(warmup, 2))
        out[name] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1)}
        torch.cuda.empty_cache()
    return out


def secondary(h, stream, steps, warmup):
    """Forward-only throughput on the 4 x 4096 and the 12-sequence varlen packs, the
    decode step against the HBM roofline, the paged prefill, the recomputing
    backward and the local transitions, the short convolution, the same packs
    at one GPU's share of a TP = 2 head split (8 key / 16 value heads), the
    fwd+bwd step on packs of short sequences (32 x 512, 128 x 128 tokens), and
    one long sequence of 65,536 and 131,072 tokens."""
    out = forward_packs(h, stream, FWD_PACKS + FWD_PACKS_TP2, steps, warmup)
    out.update(decode_step(h, stream, steps, warmup))
    out.update(paged_prefill(h, stream, steps, warmup))
    out.update(recompute_and_transition(h, stream, steps, warmup))
    out.update(short_conv(h, stream, steps, warmup))
    out.update(long_and_tp2_steps(h, stream, steps, warmup))
    return out


def short_conv(h, stream, steps, warmup):
    """The short convolution at the fwd+bwd pack's channels (2 x 8192 tokens,
    8192 channels, width 4, SiLU) against the HBM roofline, its decode update
    (256 rows, pool of 512) and its paged prefill (8 x 512 tokens, 4096
    channels, pool of 64)."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    name = "conv_2x8192_c8192_w4"
    inp = synth.workload_inputs(name)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, C = inp["x"].shape
    W = inp["weight"].shape[1]
    p = gdn.make_conv_problem(2, T, C, W, d["cu_seqlens"], inp["cu_seqlens"], "silu")
    y = torch.empty_like(d["x"])
    ms_f = time_call(h, stream, lambda: gdn.gdn_conv_fwd(p, d["x"], d["weight"], None, None, y,
                                                         None, stream), steps, warmup)
    dx = torch.empty_like(d["x"])
    dw = torch.empty(C, W, dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.gdn_conv_bwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    ms_b = time_call(h, stream, lambda: gdn.gdn_conv_bwd(
        p, d["x"], d["weight"], None, None, d["dy"], dx, dw, None, None, ws, stream),
        steps, warmup)
    row = T * C * 2
    bf, bb = 2 * row + C * W * 2, 3 * row + C * W * 2 + C * W * 4
    out = {name + "_fwd": {"ms": round(ms_f, 4), "algorithmic_bytes": bf,
                           "achieved_GBps": round(bf / (ms_f * 1e-3) / 1e9, 1),
                           "hbm_frac": round(bf / (ms_f * 1e-3) / PEAK_HBM, 4)},
           name + "_bwd": {"ms": round(ms_b, 4), "algorithmic_bytes": bb,
                           "achieved_GBps": round(bb / (ms_b * 1e-3) / 1e9, 1),
                           "hbm_frac": round(bb / (ms_b * 1e-3) / PEAK_HBM, 4)}}
    del d, y, dx, ws
    pool, idx = synth.conv_pool_inputs(256, 8192, 4, slots=512, n_null=16, seed=synth.BASE_SEED + 7)
    x1 = synth.conv_inputs([256], 8192, 4, seed=synth.BASE_SEED + 8)
    pd, idd = pool.cuda(), idx.cuda()
    xd, wd = x1["x"].cuda(), x1["weight"].cuda()
    yd = torch.empty_like(xd)
    ms_u = time_call(h, stream, lambda: gdn.gdn_conv_update(
        256, 8192, 4, "silu", xd, wd, None, pd, 512, idd, None, yd, stream), steps, warmup)
    out["conv_update_256_c8192_w4_pool512"] = {"ms": round(ms_u, 4)}
    lens = [512] * 8
    xp = synth.conv_inputs(lens, 4096, 4, seed=synth.BASE_SEED + 9)
    pool, idx = synth.conv_pool_inputs(8, 4096, 4, slots=64, n_null=0, seed=synth.BASE_SEED + 10)
    init = torch.tensor([1, 0] * 4, dtype=torch.int32, device="cuda")
    cu = xp["cu_seqlens"]
    pp = gdn.make_conv_problem(8, 4096, 4096, 4, cu.cuda(), cu, "silu")
    xpd, wpd, ppd, ipd = xp["x"].cuda(), xp["weight"].cuda(), pool.cuda(), idx.cuda()
    ypd = torch.empty_like(xpd)
    ms_p = time_call(h, stream, lambda: gdn.gdn_conv_fwd_paged(
        pp, xpd, wpd, None, ppd, 64, ipd, init, None, ypd, stream), steps, warmup)
    out["conv_paged_8x512_c4096_w4_pool64"] = {"ms": round(ms_p, 4)}
    return out


def recompute_and_transition(h, stream, steps, warmup):
    """On the fwd+bwd pack (2 x 8192 tokens, 16 / 32 heads): the step with the
    recomputing backward (a forward that saves nothing, then
    gdn_chunk_bwd_recompute), and the local transitions of the pack cut into 8
    shards of 2048 tokens (one context-parallel rank's work per shard)."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    inp = synth.workload_inputs("fwdbwd_2x8192_h16_hv32")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    N = inp["cu_seqlens"].numel() - 1
    p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], inp["cu_seqlens"])
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device="cuda")
    hT = torch.empty(N, HV, 128, 128, dtype=torch.float32, device="cuda")
    fws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    bws = torch.empty(gdn.gdn_chunk_bwd_recompute_workspace_size(p), dtype=torch.uint8,
                      device="cuda")
    g_ = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
              dg=torch.empty_like(d["g"]), dbeta=torch.empty_like(d["beta"]),
              dh0=torch.empty_like(d["h0"]))

    def step():
        gdn.gdn_chunk_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o, hT, None,
                          fws, stream)
        gdn.gdn_chunk_bwd_recompute(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                    d["do"], None, g_["dq"], g_["dk"], g_["dv"], g_["dg"],
                                    g_["dbeta"], g_["dh0"], bws, stream)
    ms = time_call(h, stream, step, steps, warmup)
    out = {"fwdbwd_2x8192_h16_hv32_recompute": {
        "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
        "workspace_bytes": bws.numel(), "saved_bytes_avoided": gdn.gdn_chunk_saved_size(p)}}
    del bws, g_
    cu8 = torch.arange(0, T + 1, 2048, dtype=torch.int32)
    p8 = gdn.make_problem(8, T, H, HV, cu8.cuda(), cu8)
    M = torch.empty(8, HV, 128, 128, dtype=torch.float32, device="cuda")
    sT = torch.empty_like(M)
    tws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p8), dtype=torch.uint8, device="cuda")
    ms = time_call(h, stream, lambda: gdn.gdn_chunk_transition(
        p8, d["q"], d["k"], d["v"], d["g"], d["beta"], M, sT, tws, stream), steps, warmup)
    out["transition_8x2048_h16_hv32"] = {"ms": round(ms, 4),
                                         "tokens_per_s": round(T / (ms * 1e-3), 1)}
    return out


def paged_prefill(h, stream, steps, warmup):
    """The paged prefill (8 x 512 tokens, 8 key / 16 value heads, 64-slot pool,
    half the sequences fresh) in place on the pool, next to the same forward
    with the start states gathered from the pool and the end states scattered
    back by torch index copies."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    name = "paged_8x512_h8_hv16_pool64"
    inp = synth.workload_inputs(name)
    d = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    T, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    N = inp["cu_seqlens"].numel() - 1
    p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], inp["cu_seqlens"])
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    pool = d["state_pool"]
    slots = pool.shape[0]
    idx_l = d["ssm_state_indices"].long()
    keep = d["has_initial_state"].float()[:, None, None, None]
    h0 = torch.empty(N, HV, 128, 128, dtype=torch.float32, device="cuda")
    hT = torch.empty_like(h0)
    ms_paged = time_call(h, stream, lambda: gdn.gdn_chunk_fwd_paged(
        p, d["q"], d["k"], d["v"], d["g"], d["beta"], pool, slots, d["ssm_state_indices"],
        d["has_initial_state"], None, o, None, ws, stream), steps, warmup)

    def copies():
        torch.index_select(pool, 0, idx_l, out=h0)
        h0.mul_(keep)
        gdn.gdn_chunk_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], h0, o, hT, None, ws,
                          stream)
        pool.index_copy_(0, idx_l, hT)
    with torch.cuda.stream(stream):
        ms_copies = time_call(h, stream, copies, steps, warmup)
    return {name: {"ms": round(ms_paged, 4), "tokens_per_s": round(T / (ms_paged * 1e-3), 1),
                   "gather_scatter_ms": round(ms_copies, 4)}}


def setup_step(dev):
    """Inputs, outputs and workspaces of the fwd+bwd step, resident on `dev`;
    returns (meta, step) where step(ev_f, ev_b) runs one forward (saving for the
    backward) and one backward, recording per-kernel events when given, and
    returns the numbers of stages the timed calls launched."""
    import torch
    from chunked_gated_delta_04_amd import gdn, synth
    inp = synth.workload_inputs(WORKLOAD)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, H, _ = inp["q"].shape
    HV = inp["v"].shape[1]
    N = inp["cu_seqlens"].numel() - 1
    host = inp["cu_seqlens"].to(torch.int32)
    p = gdn.make_problem(N, T, H, HV, d["cu_seqlens"], host)
    lens = (host[1:] - host[:-1]).tolist()
    n_chunks = sum((L + 63) // 64 for L in lens)
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device=dev)
    hT = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev)
    saved = torch.empty(gdn.gdn_chunk_saved_size(p), dtype=torch.uint8, device=dev)
    wsf = torch.empty(gdn.gdn_chunk_fwd_workspace_size(p), dtype=torch.uint8, device=dev)
    wsb = torch.empty(gdn.gdn_chunk_bwd_workspace_size(p), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    dg = torch.empty(T, HV, dtype=torch.float32, device=dev)
    dbeta = torch.empty_like(dg)
    dh0 = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev_f=None, ev_b=None):
        nf = nb = 0
        if ev_f is None:
            gdn.gdn_chunk_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o, hT, saved,
                              wsf, stream)
        else:
            nf = gdn.gdn_chunk_fwd_timed(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], o,
                                         hT, saved, wsf, ev_f, stream)
        if ev_b is None:
            gdn.gdn_chunk_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], saved, d["do"], None,
                              dq, dk, dv, dg, dbeta, dh0, wsb, stream)
        else:
            nb = gdn.gdn_chunk_bwd_timed(p, d["q"], d["k"], d["v"], d["g"], d["beta"], saved,
                                         d["do"], None, dq, dk, dv, dg, dbeta, dh0, wsb, ev_b,
                                         stream)
        return nf, nb

    # `host` must outlive the problem descriptor, which points at it
    meta = dict(T=T, H=H, HV=HV, N=N, n_chunks=n_chunks, stream=stream, host=host,
                saved_bytes=saved.numel(), workspace_bytes=wsf.numel() + wsb.numel())
    step.keep = (host, p)
    return meta, step


FLUSH_BYTES = 512 * 2 ** 20


def cold_protocol(h, stream, step, reps, warmup, dev):
    """The pages' operator timing (cake_gdn page, 'Performance', operator level):
    `warmup` untimed steps, then `reps` steps timed one by one with events, each
    after a 512 MiB device fill (outside the events) that evicts L2 and the
    Infinity Cache. Returns the sorted per-rep ms."""
    import torch
    for _ in range(warmup):
        step()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    ev = make_events(h, 2 * reps)
    for i in range(reps):
        flush.fill_(float(i))
        h.hipEventRecord(ev[2 * i], ctypes.c_void_p(stream.cuda_stream))
        step()
        h.hipEventRecord(ev[2 * i + 1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    del flush
    return sorted(elapsed_ms(h, ev[2 * i], ev[2 * i + 1]) for i in range(reps))


def child_protocol(reps, warmup):
    """One fresh process's run of the cold protocol; prints its median."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    meta, step = setup_step(dev)
    ms = cold_protocol(hip(), meta["stream"], step, reps, warmup, dev)
    print(json.dumps({"median_ms": ms[len(ms) // 2], "min_ms": ms[0], "max_ms": ms[-1]}),
          flush=True)


def fresh_processes(n, reps, warmup):
    """The cold protocol in `n` fresh processes, one after another (the Cake page's
    protocol: fresh processes, the median of their medians)."""
    import subprocess
    meds = []
    for _ in range(n):
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--child-protocol",
                            "--steps", str(reps), "--warmup", str(warmup)],
                           capture_output=True, text=True, timeout=300)
        if r.returncode != 0:
            raise RuntimeError(f"fresh-process timing failed:\n{r.stderr[-2000:]}")
        meds.append(json.loads(r.stdout.strip().splitlines()[-1])["median_ms"])
    s = sorted(meds)
    return {"processes": n, "reps_per_process": reps, "medians_ms": [round(x, 4) for x in meds],
            "median_of_medians_ms": round(s[len(s) // 2] if n % 2 else
                                          0.5 * (s[n // 2 - 1] + s[n // 2]), 4)}


# --profile SECTION: run one section alone (warmup + steps calls of each of its
# operations), so that every dispatch a profiler records belongs to it
PROFILE_SECTIONS = {
    "fwd": lambda h, s, n, w: forward_packs(h, s, FWD_PACKS, n, w),
    "decode": decode_step,
    "paged": lambda h, s, n, w: paged_prefill(h, s, n, w),
    "recompute": lambda h, s, n, w: recompute_and_transition(h, s, n, w),
    "conv": lambda h, s, n, w: short_conv(h, s, n, w),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the timings of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="target oracle seconds per CPU-baseline workload")
    ap.add_argument("--fresh-processes", type=int, default=4,
                    help="fresh processes for the median-of-medians timing (0: skip)")
    ap.add_argument("--profile-step", action="store_true",
                    help="only run warmup + steps of the fwd+bwd step (for rocprofv3)")
    ap.add_argument("--profile", default=None, choices=["step"] + sorted(PROFILE_SECTIONS),
                    help="only run warmup + steps calls of one section (step: the fwd+bwd "
                         "step, as --profile-step), for rocprofv3")
    ap.add_argument("--child-protocol", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.child_protocol:
        child_protocol(args.steps, args.warmup)
        return

    import torch

    from chunked_gated_delta_04_amd import gdn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile in PROFILE_SECTIONS:
        res = PROFILE_SECTIONS[args.profile](hip(), torch.cuda.current_stream(), args.steps,
                                             args.warmup)
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "result": res}), flush=True)
        return
    meta, step = setup_step(dev)
    T, H, HV, N, stream = meta["T"], meta["H"], meta["HV"], meta["N"], meta["stream"]
    h = hip()
    if args.profile_step or args.profile == "step":
        for _ in range(args.warmup + args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_step": WORKLOAD, "steps": args.warmup + args.steps}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-kernel times: K steps with events around every kernel. The markers
    # between kernels lengthen the step (about 4 us each), so these steps are
    # not the timed ones.
    S = gdn.GDN_MAX_STAGES
    evf = [make_events(h, 2 * S) for _ in range(args.steps)]
    evb = [make_events(h, 2 * S) for _ in range(args.steps)]
    counts = None
    for i in range(args.steps):
        counts = step(evf[i], evb[i])
    torch.cuda.synchronize()
    stages = {}
    where = {}  # stage name -> (0 forward / 1 backward, stage index)
    nf, nb = counts
    for i in range(args.steps):
        for j in range(nf):
            name = gdn.gdn_stage_name(0, j)
            where[name] = (0, j)
            stages.setdefault(name, []).append(elapsed_ms(h, evf[i][2 * j], evf[i][2 * j + 1]))
        for j in range(nb):
            name = gdn.gdn_stage_name(1, j)
            if name == "chunk_table":
                name = "chunk_table_bwd"
            where[name] = (1, j)
            stages.setdefault(name, []).append(elapsed_ms(h, evb[i][2 * j], evb[i][2 * j + 1]))
    stage_ms = {k: sum(v) / len(v) for k, v in stages.items()}
    per_bytes, totals = method_bytes(T, N, H, HV, meta["n_chunks"])
    dom = max((k for k in stage_ms if k in per_bytes), key=stage_ms.get)

    # The timed steps: events only around the dominant kernel (its time for the
    # roofline, measured on the launch stream inside the timed region) and
    # around the whole region.
    op, j = where[dom]
    evd = [sparse_events(h, 2 * S, (2 * j, 2 * j + 1)) for _ in range(args.steps)]
    outer = make_events(h, 2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    h.hipEventRecord(outer[0], ctypes.c_void_p(stream.cuda_stream))
    for i in range(args.steps):
        if op == 0:
            step(evd[i], None)
        else:
            step(None, evd[i])
    h.hipEventRecord(outer[1], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    h.hipEventSynchronize(outer[1])
    total_ms = elapsed_ms(h, outer[0], outer[1])
    ms_per_step = total_ms / args.steps
    dom_ms = sum(elapsed_ms(h, e[2 * j], e[2 * j + 1]) for e in evd) / args.steps

    # Rooflines on the method's own bytes and flops (no hand-offs of this library).
    n_chunks = meta["n_chunks"]
    units = n_chunks * HV                            # (chunk, value head) pairs
    counters = recorded_counters()
    kernels = {}
    for stage, ms in stage_ms.items():
        b = per_bytes.get(stage)
        f = KERNEL_FLOPS.get(stage, 0) * units
        row = {"ms": round(ms, 4)}
        if b:
            row.update(algorithmic_bytes=b, GBps=round(b / (ms * 1e-3) / 1e9, 1),
                       hbm_frac=round(b / (ms * 1e-3) / PEAK_HBM, 4),
                       flops=f, mfma_frac=round(f / (ms * 1e-3) / PEAK_BF16, 4))
            c = counters.get(STAGE_KERNELS.get(stage, stage))
            if c:
                tb = c.get("fetch_bytes", 0) + c.get("write_bytes", 0)
                row.update(traffic_bytes=tb, traffic_over_algorithmic=round(tb / b, 3))
                for key in ("mfma_busy_frac", "mfma_bf16_flops_counted"):
                    if key in c:
                        row[key] = c[key]
        kernels[stage] = row
    dk_ = kernels[dom]
    db_, df_ = dk_["algorithmic_bytes"], dk_["flops"]
    # every kernel of the step is below the chip's balance point (2.5e15 / 8e12 =
    # 312 flop per byte) on these bytes, so HBM bandwidth is the roof
    roofline = {"bound": "hbm", "achieved": round(db_ / (dom_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(db_ / (dom_ms * 1e-3) / PEAK_HBM, 4),
                "traffic": dk_.get("traffic_bytes"),
                "kernel": dom, "kernel_ms": round(dom_ms, 4), "algorithmic_bytes": db_,
                "traffic_over_algorithmic": dk_.get("traffic_over_algorithmic"),
                "mfma_frac": round(df_ / (dom_ms * 1e-3) / PEAK_BF16, 4),
                "mfma_busy_frac": dk_.get("mfma_busy_frac"),
                "kernel_ms_timed_steps": "events around this kernel only, in the timed steps; "
                                         "the per-kernel table comes from K separate steps with "
                                         "events around every kernel"}
    step_flops = F_FWDBWD * units
    t_attain = max(step_flops / PEAK_BF16, totals["step"] / PEAK_HBM)
    step_roof = {"algorithmic_bytes": totals["step"], "fwd_bytes": totals["fwd"],
                 "bwd_bytes": totals["bwd"],
                 "achieved_GBps": round(totals["step"] / (ms_per_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(totals["step"] / (ms_per_step * 1e-3) / PEAK_HBM, 4),
                 "flops": step_flops,
                 "mfma_frac": round(step_flops / (ms_per_step * 1e-3) / PEAK_BF16, 4),
                 "attainable_ms": round(t_attain * 1e3, 4),
                 "frac_of_attainable": round(t_attain / (ms_per_step * 1e-3), 4)}
    tokens_per_s = T / (ms_per_step * 1e-3)

    cold = cold_protocol(h, stream, step, args.steps, args.warmup, dev)
    cold_ms = cold[len(cold) // 2]
    protocol = {"cold_cache": {"ms_median": round(cold_ms, 4), "ms_min": round(cold[0], 4),
                               "ms_max": round(cold[-1], 4),
                               "tokens_per_s": round(T / (cold_ms * 1e-3), 1),
                               "reps": args.steps, "warmup": args.warmup,
                               "flush_bytes": FLUSH_BYTES}}
    if args.fresh_processes > 0:
        fp = fresh_processes(args.fresh_processes, args.steps, args.warmup)
        fp["tokens_per_s"] = round(T / (fp["median_of_medians_ms"] * 1e-3), 1)
        protocol["fresh_processes"] = fp

    extra = None
    if not args.no_secondary:
        del step
        torch.cuda.empty_cache()
        extra = secondary(h, stream, args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "global_batch": N, "seq_len": T // N,
                   "tokens_per_step": T, "H": H, "HV": HV, "K": 128, "V": 128, "chunk": 64,
                   "parallelism": "single-gpu"},
        "mfma_frac_of_bf16_peak": step_roof["mfma_frac"],
        "algorithmic_tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "roofline": roofline,
        "step_roofline": step_roof,
        "kernels": kernels,
        "timing_protocol": protocol,
        "memory": {"saved_bytes": meta["saved_bytes"], "workspace_bytes": meta["workspace_bytes"]},
        "cpu_baseline": cpu,
        "secondary": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
