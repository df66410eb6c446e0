"""The C ABI on the CPU: the library loads, exports what include/gdn.h declares,
and rejects every bad argument before anything is enqueued.

No test here reaches a kernel launch: each call fails validation first, so the
fake device addresses below are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "chunked_gated_delta_04_amd", "libgdn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libgdn.so not built")

FAKE = 0x10000          # 16-byte aligned, never dereferenced
FAKE_MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def G():
    from chunked_gated_delta_04_amd import gdn
    return gdn


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", src)))


def test_every_declared_function_is_exported(G):
    names = declared_functions()
    assert set(names) == set(G.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    assert set(names) <= exported
    # nothing but the declared API is exported under the gdn_ prefix
    assert exported == set(names)


def test_status_strings(G):
    for s in range(9):
        assert G.gdn_status_string(s) and G.gdn_status_string(s) != "unknown status"
    assert G.gdn_status_string(99) == "unknown status"


def problem(G, N=2, T=130, H=2, HV=4, K=128, V=128, chunk=64, cu_host=(0, 70, 130), dev=FAKE):
    p = G.GdnProblem()
    p.N, p.T, p.H, p.HV, p.K, p.V, p.chunk = N, T, H, HV, K, V, chunk
    p.scale = 0.0
    p.cu_seqlens = dev
    keep = None
    if cu_host is not None:
        keep = (ctypes.c_int32 * len(cu_host))(*cu_host)
        p.cu_seqlens_host = ctypes.cast(keep, ctypes.c_void_p)
    p._keep = keep
    return p


def fwd(G, p, ws_bytes=1 << 40, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, o=FAKE, hT=None,
                saved=None, ws=FAKE)
    args.update(over)
    return G._lib.gdn_chunk_fwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["g"],
                                args["beta"], args["h0"], args["o"], args["hT"], args["saved"],
                                args["ws"], ws_bytes, None)


def bwd(G, p, ws_bytes=1 << 40, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, saved=FAKE, dO=FAKE, dhT=None,
                dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dh0=None, ws=FAKE)
    args.update(over)
    return G._lib.gdn_chunk_bwd(ctypes.byref(p), *[args[n] for n in (
        "q", "k", "v", "g", "beta", "saved", "dO", "dhT", "dq", "dk", "dv", "dg", "dbeta",
        "dh0", "ws")], ws_bytes, None)


def test_chunk_counts_and_sizes(G):
    p = problem(G)
    # the slot count is the bound T/64 + N (>= ceil(70/64) + ceil(60/64) = 3 chunks),
    # with or without the host copy of the boundaries
    assert G.gdn_num_chunks(p) == 130 // 64 + 2
    p2 = problem(G, cu_host=None)
    assert G.gdn_num_chunks(p2) == 130 // 64 + 2
    s = G.gdn_chunk_saved_size(p)
    blocks = 4 * 4  # value heads x chunk slots
    kblocks = 2 * 4  # key heads x chunk slots
    # per value-head block: the bf16 start state and D, W, P, T, T^T in bf16,
    # e^gamma_L, 192 per-token gate factors (e^gamma, e^(gamma_L - gamma), beta)
    # and 128 per-token gamma, beta in fp32 (the factors start 16-byte aligned);
    # per key-head block: Q~ and K^T in bf16
    assert s == (blocks * ((128 * 128 + 64 * 128) + 64 * 128 + 3 * 64 * 64)
                 + kblocks * 2 * 64 * 128) * 2 + ((blocks + 3) // 4 * 4 + blocks * (192 + 128)) * 4
    assert G.gdn_chunk_fwd_workspace_size(p) > 0
    assert G.gdn_chunk_bwd_workspace_size(p) > G.gdn_chunk_fwd_workspace_size(p) // 2
    assert G.gdn_chunk_fwd_workspace_size(p) == G.gdn_chunk_fwd_workspace_size(p)
    bad = problem(G, K=64)
    assert G.gdn_num_chunks(bad) == 0 and G.gdn_chunk_fwd_workspace_size(bad) == 0


@pytest.mark.parametrize("cu", [(0, 70, 130), (0, 64, 130), (0, 0, 130), (0, 130, 130)])
def test_saved_layout_does_not_depend_on_the_host_copy(G, cu):
    """A forward given the host copy of the boundaries and a backward given only
    the device copy (or the reverse) must agree on the saved buffer's layout:
    every size query depends on (N, T, H, HV) alone."""
    a, b = problem(G, cu_host=cu), problem(G, cu_host=None)
    for q in ("gdn_num_chunks", "gdn_chunk_saved_size", "gdn_chunk_fwd_workspace_size",
              "gdn_chunk_bwd_workspace_size", "gdn_chunk_bwd_recompute_workspace_size"):
        assert getattr(G, q)(a) == getattr(G, q)(b), q


def test_binding_refuses_a_short_saved_buffer(G):
    import torch
    p = problem(G)
    short = torch.empty(G.gdn_chunk_saved_size(p) - 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="saved"):
        G.gdn_chunk_bwd(p, None, None, None, None, None, short, None, None, None, None, None,
                        None, None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=64), 3), (dict(V=256), 3), (dict(chunk=32), 3), (dict(H=3, HV=4), 3),
    (dict(N=-1), 2), (dict(T=-5), 2), (dict(H=0), 2),
    (dict(cu_host=(0, 70, 131)), 4), (dict(cu_host=(1, 70, 130)), 4),
    (dict(cu_host=(0, 80, 70, 130)[:3]), 4),
])
def test_forward_rejects_bad_problems(G, kw, status):
    p = problem(G, **kw)
    assert fwd(G, p) == status
    assert bwd(G, p) == status


def test_non_monotone_host_boundaries(G):
    p = problem(G, N=3, T=130, cu_host=(0, 90, 60, 130))
    assert fwd(G, p) == 4


def test_null_pointers(G):
    p = problem(G)
    assert G._lib.gdn_chunk_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE,
                                1 << 40, None) == 1
    for name in ("q", "k", "v", "g", "beta", "o"):
        assert fwd(G, p, **{name: None}) == 1, name
    for name in ("q", "k", "v", "g", "beta", "saved", "dO", "dq", "dk", "dv", "dg", "dbeta"):
        assert bwd(G, p, **{name: None}) == 1, name
    p.cu_seqlens = None
    assert fwd(G, p) == 1


def test_workspace_checks(G):
    p = problem(G)
    need = G.gdn_chunk_fwd_workspace_size(p)
    assert fwd(G, p, ws_bytes=need - 1) == 6
    assert fwd(G, p, ws=None) == 6
    needb = G.gdn_chunk_bwd_workspace_size(p)
    assert bwd(G, p, ws_bytes=needb - 1) == 6


def test_alignment_checks(G):
    p = problem(G)
    assert fwd(G, p, q=FAKE_MISALIGNED) == 8
    assert fwd(G, p, hT=FAKE_MISALIGNED) == 8
    assert bwd(G, p, dv=FAKE_MISALIGNED) == 8


def decode(G, N=4, H=2, HV=4, K=128, V=128, slots=8, host=None, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, A_log=FAKE, dt_bias=None, pool=FAKE,
                idx=FAKE, o=FAKE)
    args.update(over)
    keep = None
    hp = None
    if host is not None:
        keep = (ctypes.c_int32 * len(host))(*host)
        hp = ctypes.cast(keep, ctypes.c_void_p)
    return G._lib.gdn_recurrent_step(N, H, HV, K, V, 0.0, args["q"], args["k"], args["v"],
                                     args["a"], args["b"], args["A_log"], args["dt_bias"],
                                     args["pool"], slots, args["idx"], hp, args["o"], None)


def test_decode_rejects_bad_arguments(G):
    assert decode(G, K=64) == 3
    assert decode(G, H=3, HV=4) == 3
    assert decode(G, N=-1) == 2
    assert decode(G, slots=-1) == 2
    assert decode(G, N=0) == 0          # nothing to do, nothing enqueued
    for name in ("q", "k", "v", "a", "b", "A_log", "pool", "idx", "o"):
        assert decode(G, **{name: None}) == 1, name
    assert decode(G, pool=FAKE_MISALIGNED) == 8


def test_decode_index_rules_on_the_host_copy(G):
    # out of range, repeated: errors before any launch
    assert decode(G, host=[1, 8, 2, 3]) == 5
    assert decode(G, host=[1, 2, 2, 3]) == 5
    assert decode(G, host=[1, 2, 7, 7]) == 5


def paged(G, p, slots=8, host=None, ws_bytes=1 << 40, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, idx=FAKE, init=None,
                o=FAKE, saved=None, ws=FAKE)
    args.update(over)
    keep = None
    hp = None
    if host is not None:
        keep = (ctypes.c_int32 * len(host))(*host)
        hp = ctypes.cast(keep, ctypes.c_void_p)
    return G._lib.gdn_chunk_fwd_paged(ctypes.byref(p), args["q"], args["k"], args["v"],
                                      args["g"], args["beta"], args["pool"], slots, args["idx"],
                                      args["init"], hp, args["o"], args["saved"], args["ws"],
                                      ws_bytes, None)


def test_paged_forward_rejects_bad_arguments(G):
    p = problem(G)
    assert paged(G, problem(G, K=64)) == 3
    assert paged(G, problem(G, cu_host=(0, 70, 131))) == 4
    assert paged(G, p, slots=-1) == 2
    for name in ("pool", "idx", "q", "o"):
        assert paged(G, p, **{name: None}) == 1, name
    assert paged(G, p, pool=FAKE_MISALIGNED) == 8
    assert paged(G, p, ws=None) == 6
    assert paged(G, p, ws_bytes=G.gdn_chunk_fwd_workspace_size(p) - 1) == 6


def test_paged_forward_with_no_sequences_is_a_no_op(G):
    """N = 0, T = 0: nothing to read or write, OK before any launch (as for
    gdn_chunk_fwd, the transition and the decode step)."""
    p = problem(G, N=0, T=0, cu_host=(0,))
    assert paged(G, p, q=None, k=None, v=None, g=None, beta=None, o=None, pool=None,
                 idx=None) == 0
    assert fwd(G, p, q=None, k=None, v=None, g=None, beta=None, o=None) == 0


def test_paged_forward_index_rules_on_the_host_copy(G):
    p = problem(G)
    assert paged(G, p, host=[1, 8]) == 5      # past the pool
    assert paged(G, p, host=[3, 3]) == 5      # one block for two sequences
    assert paged(G, p, host=[-2, 9], idx=FAKE, pool=None) == 1   # null checks come first


def transition(G, p, ws_bytes=1 << 40, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, M=FAKE, s=FAKE, ws=FAKE)
    args.update(over)
    return G._lib.gdn_chunk_transition(ctypes.byref(p), *[args[n] for n in (
        "q", "k", "v", "g", "beta", "M", "s", "ws")], ws_bytes, None)


def bwd_recompute(G, p, ws_bytes=1 << 40, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, dO=FAKE, dhT=None,
                dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dh0=None, ws=FAKE)
    args.update(over)
    return G._lib.gdn_chunk_bwd_recompute(ctypes.byref(p), *[args[n] for n in (
        "q", "k", "v", "g", "beta", "h0", "dO", "dhT", "dq", "dk", "dv", "dg", "dbeta",
        "dh0", "ws")], ws_bytes, None)


def test_transition_rejects_bad_arguments(G):
    p = problem(G)
    assert transition(G, problem(G, K=64)) == 3
    assert transition(G, problem(G, cu_host=(0, 70, 131))) == 4
    for name in ("q", "k", "v", "g", "beta", "M", "s"):
        assert transition(G, p, **{name: None}) == 1, name
    assert transition(G, p, M=FAKE_MISALIGNED) == 8
    assert transition(G, p, ws=None) == 6
    assert transition(G, p, ws_bytes=G.gdn_chunk_fwd_workspace_size(p) - 1) == 6


def test_recomputing_backward_rejects_bad_arguments(G):
    p = problem(G)
    need = G.gdn_chunk_bwd_recompute_workspace_size(p)
    # the rebuilt saved buffer sits after the larger of the two workspace layouts
    assert need == max(G.gdn_chunk_bwd_workspace_size(p), G.gdn_chunk_fwd_workspace_size(p)) + \
        G.gdn_chunk_saved_size(p)
    assert bwd_recompute(G, p, ws_bytes=need - 1) == 6
    assert bwd_recompute(G, problem(G, V=64)) == 3
    for name in ("q", "k", "v", "g", "beta", "dO", "dq", "dk", "dv", "dg", "dbeta"):
        assert bwd_recompute(G, p, **{name: None}) == 1, name
    assert bwd_recompute(G, p, h0=FAKE_MISALIGNED) == 8


def conv_problem(G, N=2, T=130, C=64, W=4, act=1, cu_host=(0, 70, 130), dev=FAKE):
    p = G.GdnConvProblem()
    p.N, p.T, p.C, p.W, p.activation = N, T, C, W, act
    p.cu_seqlens = dev
    keep = None
    if cu_host is not None:
        keep = (ctypes.c_int32 * len(cu_host))(*cu_host)
        p.cu_seqlens_host = ctypes.cast(keep, ctypes.c_void_p)
    p._keep = keep
    return p


def conv_fwd(G, p, **over):
    a = dict(x=FAKE, w=FAKE, b=None, si=None, y=FAKE, so=None)
    a.update(over)
    return G._lib.gdn_conv_fwd(ctypes.byref(p), a["x"], a["w"], a["b"], a["si"], a["y"], a["so"],
                               None)


def conv_bwd(G, p, ws_bytes=1 << 40, **over):
    a = dict(x=FAKE, w=FAKE, b=None, si=None, dy=FAKE, dx=FAKE, dw=FAKE, db=None, ds=None,
             ws=FAKE)
    a.update(over)
    return G._lib.gdn_conv_bwd(ctypes.byref(p), *[a[n] for n in (
        "x", "w", "b", "si", "dy", "dx", "dw", "db", "ds", "ws")], ws_bytes, None)


def test_conv_rejects_bad_problems(G):
    for kw, status in ((dict(W=5), 3), (dict(W=1), 3), (dict(C=66), 3), (dict(act=2), 3),
                       (dict(C=0), 2), (dict(N=-1), 2), (dict(N=0), 2),
                       (dict(cu_host=(0, 70, 131)), 4), (dict(cu_host=(0, 90, 80)[:3]), 4)):
        p = conv_problem(G, **kw)
        assert conv_fwd(G, p) == status, kw
        assert conv_bwd(G, p) == status, kw
    assert G._lib.gdn_conv_fwd(None, FAKE, FAKE, None, None, FAKE, None, None) == 1


def test_conv_null_alignment_and_workspace(G):
    p = conv_problem(G)
    for name in ("x", "w", "y"):
        assert conv_fwd(G, p, **{name: None}) == 1, name
    for name in ("x", "w", "dy", "dx", "dw"):
        assert conv_bwd(G, p, **{name: None}) == 1, name
    assert conv_fwd(G, p, x=FAKE + 4) == 8
    assert conv_bwd(G, p, dx=FAKE + 2) == 8
    need = G.gdn_conv_bwd_workspace_size(p)
    assert need > 0 and conv_bwd(G, p, ws_bytes=need - 1) == 6 and conv_bwd(G, p, ws=None) == 6
    q = conv_problem(G)
    q.cu_seqlens = None
    assert conv_fwd(G, q) == 1


def test_conv_paged_and_update_index_rules(G):
    p = conv_problem(G)

    def paged(host, slots=8, **over):
        a = dict(pool=FAKE, idx=FAKE)
        a.update(over)
        keep = (ctypes.c_int32 * len(host))(*host)
        return G._lib.gdn_conv_fwd_paged(ctypes.byref(p), FAKE, FAKE, None, a["pool"], slots,
                                         a["idx"], None, ctypes.cast(keep, ctypes.c_void_p),
                                         FAKE, None)

    assert paged([1, -1]) == 5 and paged([1, 8]) == 5 and paged([3, 3]) == 5
    assert paged([0, 0], pool=None) == 1 and paged([0, 0], slots=-1) == 2

    def upd(host, N=3, C=64, W=4, slots=8, **over):
        a = dict(x=FAKE, w=FAKE, pool=FAKE, idx=FAKE, y=FAKE)
        a.update(over)
        keep = (ctypes.c_int32 * len(host))(*host)
        return G._lib.gdn_conv_update(N, C, W, 1, a["x"], a["w"], None, a["pool"], slots,
                                      a["idx"], ctypes.cast(keep, ctypes.c_void_p), a["y"], None)

    assert upd([1, 0, -3]) == 5 and upd([1, 0, 8]) == 5 and upd([2, 0, 2]) == 5
    assert upd([1, 0, 0], W=5) == 3 and upd([1, 0, 0], C=62) == 3
    assert upd([1, 0, 0], N=0) == 0
    for name in ("x", "w", "pool", "idx", "y"):
        assert upd([1, 0, 2], **{name: None}) == 1, name


def test_allocation_free_paged_prefill_checks_before_touching_the_device(G):
    """Argument errors and a problem past the scratch array are returned before
    the entry point looks up its device array (so nothing here needs a GPU)."""
    assert G.gdn_chunk_fwd_paged_noalloc_max_bytes() == 96 << 20

    def na(p, slots=8, host=None, **over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, idx=FAKE, init=None,
                 o=FAKE, saved=None)
        a.update(over)
        keep = None
        hp = None
        if host is not None:
            keep = (ctypes.c_int32 * len(host))(*host)
            hp = ctypes.cast(keep, ctypes.c_void_p)
        return G._lib.gdn_chunk_fwd_paged_noalloc(
            ctypes.byref(p), a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], slots,
            a["idx"], a["init"], hp, a["o"], a["saved"], None)

    p = problem(G)
    assert na(problem(G, K=64)) == 3
    assert na(p, slots=-1) == 2
    for name in ("pool", "idx", "q", "o"):
        assert na(p, **{name: None}) == 1, name
    assert na(p, host=[1, 8]) == 5
    assert na(p, q=FAKE_MISALIGNED) == 8
    T = 64 * 1024
    big = problem(G, N=2, T=T, H=16, HV=32, cu_host=(0, T // 2, T))
    assert G.gdn_chunk_fwd_workspace_size(big) > G.gdn_chunk_fwd_paged_noalloc_max_bytes()
    assert na(big) == 9
