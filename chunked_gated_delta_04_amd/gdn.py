"""Thin Python binding of libgdn.so (the C ABI declared in include/gdn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library. Functions named gdn_* mirror the C entry points one
for one and take torch tensors (or None for a NULL pointer); the lower-case
helpers at the end allocate outputs and workspaces with torch and call them.

The library is loaded from this package directory. If it is missing, importing
this module raises ImportError: there is no fallback of any kind.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -m chunked_gated_delta_04_amd.build` "
        "(hipcc, gfx950) first")
_lib = ctypes.CDLL(_LIB_PATH)

GDN_OK = 0
STATUS_NAMES = {
    0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
    4: "GDN_ERR_SEQLENS", 5: "GDN_ERR_INDEX", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP",
    8: "GDN_ERR_ALIGN", 9: "GDN_ERR_SCRATCH",
}
EXPORTED = (
    "gdn_status_string", "gdn_num_chunks", "gdn_chunk_saved_size",
    "gdn_chunk_fwd_workspace_size", "gdn_chunk_bwd_workspace_size",
    "gdn_chunk_bwd_recompute_workspace_size",
    "gdn_chunk_fwd", "gdn_chunk_fwd_paged", "gdn_chunk_bwd", "gdn_chunk_bwd_recompute",
    "gdn_chunk_transition", "gdn_recurrent_step",
    "gdn_conv_fwd", "gdn_conv_fwd_paged", "gdn_conv_bwd", "gdn_conv_bwd_workspace_size",
    "gdn_conv_update",
    "gdn_chunk_fwd_timed", "gdn_chunk_bwd_timed", "gdn_stage_name",
    "gdn_chunk_fwd_paged_noalloc", "gdn_chunk_fwd_paged_noalloc_max_bytes",
)
GDN_MAX_STAGES = 8


class GdnProblem(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("scale", ctypes.c_float),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
    ]


class GdnConvProblem(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32),
        ("W", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
    ]


class GdnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({gdn_status_string(status)})")


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i32 = ctypes.c_int32
_P = ctypes.POINTER(GdnProblem)

_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_status_string.argtypes = [ctypes.c_int]
_lib.gdn_num_chunks.restype = ctypes.c_int64
_lib.gdn_num_chunks.argtypes = [_P]
for _n in ("gdn_chunk_saved_size", "gdn_chunk_fwd_workspace_size", "gdn_chunk_bwd_workspace_size",
           "gdn_chunk_bwd_recompute_workspace_size"):
    getattr(_lib, _n).restype = _sz
    getattr(_lib, _n).argtypes = [_P]
_lib.gdn_chunk_fwd.restype = ctypes.c_int
_lib.gdn_chunk_fwd.argtypes = [_P] + [_vp] * 10 + [_sz, _vp]
_lib.gdn_chunk_fwd_paged.restype = ctypes.c_int
_lib.gdn_chunk_fwd_paged.argtypes = [_P] + [_vp] * 6 + [_i32] + [_vp] * 6 + [_sz, _vp]
_lib.gdn_chunk_fwd_paged_noalloc.restype = ctypes.c_int
_lib.gdn_chunk_fwd_paged_noalloc.argtypes = [_P] + [_vp] * 6 + [_i32] + [_vp] * 6
_lib.gdn_chunk_fwd_paged_noalloc_max_bytes.restype = _sz
_lib.gdn_chunk_fwd_paged_noalloc_max_bytes.argtypes = []
_lib.gdn_chunk_bwd.restype = ctypes.c_int
_lib.gdn_chunk_bwd.argtypes = [_P] + [_vp] * 15 + [_sz, _vp]
_lib.gdn_chunk_bwd_recompute.restype = ctypes.c_int
_lib.gdn_chunk_bwd_recompute.argtypes = [_P] + [_vp] * 15 + [_sz, _vp]
_lib.gdn_chunk_transition.restype = ctypes.c_int
_lib.gdn_chunk_transition.argtypes = [_P] + [_vp] * 8 + [_sz, _vp]
_lib.gdn_chunk_fwd_timed.restype = ctypes.c_int
_lib.gdn_chunk_fwd_timed.argtypes = ([_P] + [_vp] * 10 + [_sz, _vp] +
                                     [ctypes.POINTER(_vp), ctypes.POINTER(ctypes.c_int)])
_lib.gdn_chunk_bwd_timed.restype = ctypes.c_int
_lib.gdn_chunk_bwd_timed.argtypes = ([_P] + [_vp] * 15 + [_sz, _vp] +
                                     [ctypes.POINTER(_vp), ctypes.POINTER(ctypes.c_int)])
_CP = ctypes.POINTER(GdnConvProblem)
_lib.gdn_conv_fwd.restype = ctypes.c_int
_lib.gdn_conv_fwd.argtypes = [_CP] + [_vp] * 7
_lib.gdn_conv_fwd_paged.restype = ctypes.c_int
_lib.gdn_conv_fwd_paged.argtypes = [_CP] + [_vp] * 4 + [_i32] + [_vp] * 5
_lib.gdn_conv_bwd_workspace_size.restype = _sz
_lib.gdn_conv_bwd_workspace_size.argtypes = [_CP]
_lib.gdn_conv_bwd.restype = ctypes.c_int
_lib.gdn_conv_bwd.argtypes = [_CP] + [_vp] * 10 + [_sz, _vp]
_lib.gdn_conv_update.restype = ctypes.c_int
_lib.gdn_conv_update.argtypes = [_i32] * 4 + [_vp] * 4 + [_i32] + [_vp] * 4
_lib.gdn_stage_name.restype = ctypes.c_char_p
_lib.gdn_stage_name.argtypes = [ctypes.c_int, ctypes.c_int]
_lib.gdn_recurrent_step.restype = ctypes.c_int
_lib.gdn_recurrent_step.argtypes = ([_i32] * 5 + [ctypes.c_float] + [_vp] * 8 + [_i32] +
                                    [_vp] * 4)


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _host_ptr(t, name):
    """Pointer of a host-side int32 tensor (None -> NULL)."""
    if t is not None and isinstance(t, torch.Tensor) and t.device.type != "cpu":
        raise ValueError(f"{name} must be a CPU tensor")
    return _ptr(t, torch.int32, name)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def make_problem(N, T, H, HV, cu_seqlens, cu_seqlens_host=None, scale=0.0, K=128, V=128,
                 chunk=64):
    """Build the gdn_problem descriptor. cu_seqlens: int32 device tensor [N+1];
    cu_seqlens_host: optional int32 CPU tensor [N+1] (kept alive by the caller)."""
    p = GdnProblem()
    p.N, p.T, p.H, p.HV, p.K, p.V, p.chunk = N, T, H, HV, K, V, chunk
    p.scale = float(scale)
    p.cu_seqlens = _ptr(cu_seqlens, torch.int32, "cu_seqlens")
    if cu_seqlens_host is not None:
        if cu_seqlens_host.device.type != "cpu":
            raise ValueError("cu_seqlens_host must be a CPU tensor")
        p.cu_seqlens_host = _host_ptr(cu_seqlens_host, "cu_seqlens_host")
    return p


def gdn_status_string(status):
    return _lib.gdn_status_string(int(status)).decode()


def gdn_num_chunks(problem):
    return int(_lib.gdn_num_chunks(ctypes.byref(problem)))


def gdn_chunk_saved_size(problem):
    return int(_lib.gdn_chunk_saved_size(ctypes.byref(problem)))


def gdn_chunk_fwd_workspace_size(problem):
    return int(_lib.gdn_chunk_fwd_workspace_size(ctypes.byref(problem)))


def gdn_chunk_bwd_workspace_size(problem):
    return int(_lib.gdn_chunk_bwd_workspace_size(ctypes.byref(problem)))


def gdn_chunk_bwd_recompute_workspace_size(problem):
    return int(_lib.gdn_chunk_bwd_recompute_workspace_size(ctypes.byref(problem)))


def _check(status, where):
    if status != GDN_OK:
        raise GdnError(status, where)


def _check_saved(problem, saved, where):
    """The C calls take `saved` as a bare pointer; refuse a buffer smaller than
    the layout the library reads and writes for this problem."""
    if saved is None:
        return
    have = saved.numel() * saved.element_size()
    need = gdn_chunk_saved_size(problem)
    if have < need:
        raise ValueError(f"{where}: saved holds {have} bytes, the problem needs {need} "
                         "(gdn_chunk_saved_size)")


def gdn_chunk_fwd(problem, q, k, v, g, beta, h0, o, hT, saved, workspace, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    _check_saved(problem, saved, "gdn_chunk_fwd")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gdn_chunk_fwd(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(h0, f32, "h0"), _ptr(o, bf, "o"),
        _ptr(hT, f32, "hT"), _ptr(saved, None, "saved"), _ptr(workspace, None, "workspace"),
        ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_fwd")


def gdn_chunk_fwd_paged(problem, q, k, v, g, beta, state_pool, slots, ssm_state_indices,
                        has_initial_state, indices_host, o, saved, workspace, stream=None):
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _check_saved(problem, saved, "gdn_chunk_fwd_paged")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gdn_chunk_fwd_paged(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(state_pool, f32, "state_pool"),
        int(slots), _ptr(ssm_state_indices, i32, "ssm_state_indices"),
        _ptr(has_initial_state, i32, "has_initial_state"),
        _host_ptr(indices_host, "indices_host"), _ptr(o, bf, "o"), _ptr(saved, None, "saved"),
        _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_fwd_paged")


def gdn_chunk_fwd_paged_noalloc_max_bytes():
    return int(_lib.gdn_chunk_fwd_paged_noalloc_max_bytes())


def gdn_chunk_fwd_paged_noalloc(problem, q, k, v, g, beta, state_pool, slots, ssm_state_indices,
                                has_initial_state, indices_host, o, saved, stream=None):
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _check_saved(problem, saved, "gdn_chunk_fwd_paged_noalloc")
    st = _lib.gdn_chunk_fwd_paged_noalloc(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(state_pool, f32, "state_pool"),
        int(slots), _ptr(ssm_state_indices, i32, "ssm_state_indices"),
        _ptr(has_initial_state, i32, "has_initial_state"),
        _host_ptr(indices_host, "indices_host"), _ptr(o, bf, "o"), _ptr(saved, None, "saved"),
        _stream(stream))
    _check(st, "gdn_chunk_fwd_paged_noalloc")


def gdn_stage_name(op, stage):
    return _lib.gdn_stage_name(int(op), int(stage)).decode()


def gdn_chunk_fwd_timed(problem, q, k, v, g, beta, h0, o, hT, saved, workspace, events,
                        stream=None):
    """gdn_chunk_fwd recording events (a ctypes array of 2*GDN_MAX_STAGES hipEvent_t;
    NULL entries are skipped) around each stage. Returns the number of stages launched."""
    bf, f32 = torch.bfloat16, torch.float32
    _check_saved(problem, saved, "gdn_chunk_fwd_timed")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    n = ctypes.c_int(0)
    st = _lib.gdn_chunk_fwd_timed(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(h0, f32, "h0"), _ptr(o, bf, "o"),
        _ptr(hT, f32, "hT"), _ptr(saved, None, "saved"), _ptr(workspace, None, "workspace"),
        ws_bytes, _stream(stream), events, ctypes.byref(n))
    _check(st, "gdn_chunk_fwd_timed")
    return n.value


def gdn_chunk_bwd_timed(problem, q, k, v, g, beta, saved, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                        workspace, events, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    _check_saved(problem, saved, "gdn_chunk_bwd_timed")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    n = ctypes.c_int(0)
    st = _lib.gdn_chunk_bwd_timed(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(saved, None, "saved"),
        _ptr(dO, bf, "dO"), _ptr(dhT, f32, "dhT"), _ptr(dq, bf, "dq"), _ptr(dk, bf, "dk"),
        _ptr(dv, bf, "dv"), _ptr(dg, f32, "dg"), _ptr(dbeta, f32, "dbeta"),
        _ptr(dh0, f32, "dh0"), _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream),
        events, ctypes.byref(n))
    _check(st, "gdn_chunk_bwd_timed")
    return n.value


def gdn_chunk_bwd(problem, q, k, v, g, beta, saved, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                  workspace, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    _check_saved(problem, saved, "gdn_chunk_bwd")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gdn_chunk_bwd(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(saved, None, "saved"),
        _ptr(dO, bf, "dO"), _ptr(dhT, f32, "dhT"), _ptr(dq, bf, "dq"), _ptr(dk, bf, "dk"),
        _ptr(dv, bf, "dv"), _ptr(dg, f32, "dg"), _ptr(dbeta, f32, "dbeta"),
        _ptr(dh0, f32, "dh0"), _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_bwd")


def gdn_chunk_bwd_recompute(problem, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                            workspace, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gdn_chunk_bwd_recompute(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(h0, f32, "h0"),
        _ptr(dO, bf, "dO"), _ptr(dhT, f32, "dhT"), _ptr(dq, bf, "dq"), _ptr(dk, bf, "dk"),
        _ptr(dv, bf, "dv"), _ptr(dg, f32, "dg"), _ptr(dbeta, f32, "dbeta"),
        _ptr(dh0, f32, "dh0"), _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_bwd_recompute")


def gdn_chunk_transition(problem, q, k, v, g, beta, M, s, workspace, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gdn_chunk_transition(
        ctypes.byref(problem), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(g, f32, "g"), _ptr(beta, f32, "beta"), _ptr(M, f32, "M"), _ptr(s, f32, "s"),
        _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream))
    _check(st, "gdn_chunk_transition")


def gdn_recurrent_step(N, H, HV, K, V, scale, q, k, v, a, b, A_log, dt_bias, state_pool, slots,
                       ssm_state_indices, indices_host, o, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    st = _lib.gdn_recurrent_step(
        N, H, HV, K, V, float(scale), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(a, bf, "a"), _ptr(b, bf, "b"), _ptr(A_log, f32, "A_log"),
        _ptr(dt_bias, f32, "dt_bias"), _ptr(state_pool, f32, "state_pool"), slots,
        _ptr(ssm_state_indices, torch.int32, "ssm_state_indices"),
        _host_ptr(indices_host, "indices_host"), _ptr(o, bf, "o"), _stream(stream))
    _check(st, "gdn_recurrent_step")


# ---------------------------------------------------------------- allocating helpers
def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def chunk_fwd(q, k, v, g, beta, cu_seqlens, h0=None, scale=0.0, cu_seqlens_host=None,
              save_for_backward=False, output_final_state=True, stream=None):
    """Allocate outputs and workspace and run gdn_chunk_fwd.

    q, k [T, H, 128] bf16; v [T, HV, 128] bf16; g, beta [T, HV] fp32 (device);
    cu_seqlens [N+1] int32 (device). Returns (o, hT or None, saved or None).
    """
    T, H, _ = q.shape
    HV = v.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_problem(N, T, H, HV, cu_seqlens, cu_seqlens_host, scale)
    dev = q.device
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device=dev)
    hT = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev) if output_final_state else None
    saved = _ws(gdn_chunk_saved_size(p), dev) if save_for_backward else None
    ws = _ws(gdn_chunk_fwd_workspace_size(p), dev)
    gdn_chunk_fwd(p, q, k, v, g, beta, h0, o, hT, saved, ws, stream)
    return o, hT, saved


def chunk_fwd_paged(q, k, v, g, beta, cu_seqlens, state_pool, ssm_state_indices,
                    has_initial_state=None, indices_host=None, scale=0.0, cu_seqlens_host=None,
                    save_for_backward=False, stream=None):
    """Allocate o (and saved, workspace) and run gdn_chunk_fwd_paged; the pool
    [slots, HV, 128, 128] fp32 is updated in place. Returns (o, saved or None)."""
    T, H, _ = q.shape
    HV = v.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_problem(N, T, H, HV, cu_seqlens, cu_seqlens_host, scale)
    dev = q.device
    o = torch.empty(T, HV, 128, dtype=torch.bfloat16, device=dev)
    saved = _ws(gdn_chunk_saved_size(p), dev) if save_for_backward else None
    ws = _ws(gdn_chunk_fwd_workspace_size(p), dev)
    gdn_chunk_fwd_paged(p, q, k, v, g, beta, state_pool, state_pool.shape[0], ssm_state_indices,
                        has_initial_state, indices_host, o, saved, ws, stream)
    return o, saved


def chunk_bwd(q, k, v, g, beta, cu_seqlens, saved, dO, dhT=None, scale=0.0,
              cu_seqlens_host=None, want_dh0=True, stream=None):
    """Allocate gradients and workspace and run gdn_chunk_bwd.

    Returns dict dq, dk, dv, dg, dbeta, dh0 (dh0 None unless want_dh0).
    """
    T, H, _ = q.shape
    HV = v.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_problem(N, T, H, HV, cu_seqlens, cu_seqlens_host, scale)
    dev = q.device
    out = dict(
        dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
        dg=torch.empty(T, HV, dtype=torch.float32, device=dev),
        dbeta=torch.empty(T, HV, dtype=torch.float32, device=dev),
        dh0=torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev) if want_dh0 else None,
    )
    ws = _ws(gdn_chunk_bwd_workspace_size(p), dev)
    gdn_chunk_bwd(p, q, k, v, g, beta, saved, dO, dhT, out["dq"], out["dk"], out["dv"],
                  out["dg"], out["dbeta"], out["dh0"], ws, stream)
    return out


def chunk_bwd_recompute(q, k, v, g, beta, cu_seqlens, dO, h0=None, dhT=None, scale=0.0,
                        cu_seqlens_host=None, want_dh0=True, stream=None):
    """Allocate gradients and workspace and run gdn_chunk_bwd_recompute (no saved
    buffer: the per-chunk states are rebuilt from h0). Returns the dict of chunk_bwd."""
    T, H, _ = q.shape
    HV = v.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_problem(N, T, H, HV, cu_seqlens, cu_seqlens_host, scale)
    dev = q.device
    out = dict(
        dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
        dg=torch.empty(T, HV, dtype=torch.float32, device=dev),
        dbeta=torch.empty(T, HV, dtype=torch.float32, device=dev),
        dh0=torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev) if want_dh0 else None,
    )
    ws = _ws(gdn_chunk_bwd_recompute_workspace_size(p), dev)
    gdn_chunk_bwd_recompute(p, q, k, v, g, beta, h0, dO, dhT, out["dq"], out["dk"], out["dv"],
                            out["dg"], out["dbeta"], out["dh0"], ws, stream)
    return out


def chunk_transition(q, k, v, g, beta, cu_seqlens, scale=0.0, cu_seqlens_host=None,
                     stream=None):
    """Allocate M [N, HV, 128, 128] and s [N, HV, 128, 128] (fp32) and run
    gdn_chunk_transition: each sequence's end state is S_0 @ M + s."""
    T, H, _ = q.shape
    HV = v.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_problem(N, T, H, HV, cu_seqlens, cu_seqlens_host, scale)
    dev = q.device
    M = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev)
    s = torch.empty(N, HV, 128, 128, dtype=torch.float32, device=dev)
    ws = _ws(gdn_chunk_fwd_workspace_size(p), dev)
    gdn_chunk_transition(p, q, k, v, g, beta, M, s, ws, stream)
    return M, s


def recurrent_step(q, k, v, a, b, A_log, dt_bias, state_pool, ssm_state_indices,
                   indices_host=None, scale=0.0, stream=None):
    """Allocate o and run gdn_recurrent_step (the pool is updated in place)."""
    N, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    o = torch.empty(N, HV, V, dtype=torch.bfloat16, device=q.device)
    gdn_recurrent_step(N, H, HV, K, V, scale, q, k, v, a, b, A_log, dt_bias, state_pool,
                       state_pool.shape[0], ssm_state_indices, indices_host, o, stream)
    return o


# ---------------------------------------------------------------- short convolution
_ACT = {None: 0, "none": 0, "silu": 1}


def make_conv_problem(N, T, C, W, cu_seqlens, cu_seqlens_host=None, activation="silu"):
    """Descriptor of one short-convolution call (cu_seqlens: int32 device [N+1];
    cu_seqlens_host: optional int32 CPU copy, kept alive by the caller)."""
    p = GdnConvProblem()
    p.N, p.T, p.C, p.W = N, T, C, W
    p.activation = _ACT[activation]
    p.cu_seqlens = _ptr(cu_seqlens, torch.int32, "cu_seqlens")
    if cu_seqlens_host is not None:
        p.cu_seqlens_host = _host_ptr(cu_seqlens_host, "cu_seqlens_host")
    return p


def gdn_conv_fwd(problem, x, weight, bias, state_in, y, state_out, stream=None):
    bf = torch.bfloat16
    st = _lib.gdn_conv_fwd(ctypes.byref(problem), _ptr(x, bf, "x"), _ptr(weight, bf, "weight"),
                           _ptr(bias, bf, "bias"), _ptr(state_in, bf, "state_in"),
                           _ptr(y, bf, "y"), _ptr(state_out, bf, "state_out"), _stream(stream))
    _check(st, "gdn_conv_fwd")


def gdn_conv_fwd_paged(problem, x, weight, bias, state_pool, slots, indices, has_initial_state,
                       indices_host, y, stream=None):
    bf, i32 = torch.bfloat16, torch.int32
    st = _lib.gdn_conv_fwd_paged(
        ctypes.byref(problem), _ptr(x, bf, "x"), _ptr(weight, bf, "weight"),
        _ptr(bias, bf, "bias"), _ptr(state_pool, bf, "state_pool"), int(slots),
        _ptr(indices, i32, "indices"), _ptr(has_initial_state, i32, "has_initial_state"),
        _host_ptr(indices_host, "indices_host"), _ptr(y, bf, "y"), _stream(stream))
    _check(st, "gdn_conv_fwd_paged")


def gdn_conv_bwd_workspace_size(problem):
    return int(_lib.gdn_conv_bwd_workspace_size(ctypes.byref(problem)))


def gdn_conv_bwd(problem, x, weight, bias, state_in, dy, dx, dweight, dbias, dstate_in,
                 workspace, stream=None):
    bf, f32 = torch.bfloat16, torch.float32
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gdn_conv_bwd(
        ctypes.byref(problem), _ptr(x, bf, "x"), _ptr(weight, bf, "weight"),
        _ptr(bias, bf, "bias"), _ptr(state_in, bf, "state_in"), _ptr(dy, bf, "dy"),
        _ptr(dx, bf, "dx"), _ptr(dweight, f32, "dweight"), _ptr(dbias, f32, "dbias"),
        _ptr(dstate_in, f32, "dstate_in"), _ptr(workspace, None, "workspace"), ws_bytes,
        _stream(stream))
    _check(st, "gdn_conv_bwd")


def gdn_conv_update(N, C, W, activation, x, weight, bias, state_pool, slots, indices,
                    indices_host, y, stream=None):
    bf, i32 = torch.bfloat16, torch.int32
    st = _lib.gdn_conv_update(
        int(N), int(C), int(W), _ACT[activation], _ptr(x, bf, "x"), _ptr(weight, bf, "weight"),
        _ptr(bias, bf, "bias"), _ptr(state_pool, bf, "state_pool"), int(slots),
        _ptr(indices, i32, "indices"), _host_ptr(indices_host, "indices_host"), _ptr(y, bf, "y"),
        _stream(stream))
    _check(st, "gdn_conv_update")


def conv_fwd(x, weight, bias, cu_seqlens, state_in=None, activation="silu",
             cu_seqlens_host=None, want_state=True, stream=None):
    """x [T, C] bf16, weight [C, W] bf16, bias [C] bf16 or None (device).
    Returns (y [T, C] bf16, end states [N, C, W-1] bf16 or None)."""
    T, C = x.shape
    W = weight.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_conv_problem(N, T, C, W, cu_seqlens, cu_seqlens_host, activation)
    y = torch.empty_like(x)
    so = torch.empty(N, C, W - 1, dtype=torch.bfloat16, device=x.device) if want_state else None
    gdn_conv_fwd(p, x, weight, bias, state_in, y, so, stream)
    return y, so


def conv_fwd_paged(x, weight, bias, cu_seqlens, state_pool, indices, has_initial_state=None,
                   indices_host=None, activation="silu", cu_seqlens_host=None, stream=None):
    """Paged forward: state_pool [slots, C, W-1] bf16 is read and updated in place."""
    T, C = x.shape
    W = weight.shape[1]
    N = cu_seqlens.numel() - 1
    p = make_conv_problem(N, T, C, W, cu_seqlens, cu_seqlens_host, activation)
    y = torch.empty_like(x)
    gdn_conv_fwd_paged(p, x, weight, bias, state_pool, state_pool.shape[0], indices,
                       has_initial_state, indices_host, y, stream)
    return y


def conv_bwd(x, weight, bias, cu_seqlens, dy, state_in=None, activation="silu",
             cu_seqlens_host=None, want_dstate=True, stream=None):
    """Returns dict dx [T, C] bf16, dweight [C, W] fp32, dbias [C] fp32 (None
    without a bias), dstate [N, C, W-1] fp32 (None unless want_dstate)."""
    T, C = x.shape
    W = weight.shape[1]
    N = cu_seqlens.numel() - 1
    dev = x.device
    p = make_conv_problem(N, T, C, W, cu_seqlens, cu_seqlens_host, activation)
    out = dict(dx=torch.empty_like(x),
               dweight=torch.empty(C, W, dtype=torch.float32, device=dev),
               dbias=torch.empty(C, dtype=torch.float32, device=dev) if bias is not None else None,
               dstate=torch.empty(N, C, W - 1, dtype=torch.float32, device=dev)
               if want_dstate else None)
    ws = _ws(gdn_conv_bwd_workspace_size(p), dev)
    gdn_conv_bwd(p, x, weight, bias, state_in, dy, out["dx"], out["dweight"], out["dbias"],
                 out["dstate"], ws, stream)
    return out


def conv_update(x, weight, bias, state_pool, indices, indices_host=None, activation="silu",
                stream=None):
    """One decode token per row; state_pool [slots, C, W-1] bf16 updated in place."""
    N, C = x.shape
    W = weight.shape[1]
    y = torch.empty_like(x)
    gdn_conv_update(N, C, W, activation, x, weight, bias, state_pool, state_pool.shape[0],
                    indices, indices_host, y, stream)
    return y
