"""Token-by-token fp64 oracle of the gated delta rule: forward, adjoint, decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What it computes, and where the pages define it
-----------------------------------------------
* Recurrence. Per sequence and value head the state S is a V x K matrix and
  S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
  o_t = S_t q_t with q already scaled. Written as in the method's statement of
  the state recurrence on the "[WS1][CUDA][Qwen3-Next] C6: GDN decode-step
  goldens" page (RL-Kernel PR #469, "What" section and the agent note listing
  where the kernel and the HF model disagree): decay first, then the
  delta-rule correction delta = beta (v - S k), then the rank-1 write, then
  the read-out with the updated state.
* Normalisation. q and k are divided by sqrt(sum(x*x) + 1e-6) (a division by
  the square root, not a multiply by an rsqrt), q is then multiplied by the
  scale, K^-1/2 unless given, and k is never scaled; each is normalised
  exactly once (same page, same note).
* Grouped value heads. Value head hv reads key head hv // (HV // H), with no
  copy of q or k (same page, "What" section; the Cake page, "API and flags",
  requires HV % H == 0).
* Varlen packing. Sequences are packed along the token axis and delimited by
  cu_seqlens [N+1]; each sequence starts from its own initial state, zero if
  none is given (the Cake page "[Cake 1/13] gdn", "API and flags").
* Decode step. beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias),
  softplus(x) = x above the threshold 20 and log(1 + e^x) otherwise, then one
  recurrence step in place on a state pool [slots, HV, V, K] addressed by
  ssm_state_indices; every index <= 0 is skipped (zero output, state block
  untouched) and an active index out of range or repeated raises (RL-Kernel
  PR #469, "What" section, the state-contract bullet).
* Paged prefill. The forward above with each sequence's start state read
  from, and its end state written back to, block ssm_state_indices[n] of the
  decode pool, in place of a gathered h0 and a scattered hT; a sequence whose
  has_initial_state flag is 0 starts from zero (a fresh prompt), one with a
  flag of 1 resumes from the block (the torchtitan PR #4389 page, its
  serving-path section and the paged-state continuity results). The pages
  leave open what a sequence with the null index does; here it runs from a
  zero state and its end state is dropped.
* Transition (one GPU's share of a context-parallel forward). Over a
  sequence the end state is affine in the start state, S_end = S_0 M + s,
  where M is the product, in token order, of the per-token maps
  e^{g_t} (I - beta_t k_t k_t^T) (K x K) and s is the end state from a zero
  start (the maxtext page "Qwen3.5-397B RL trainer on 128 v7x", the commit
  adding the gdn_cp_m_scan transition product and pass 1's end state).
* Backward. The manual adjoint of the recurrence, taken in reverse token
  order, gives dq, dk, dv, dg, dbeta and dh0 (the gradient set required by
  the cake_gdn page, miles PR #3597, "Summary" and "Tests").

Everything is float64; inputs are upcast exactly from whatever dtype they
hold, and outputs are rounded only by the caller when comparing.
"""
import numpy as np

EPS = 1e-6
SOFTPLUS_THRESHOLD = 20.0


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def l2norm(x):
    """x / sqrt(sum(x*x) + 1e-6) over the last axis."""
    x = _f64(x)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + EPS)


def l2norm_backward(x, dxhat):
    """Pull a gradient back through l2norm.

    With n = sqrt(sum x^2 + eps) and xhat = x / n, d xhat_a / d x_b =
    delta_ab / n - x_a x_b / n^3, so dx = (dxhat - xhat (xhat . dxhat)) / n.
    """
    x = _f64(x)
    dxhat = _f64(dxhat)
    n = np.sqrt((x * x).sum(-1, keepdims=True) + EPS)
    xh = x / n
    return (dxhat - xh * (xh * dxhat).sum(-1, keepdims=True)) / n


def _check_seqlens(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return cu


def _head_map(H, HV):
    if H <= 0 or HV % H != 0:
        raise ValueError("HV must be a positive multiple of H")
    return np.arange(HV) // (HV // H)


def _prepare(q, k, v, g, beta, cu_seqlens, scale):
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    T, H, K = q.shape
    HV = v.shape[1]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, HV) or beta.shape != (T, HV):
        raise ValueError("shape mismatch")
    hmap = _head_map(H, HV)
    cu = _check_seqlens(cu_seqlens, T)
    if scale is None:
        scale = K ** -0.5
    qt = scale * l2norm(q)[:, hmap, :]     # [T, HV, K]
    kh = l2norm(k)[:, hmap, :]             # [T, HV, K]
    return q, k, v, g, beta, cu, hmap, float(scale), qt, kh


def _step(S, g_t, beta_t, v_t, k_t):
    """One decayed delta-rule write. Returns (S_decayed, delta, S_new)."""
    Sd = S * np.exp(g_t)[..., None, None]
    pred = np.einsum("...vk,...k->...v", Sd, k_t)
    delta = beta_t[..., None] * (v_t - pred)
    S_new = Sd + delta[..., :, None] * k_t[..., None, :]
    return Sd, delta, S_new


def forward(q, k, v, g, beta, cu_seqlens, h0=None, scale=None):
    """Forward of the gated delta rule over a varlen pack.

    q, k  [T, H, K]; v [T, HV, V]; g, beta [T, HV] (g is the log-decay);
    cu_seqlens [N+1]; h0 [N, HV, V, K] or None (zero).
    Returns o [T, HV, V] and the final states hT [N, HV, V, K], both float64.
    """
    q, k, v, g, beta, cu, hmap, scale, qt, kh = _prepare(q, k, v, g, beta, cu_seqlens, scale)
    T, HV, V = v.shape
    K = q.shape[2]
    N = cu.size - 1
    S = np.zeros((N, HV, V, K)) if h0 is None else _f64(h0).copy()
    if S.shape != (N, HV, V, K):
        raise ValueError("h0 shape")
    o = np.zeros((T, HV, V))
    lens = np.diff(cu)
    for s in range(int(lens.max()) if N else 0):
        act = np.nonzero(lens > s)[0]
        t = cu[act] + s
        _, _, S_new = _step(S[act], g[t], beta[t], v[t], kh[t])
        o[t] = np.einsum("ahvk,ahk->ahv", S_new, qt[t])
        S[act] = S_new
    return o, S


def backward(q, k, v, g, beta, cu_seqlens, do, h0=None, dhT=None, scale=None, ckpt=64):
    """Manual adjoint of :func:`forward`.

    do [T, HV, V]; dhT [N, HV, V, K] or None (zero cotangent of the final state).
    Returns dict with dq, dk [T, H, K], dv [T, HV, V], dg, dbeta [T, HV] and
    dh0 [N, HV, V, K], float64.

    The forward states are kept at every ``ckpt``-th step and replayed segment by
    segment; per token, with S' = exp(g) S_prev the decayed state,
    delta = beta (v - S' k) and S = S' + delta k^T, the reverse step is
      dS += do q^T;  dq~ = S^T do
      ddelta = dS k;  dk = dS^T delta - beta S'^T ddelta
      dv = beta ddelta;  dbeta = ddelta . (v - S' k)
      dS' = dS - beta ddelta k^T;  dg = <dS', S'>;  dS_prev = exp(g) dS'.
    Then dq^ = scale dq~, the value-head gradients of q^ and k^ are summed per key
    head, and both go back through the L2 norm.
    """
    q, k, v, g, beta, cu, hmap, scale, qt, kh = _prepare(q, k, v, g, beta, cu_seqlens, scale)
    do = _f64(do)
    T, HV, V = v.shape
    H, K = q.shape[1], q.shape[2]
    N = cu.size - 1
    lens = np.diff(cu)
    maxlen = int(lens.max()) if N else 0
    S = np.zeros((N, HV, V, K)) if h0 is None else _f64(h0).copy()
    # checkpoints of the state before step s, for s = 0, ckpt, 2 ckpt, ...
    ckpts = []
    for s in range(maxlen):
        if s % ckpt == 0:
            ckpts.append(S.copy())
        act = np.nonzero(lens > s)[0]
        t = cu[act] + s
        _, _, S_new = _step(S[act], g[t], beta[t], v[t], kh[t])
        S[act] = S_new

    dS = np.zeros((N, HV, V, K)) if dhT is None else _f64(dhT).copy()
    dqt = np.zeros((T, HV, K))
    dkh = np.zeros((T, HV, K))
    dv = np.zeros((T, HV, V))
    dg = np.zeros((T, HV))
    dbeta = np.zeros((T, HV))
    for seg in range(len(ckpts) - 1, -1, -1):
        s0 = seg * ckpt
        s1 = min(maxlen, s0 + ckpt)
        # replay the segment, keeping the state before each step
        Sr = ckpts[seg].copy()
        before = []
        for s in range(s0, s1):
            before.append(Sr.copy())
            act = np.nonzero(lens > s)[0]
            t = cu[act] + s
            _, _, S_new = _step(Sr[act], g[t], beta[t], v[t], kh[t])
            Sr[act] = S_new
        for s in range(s1 - 1, s0 - 1, -1):
            act = np.nonzero(lens > s)[0]
            t = cu[act] + s
            kt, qtt, bt = kh[t], qt[t], beta[t]
            Sd, delta, S_new = _step(before[s - s0][act], g[t], bt, v[t], kt)
            dSa = dS[act] + do[t][:, :, :, None] * qtt[:, :, None, :]
            dqt[t] = np.einsum("ahvk,ahv->ahk", S_new, do[t])
            ddelta = np.einsum("ahvk,ahk->ahv", dSa, kt)
            dk_t = np.einsum("ahvk,ahv->ahk", dSa, delta)
            dv[t] = bt[..., None] * ddelta
            pred = np.einsum("ahvk,ahk->ahv", Sd, kt)
            dbeta[t] = (ddelta * (v[t] - pred)).sum(-1)
            dSd = dSa - bt[..., None, None] * ddelta[..., :, None] * kt[..., None, :]
            dk_t -= bt[..., None] * np.einsum("ahvk,ahv->ahk", Sd, ddelta)
            dkh[t] = dk_t
            dg[t] = (dSd * Sd).sum((-1, -2))
            dS[act] = np.exp(g[t])[..., None, None] * dSd

    # value heads of one key head share q^ and k^: sum their gradients
    dqhat = np.zeros((T, H, K))
    dkhat = np.zeros((T, H, K))
    for hv in range(HV):
        dqhat[:, hmap[hv]] += scale * dqt[:, hv]
        dkhat[:, hmap[hv]] += dkh[:, hv]
    return {
        "dq": l2norm_backward(q, dqhat),
        "dk": l2norm_backward(k, dkhat),
        "dv": dv,
        "dg": dg,
        "dbeta": dbeta,
        "dh0": dS,
    }


def softplus_thresholded(x):
    """softplus with the decode kernel's threshold: x if x > 20 else log(1 + e^x)."""
    x = _f64(x)
    return np.where(x > SOFTPLUS_THRESHOLD, x, np.log1p(np.exp(np.minimum(x, SOFTPLUS_THRESHOLD))))


def decode_gating(a, b, A_log, dt_bias):
    """Fused decode gating: beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias).

    a, b [N, HV]; A_log, dt_bias [HV]. Returns (g, beta), float64 [N, HV].
    """
    a, b, A_log, dt_bias = (_f64(x) for x in (a, b, A_log, dt_bias))
    g = -np.exp(A_log)[None, :] * softplus_thresholded(a + dt_bias[None, :])
    beta = 1.0 / (1.0 + np.exp(-b))
    return g, beta


def decode_step(q, k, v, a, b, A_log, dt_bias, state_pool, ssm_state_indices, scale=None):
    """One recurrent decode step over a state pool.

    q, k [N, H, K]; v [N, HV, V]; a, b [N, HV]; A_log, dt_bias [HV];
    state_pool [slots, HV, V, K]; ssm_state_indices [N].
    Rows whose index is <= 0 are skipped: their output is zero and no state
    block is touched (block 0 is the null block and is never written). An
    active index >= slots, or one used by two rows, raises ValueError.
    Returns (o [N, HV, V], new_pool [slots, HV, V, K]) in float64; the input
    pool is not modified.
    """
    idx = np.asarray(ssm_state_indices, dtype=np.int64).reshape(-1)
    pool = _f64(state_pool).copy()
    slots = pool.shape[0]
    N = idx.size
    active = np.nonzero(idx > 0)[0]
    ai = idx[active]
    if np.any(ai >= slots):
        raise ValueError("active state index out of range")
    if np.unique(ai).size != ai.size:
        raise ValueError("repeated active state index")
    HV, V = _f64(v).shape[1], _f64(v).shape[2]
    o = np.zeros((N, HV, V))
    if active.size == 0:
        return o, pool
    g, beta = decode_gating(a, b, A_log, dt_bias)
    sel = lambda x: _f64(x)[active]  # noqa: E731
    o_a, hT = forward(sel(q), sel(k), sel(v), g[active], beta[active],
                      np.arange(active.size + 1), h0=pool[ai], scale=scale)
    o[active] = o_a
    pool[ai] = hT
    return o, pool


def paged_forward(q, k, v, g, beta, cu_seqlens, state_pool, ssm_state_indices,
                  has_initial_state=None, scale=None):
    """Forward over a varlen pack whose states live in a pool [slots, HV, V, K].

    Sequence n uses block ssm_state_indices[n]: it starts from that block when
    has_initial_state[n] is nonzero (None: every flag is 1) and from zero
    otherwise, and its end state replaces the block. An index <= 0 names no
    block: zero start, end state dropped. An active index >= slots, or one
    used twice, raises ValueError. Returns (o [T, HV, V], new_pool) in float64;
    the input pool is not modified.
    """
    idx = np.asarray(ssm_state_indices, dtype=np.int64).reshape(-1)
    pool = _f64(state_pool).copy()
    slots = pool.shape[0]
    N = idx.size
    init = np.ones(N, dtype=np.int64) if has_initial_state is None else \
        np.asarray(has_initial_state, dtype=np.int64).reshape(-1)
    live = np.nonzero(idx > 0)[0]
    if np.any(idx[live] >= slots):
        raise ValueError("active state index out of range")
    if np.unique(idx[live]).size != live.size:
        raise ValueError("repeated active state index")
    h0 = np.zeros((N,) + pool.shape[1:])
    resumed = live[init[live] != 0]
    h0[resumed] = pool[idx[resumed]]
    o, hT = forward(q, k, v, g, beta, cu_seqlens, h0=h0, scale=scale)
    pool[idx[live]] = hT[live]
    return o, pool


def transition(q, k, v, g, beta, cu_seqlens, scale=None):
    """Per sequence and value head, M [K, K] and s [V, K] with S_end = S_0 @ M + s.

    M multiplies the token maps e^{g_t} (I - beta_t k_t k_t^T) in token order;
    s is the forward's end state from a zero start. A sequence without tokens
    gets M = I and s = 0. Returns (M [N, HV, K, K], s [N, HV, V, K]) in float64.
    """
    q, k, v, g, beta, cu, hmap, scale, qt, kh = _prepare(q, k, v, g, beta, cu_seqlens, scale)
    T, HV, V = v.shape
    K = q.shape[2]
    N = cu.size - 1
    M = np.broadcast_to(np.eye(K), (N, HV, K, K)).copy()
    eye = np.eye(K)
    for n in range(N):
        for t in range(cu[n], cu[n + 1]):
            kt = kh[t]                                        # [HV, K]
            step = np.exp(g[t])[:, None, None] * (
                eye[None] - beta[t][:, None, None] * kt[:, :, None] * kt[:, None, :])
            M[n] = M[n] @ step
    _, s = forward(q, k, v, g, beta, cu, None, scale)
    return M, s
