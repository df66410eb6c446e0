"""fp64 oracle of the causal short convolution that precedes the gated delta
rule: varlen forward with carried states, its adjoint, the decode update over
a state pool, and the paged prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What it computes, and where the pages define it
-----------------------------------------------
* Forward. Per channel c a depthwise causal filter of width W over the
  tokens of one sequence, preceded by that sequence's W - 1 carried inputs
  (its conv state, zero for a fresh sequence):
      pre_t = bias_c + sum_{i<W} w[c, i] * xe[t + i],   y_t = act(pre_t)
  where xe is the state followed by the sequence's inputs, so that tap W - 1
  meets the current token. act is SiLU (x * sigmoid(x)) or the identity. The
  end state is the last W - 1 entries of xe. The goldens page
  ("[WS1][CUDA][Qwen3-Next] C6: GDN decode-step goldens and recurrent/conv
  state contract", RL-Kernel PR #469, "What": the conv update golden, its
  bias and SiLU, and the state contract [num_blocks, dim, W - 1]) and its
  provider comparison (W = 4, dim 8192, SiLU) fix the shape; the cake_gdn page
  (miles PR #3597, "What the commits add") places the short convolution in
  front of the recurrence and asks for a weight gradient without atomics.
* Backward. The adjoint of the forward: dpre = dy * act'(pre), dxe gathers
  w * dpre over the taps, dw and dbias sum over the tokens; the first W - 1
  entries of dxe are the gradient of the carried state. act' of SiLU is
  sigmoid(x) (1 + x (1 - sigmoid(x))), with the sigmoid evaluated without
  overflow (the goldens page's review notes a NaN from exp(-x) overflowing
  below -88.7 in a reference; this one has none).
* Update (decode). One token per row on a pool [slots, dim, W - 1] addressed
  by indices: index 0 is the null block (row skipped: zero output, no block
  touched); an index that is negative, >= slots or repeated among active
  rows raises (the goldens page's conv rule, which differs from the
  recurrent step's <= 0 rule).
* Paged prefill. The forward whose carried states come from pool blocks and
  whose end states are written back, with has_initial_state choosing a
  resumed or a fresh start (the torchtitan PR #4389 page: paged causal
  convolution reading fresh or resumed cache slots and advancing them in
  place). Index 0 gives the sequence no block (zero start, end state
  dropped); the pages leave that case open and this is the reading taken.

Everything is float64; inputs are upcast exactly.
"""
import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def act_forward(pre, activation):
    return pre * sigmoid(pre) if activation == "silu" else pre


def act_grad(pre, activation):
    if activation != "silu":
        return np.ones_like(pre)
    s = sigmoid(pre)
    return s * (1.0 + pre * (1.0 - s))


def _bounds(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("bad cu_seqlens")
    return cu


def _extended(x, cu, n, state_in, W):
    """xe for sequence n: [W - 1 + L, C], the carried inputs then the tokens."""
    C = x.shape[1]
    hist = np.zeros((W - 1, C)) if state_in is None else _f64(state_in)[n].T
    return np.concatenate([hist, x[cu[n]:cu[n + 1]]], axis=0)


def conv_forward(x, weight, bias, cu_seqlens, state_in=None, activation="silu"):
    """x [T, C]; weight [C, W]; bias [C] or None; state_in [N, C, W-1] or None.

    Returns y [T, C] and the end states [N, C, W-1], float64.
    """
    x, w = _f64(x), _f64(weight)
    T, C = x.shape
    W = w.shape[1]
    b = np.zeros(C) if bias is None else _f64(bias)
    cu = _bounds(cu_seqlens, T)
    N = cu.size - 1
    y = np.zeros((T, C))
    state_out = np.zeros((N, C, W - 1))
    for n in range(N):
        xe = _extended(x, cu, n, state_in, W)
        L = cu[n + 1] - cu[n]
        pre = np.tile(b, (L, 1))
        for i in range(W):
            pre += w[:, i][None, :] * xe[i:i + L]
        y[cu[n]:cu[n + 1]] = act_forward(pre, activation)
        state_out[n] = xe[L:L + W - 1].T
    return y, state_out


def conv_backward(x, weight, bias, cu_seqlens, dy, state_in=None, activation="silu"):
    """Adjoint of conv_forward. Returns dx [T, C], dweight [C, W], dbias [C] and
    dstate_in [N, C, W-1], float64."""
    x, w, dy = _f64(x), _f64(weight), _f64(dy)
    T, C = x.shape
    W = w.shape[1]
    b = np.zeros(C) if bias is None else _f64(bias)
    cu = _bounds(cu_seqlens, T)
    N = cu.size - 1
    dx = np.zeros((T, C))
    dw = np.zeros((C, W))
    db = np.zeros(C)
    dstate = np.zeros((N, C, W - 1))
    for n in range(N):
        xe = _extended(x, cu, n, state_in, W)
        L = cu[n + 1] - cu[n]
        pre = np.tile(b, (L, 1))
        for i in range(W):
            pre += w[:, i][None, :] * xe[i:i + L]
        dpre = dy[cu[n]:cu[n + 1]] * act_grad(pre, activation)
        dxe = np.zeros_like(xe)
        for i in range(W):
            dxe[i:i + L] += w[:, i][None, :] * dpre
            dw[:, i] += (dpre * xe[i:i + L]).sum(axis=0)
        db += dpre.sum(axis=0)
        dstate[n] = dxe[:W - 1].T
        dx[cu[n]:cu[n + 1]] = dxe[W - 1:]
    return dx, dw, db, dstate


def _check_conv_indices(idx, slots):
    active = idx[idx != 0]
    if np.any(active < 0):
        raise ValueError("negative conv state index")
    if np.any(active >= slots):
        raise ValueError("conv state index out of range")
    if np.unique(active).size != active.size:
        raise ValueError("repeated conv state index")


def conv_update(x, weight, bias, state_pool, indices, activation="silu"):
    """One decode token per row. x [N, C]; state_pool [slots, C, W-1].

    Returns (y [N, C], new_pool) in float64; the input pool is not modified.
    """
    x = _f64(x)
    pool = _f64(state_pool).copy()
    idx = np.asarray(indices, dtype=np.int64).reshape(-1)
    _check_conv_indices(idx, pool.shape[0])
    N, C = x.shape
    y = np.zeros((N, C))
    for n in range(N):
        s = idx[n]
        if s == 0:
            continue
        yn, st = conv_forward(x[n:n + 1], weight, bias, [0, 1], pool[s:s + 1], activation)
        y[n] = yn[0]
        pool[s] = st[0]
    return y, pool


def conv_forward_paged(x, weight, bias, cu_seqlens, state_pool, indices,
                       has_initial_state=None, activation="silu"):
    """Forward whose carried states live in a pool [slots, C, W-1].

    Sequence n with a block (index != 0) starts from it when
    has_initial_state[n] is nonzero (None: all resume) and from zero
    otherwise, and its end state replaces the block; index 0 starts from zero
    and writes nothing. Returns (y [T, C], new_pool), float64.
    """
    pool = _f64(state_pool).copy()
    idx = np.asarray(indices, dtype=np.int64).reshape(-1)
    _check_conv_indices(idx, pool.shape[0])
    N = idx.size
    init = np.ones(N, dtype=np.int64) if has_initial_state is None else \
        np.asarray(has_initial_state, dtype=np.int64).reshape(-1)
    start = np.zeros((N,) + pool.shape[1:])
    for n in range(N):
        if idx[n] != 0 and init[n] != 0:
            start[n] = pool[idx[n]]
    y, end = conv_forward(x, weight, bias, cu_seqlens, start, activation)
    for n in range(N):
        if idx[n] != 0:
            pool[idx[n]] = end[n]
    return y, pool
