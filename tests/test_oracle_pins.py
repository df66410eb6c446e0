"""Pins of the CPU oracle against facts it does not compute itself.

Each test ties oracle.recurrence to something independent of it: the chunk
(WY / transition) formulation, closed forms, a textbook reduction, a library
filter, exact brute force, finite differences and the pages' invariants.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
from scipy.signal import lfilter

from oracle import chunked, recurrence as R


def rand_inputs(rng, lens, H, HV, K, V, h0=True, g_scale=1.0):
    T = sum(lens)
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, HV, V))
    g = -g_scale * np.exp(rng.uniform(0, np.log(16), HV))[None] * np.log1p(
        np.exp(rng.standard_normal((T, HV))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, HV))))
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = 0.1 * rng.standard_normal((len(lens), HV, V, K)) if h0 else None
    return q, k, v, g, beta, cu, S0


def rel_err(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- chunk form
@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 64])
def test_chunk_form_equals_recurrence(chunk):
    rng = np.random.default_rng(1 + chunk)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [5, 70, 1, 131], H=2, HV=4, K=8, V=6, g_scale=0.2)
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    oc, hc = chunked.chunked_forward(q, k, v, g, beta, cu, S0, chunk=chunk)
    assert rel_err(oc, o) < 1e-12 and rel_err(hc, hT) < 1e-12


def test_chunk_form_full_head_dim():
    rng = np.random.default_rng(7)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [130, 64], H=1, HV=2, K=128, V=128)
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    oc, hc = chunked.chunked_forward(q, k, v, g, beta, cu, S0, chunk=64)
    assert rel_err(oc, o) < 1e-12 and rel_err(hc, hT) < 1e-12


def test_transition_product_form_equals_recurrence():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [150, 37], H=1, HV=2, K=16, V=8, g_scale=0.1)
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    oc, hc = chunked.chunked_forward(q, k, v, g, beta, cu, S0, chunk=64, use_transition=True)
    assert rel_err(oc, o) < 1e-11 and rel_err(hc, hT) < 1e-11


# ---------------------------------------------------------------- closed forms
def test_beta_zero_is_pure_decay():
    """beta = 0: nothing is written; o_t = exp(sum_{s<=t} g_s) S0 q~_t and hT = exp(sum g) S0."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [40], H=1, HV=1, K=8, V=5)
    beta[:] = 0.0
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    G = np.cumsum(g[:, 0])
    qn = q[:, 0] / np.sqrt((q[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6) * 8 ** -0.5
    expect = np.exp(G)[:, None] * (qn @ S0[0, 0].T)
    assert rel_err(o[:, 0], expect) < 1e-13
    assert rel_err(hT[0, 0], np.exp(G[-1]) * S0[0, 0]) < 1e-13


def test_orthogonal_keys_reduce_to_causal_linear_attention():
    """g = 0, zero state and orthonormal keys: S_{t-1} k_t = 0, so delta_t = beta_t v_t and
    o = tril(Q~ K^T) diag(beta) V, a masked matrix product (causal linear attention)."""
    rng = np.random.default_rng(5)
    T, K, V = 48, 64, 32
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm[:T][:, None, :]                     # orthonormal rows
    q = rng.standard_normal((T, 1, K))
    v = rng.standard_normal((T, 1, V))
    beta = rng.uniform(0.1, 0.9, (T, 1))
    g = np.zeros((T, 1))
    o, _ = R.forward(q, k, v, g, beta, [0, T])
    kn = k[:, 0] / np.sqrt(1 + 1e-6)
    qn = q[:, 0] / np.sqrt((q[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6) * K ** -0.5
    expect = np.tril(qn @ kn.T) @ (beta * v[:, 0])
    assert rel_err(o[:, 0], expect) < 1e-12


def test_scalar_case_is_an_exponential_moving_average():
    """K = V = 1, g = 0, q = k = 1, constant beta: with c = 1/sqrt(1 + 1e-6),
    S_t = (1 - beta c^2) S_{t-1} + beta c v_t, a first-order IIR filter (scipy lfilter)."""
    rng = np.random.default_rng(9)
    T, b = 200, 0.3
    v = rng.standard_normal((T, 1, 1))
    ones = np.ones((T, 1, 1))
    o, hT = R.forward(ones, ones, v, np.zeros((T, 1)), np.full((T, 1), b), [0, T])
    c = 1 / np.sqrt(1 + 1e-6)
    S = lfilter([b * c], [1.0, -(1 - b * c * c)], v[:, 0, 0])
    assert rel_err(o[:, 0, 0], S * c) < 1e-12        # o = S q~, q~ = c (scale = 1)
    assert abs(hT[0, 0, 0, 0] - S[-1]) < 1e-12


def test_forget_all_decay():
    """g = -60: the carried state is wiped each step, o_t = beta_t (k^_t . q~_t) v_t, no NaN."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [64, 3], H=1, HV=1, K=16, V=8)
    g[:] = -60.0
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    kn = R.l2norm(k[:, 0])
    qn = R.l2norm(q[:, 0]) * 16 ** -0.5
    expect = (beta[:, 0] * (kn * qn).sum(-1))[:, None] * v[:, 0]
    assert np.isfinite(o).all() and np.isfinite(hT).all()
    assert rel_err(o[:, 0], expect) < 1e-13
    oc, hc = chunked.chunked_forward(q, k, v, g, beta, cu, S0, chunk=64)
    assert np.isfinite(oc).all() and rel_err(oc, o) < 1e-12


def test_brute_force_matrix_form_exact():
    """T = 4, K = V = 2: the state recurrence evaluated literally as
    S_t = a S_{t-1} (I - beta k k^T) + beta v k^T with full 2x2 matrix products in
    50-digit decimal arithmetic."""
    getcontext().prec = 50
    rng = np.random.default_rng(4)
    T, K, V = 4, 2, 2
    q = np.round(rng.standard_normal((T, 1, K)), 3)
    k = np.round(rng.standard_normal((T, 1, K)), 3)
    v = np.round(rng.standard_normal((T, 1, V)), 3)
    g = np.round(-rng.uniform(0, 1, (T, 1)), 3)
    beta = np.round(rng.uniform(0, 1, (T, 1)), 3)
    S0 = np.round(rng.standard_normal((1, 1, V, K)), 3)
    o, hT = R.forward(q, k, v, g, beta, [0, T], S0)

    D = lambda x: Decimal(repr(float(x)))  # noqa: E731
    eps = Decimal("0.000001")
    S = [[D(S0[0, 0, i, j]) for j in range(K)] for i in range(V)]
    scale = Decimal(1) / Decimal(K).sqrt()
    for t in range(T):
        kk = [D(x) for x in k[t, 0]]
        nk = (sum(x * x for x in kk) + eps).sqrt()
        kk = [x / nk for x in kk]
        qq = [D(x) for x in q[t, 0]]
        nq = (sum(x * x for x in qq) + eps).sqrt()
        qq = [scale * x / nq for x in qq]
        a = D(g[t, 0]).exp()
        b = D(beta[t, 0])
        M = [[(Decimal(1) if i == j else Decimal(0)) - b * kk[i] * kk[j] for j in range(K)]
             for i in range(K)]
        S = [[a * sum(S[r][m] * M[m][c] for m in range(K)) + b * D(v[t, 0, r]) * kk[c]
              for c in range(K)] for r in range(V)]
        ot = [sum(S[r][c] * qq[c] for c in range(K)) for r in range(V)]
        for r in range(V):
            assert abs(float(ot[r]) - o[t, 0, r]) < 1e-14
    for r in range(V):
        for c in range(K):
            assert abs(float(S[r][c]) - hT[0, 0, r, c]) < 1e-14


# ---------------------------------------------------------------- invariants
def test_state_carry_at_the_pages_split_points(contract):
    """One call equals two calls with hT -> h0, at the boundary sweep's prefixes and
    continuations (torchtitan PR #4389)."""
    rng = np.random.default_rng(21)
    pre = contract["continuity_prefixes"]["value"]
    cont = contract["continuity_continuations"]["value"]
    T = max(pre) + max(cont)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [T], H=1, HV=2, K=8, V=4, g_scale=0.05)
    for p in pre:
        for c in cont:
            n = p + c
            o, hT = R.forward(q[:n], k[:n], v[:n], g[:n], beta[:n], [0, n], S0)
            o1, h1 = R.forward(q[:p], k[:p], v[:p], g[:p], beta[:p], [0, p], S0)
            o2, h2 = R.forward(q[p:n], k[p:n], v[p:n], g[p:n], beta[p:n], [0, c], h1)
            assert rel_err(np.concatenate([o1, o2]), o) < 1e-12
            assert rel_err(h2, hT) < 1e-12


def test_a_sequence_alone_equals_it_inside_a_pack():
    rng = np.random.default_rng(8)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [17, 64, 90], H=2, HV=4, K=8, V=8)
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    s0, s1 = cu[1], cu[2]
    o1, h1 = R.forward(q[s0:s1], k[s0:s1], v[s0:s1], g[s0:s1], beta[s0:s1], [0, s1 - s0],
                       S0[1:2])
    assert np.array_equal(o1, o[s0:s1]) and np.array_equal(h1[0], hT[1])


def test_linearity_in_state_and_values():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [33, 20], H=1, HV=2, K=8, V=8)
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    o2, h2 = R.forward(q, k, 2 * v, g, beta, cu, 2 * S0)
    assert np.array_equal(o2, 2 * o) and np.array_equal(h2, 2 * hT)


def test_grouped_heads_equal_repeated_key_heads():
    """Value head hv reads key head hv // (HV/H): the same as repeating q/k per value head
    (FLA's repeat_interleave), and q/k gradients sum over the value heads of a key head."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [20, 9], H=2, HV=4, K=8, V=8)
    qr, kr = np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1)
    o, hT = R.forward(q, k, v, g, beta, cu, S0)
    o2, h2 = R.forward(qr, kr, v, g, beta, cu, S0)
    assert np.array_equal(o, o2) and np.array_equal(hT, h2)
    do = rng.standard_normal(o.shape)
    gr = R.backward(q, k, v, g, beta, cu, do, S0)
    gr2 = R.backward(qr, kr, v, g, beta, cu, do, S0)
    assert rel_err(gr["dq"], gr2["dq"].reshape(-1, 2, 2, 8).sum(2)) < 1e-13
    assert rel_err(gr["dk"], gr2["dk"].reshape(-1, 2, 2, 8).sum(2)) < 1e-13


# ---------------------------------------------------------------- gradients
def test_adjoint_matches_central_finite_differences():
    rng = np.random.default_rng(31)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [3, 5], H=1, HV=2, K=3, V=3, g_scale=0.3)
    wo = rng.standard_normal((8, 2, 3))
    wh = rng.standard_normal((2, 2, 3, 3))

    def loss(q, k, v, g, beta, S0):
        o, hT = R.forward(q, k, v, g, beta, cu, S0)
        return (o * wo).sum() + (hT * wh).sum()

    grads = R.backward(q, k, v, g, beta, cu, wo, S0, dhT=wh, ckpt=2)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="dh0")
    h = 1e-6
    for name, gname in names.items():
        x = args[name]
        num = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            num[i] = (loss(**{**args, name: xp}) - loss(**{**args, name: xm})) / (2 * h)
        assert rel_err(grads[gname], num) < 1e-6, name


def test_dh0_matches_the_reverse_chunk_state_recurrence():
    rng = np.random.default_rng(41)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [100, 64, 7], H=1, HV=2, K=16, V=8, g_scale=0.1)
    do = rng.standard_normal((171, 2, 8))
    dhT = rng.standard_normal((3, 2, 8, 16))
    gr = R.backward(q, k, v, g, beta, cu, do, S0, dhT=dhT)
    dh0 = chunked.chunked_dh0(q, k, v, g, beta, cu, do, dhT=dhT, chunk=64)
    assert rel_err(gr["dh0"], dh0) < 1e-11


def test_l2norm_backward_matches_finite_differences():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 7))
    w = rng.standard_normal((4, 7))
    num = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += 1e-6
        xm[i] -= 1e-6
        num[i] = ((R.l2norm(xp) * w).sum() - (R.l2norm(xm) * w).sum()) / 2e-6
    assert rel_err(R.l2norm_backward(x, w), num) < 1e-8


def test_l2norm_values(contract):
    eps = contract["l2norm_eps"]["value"]
    out = R.l2norm(np.array([[3.0, 4.0]]))
    assert np.allclose(out, np.array([[3.0, 4.0]]) / np.sqrt(25 + eps), rtol=0, atol=1e-16)
    assert np.array_equal(R.l2norm(np.zeros((1, 4))), np.zeros((1, 4)))


# ---------------------------------------------------------------- decode
def test_softplus_threshold_branches(contract):
    th = contract["softplus_threshold"]["value"]
    x = np.array([-30.0, -1.0, 0.0, 19.5, th, th + 1e-3, 50.0])
    sp = R.softplus_thresholded(x)
    assert sp[0] == np.log1p(np.exp(-30.0)) and sp[2] == np.log(2.0)
    assert sp[4] == np.log1p(np.exp(th))          # at the threshold: the log branch
    assert sp[5] == th + 1e-3 and sp[6] == 50.0   # above: identity
    assert abs(np.log1p(np.exp(th)) - th) < 2.1e-9


def test_decode_gating_closed_forms():
    g, beta = R.decode_gating(np.zeros((1, 2)), np.zeros((1, 2)), np.array([0.0, np.log(4.0)]),
                              np.zeros(2))
    assert beta[0, 0] == 0.5 and abs(g[0, 0] + np.log(2.0)) < 1e-16
    assert abs(g[0, 1] + 4 * np.log(2.0)) < 1e-15


def _decode_case(rng, N=6, H=2, HV=4, K=8, V=8, slots=10):
    q = rng.standard_normal((N, H, K))
    k = rng.standard_normal((N, H, K))
    v = rng.standard_normal((N, HV, V))
    a = rng.standard_normal((N, HV))
    b = rng.standard_normal((N, HV))
    A_log = rng.uniform(0, np.log(16), HV)
    dt_bias = rng.standard_normal(HV) * 0.1
    pool = 0.1 * rng.standard_normal((slots, HV, V, K))
    return q, k, v, a, b, A_log, dt_bias, pool


def test_decode_skips_null_and_negative_rows():
    rng = np.random.default_rng(51)
    q, k, v, a, b, A_log, dt_bias, pool = _decode_case(rng)
    idx = np.array([3, 0, 7, -2, 1, 9])
    o, new = R.decode_step(q, k, v, a, b, A_log, dt_bias, pool, idx)
    assert np.array_equal(o[1], np.zeros_like(o[1])) and np.array_equal(o[3], np.zeros_like(o[3]))
    untouched = [s for s in range(10) if s not in (3, 7, 1, 9)]
    assert np.array_equal(new[untouched], pool[untouched])
    assert np.array_equal(new[0], pool[0])


def test_decode_rejects_bad_active_indices():
    rng = np.random.default_rng(52)
    q, k, v, a, b, A_log, dt_bias, pool = _decode_case(rng)
    with pytest.raises(ValueError):
        R.decode_step(q, k, v, a, b, A_log, dt_bias, pool, np.array([3, 0, 7, 3, 1, 9]))
    with pytest.raises(ValueError):
        R.decode_step(q, k, v, a, b, A_log, dt_bias, pool, np.array([3, 0, 7, 10, 1, 9]))
    # repeated null rows are fine
    R.decode_step(q, k, v, a, b, A_log, dt_bias, pool, np.array([0, 0, -1, -1, 1, 9]))


def test_decode_is_one_recurrence_step_with_the_fused_gates():
    rng = np.random.default_rng(53)
    q, k, v, a, b, A_log, dt_bias, pool = _decode_case(rng)
    idx = np.array([3, 0, 7, 2, 1, 9])
    o, new = R.decode_step(q, k, v, a, b, A_log, dt_bias, pool, idx)
    x = a + dt_bias
    g = -np.exp(A_log) * np.where(x > 20, x, np.log1p(np.exp(x)))
    beta = 1 / (1 + np.exp(-b))
    for n in [0, 2, 3, 4, 5]:
        S = pool[idx[n]]
        for hv in range(4):
            kk = k[n, hv // 2] / np.sqrt((k[n, hv // 2] ** 2).sum() + 1e-6)
            qq = q[n, hv // 2] / np.sqrt((q[n, hv // 2] ** 2).sum() + 1e-6) * 8 ** -0.5
            M = np.eye(8) - beta[n, hv] * np.outer(kk, kk)
            Sn = np.exp(g[n, hv]) * S[hv] @ M + beta[n, hv] * np.outer(v[n, hv], kk)
            assert rel_err(new[idx[n], hv], Sn) < 1e-13
            assert rel_err(o[n, hv], Sn @ qq) < 1e-12


def test_decode_steps_equal_the_chunk_forward():
    """T decode steps on one slot reproduce the forward over the same T tokens
    (the pages compare the two paths: RL-Kernel PR #469, 'Decode versus chunked prefill')."""
    rng = np.random.default_rng(54)
    T, H, HV, K, V = 9, 1, 2, 8, 8
    q, k, v = (rng.standard_normal((T, H, K)), rng.standard_normal((T, H, K)),
               rng.standard_normal((T, HV, V)))
    a, b = rng.standard_normal((T, HV)), rng.standard_normal((T, HV))
    A_log, dt_bias = rng.uniform(0, 2, HV), np.zeros(HV)
    pool = 0.1 * rng.standard_normal((3, HV, V, K))
    g, beta = R.decode_gating(a, b, A_log, dt_bias)
    o_ref, hT = R.forward(q, k, v, g, beta, [0, T], pool[2:3])
    cur = pool
    for t in range(T):
        o_t, cur = R.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1],
                                 A_log, dt_bias, cur, np.array([2]))
        assert rel_err(o_t[0], o_ref[t]) < 1e-12
    assert rel_err(cur[2], hT[0]) < 1e-12


# ---------------------------------------------------------------- paged prefill
def _paged_case(rng, lens, H=1, HV=2, K=8, V=8, slots=40):
    q, k, v, g, beta, cu, _ = rand_inputs(rng, lens, H, HV, K, V, h0=False, g_scale=0.05)
    pool = 0.1 * rng.standard_normal((slots, HV, V, K))
    return q, k, v, g, beta, cu, pool


def test_paged_prefix_then_continuation_equals_one_pass():
    """The pages' continuity sweep (torchtitan PR #4389, 'Paged-state continuity':
    prefixes 528/1056/1584 tokens, continuations 1/63/64/65/527): a fresh
    prefill of the prefix into a block, then a resumed prefill of the
    continuation from it, equals one pass over the whole sequence."""
    rng = np.random.default_rng(61)
    cases = [(P, C) for P in (528, 1056, 1584) for C in (1, 63, 64, 65, 527)]
    full = [P + C for P, C in cases]
    q, k, v, g, beta, cu, pool = _paged_case(rng, full)
    o_ref, h_ref = R.forward(q, k, v, g, beta, cu)
    first = np.concatenate([np.arange(cu[i], cu[i] + P) for i, (P, C) in enumerate(cases)])
    second = np.concatenate([np.arange(cu[i] + P, cu[i + 1]) for i, (P, C) in enumerate(cases)])
    idx = rng.permutation(np.arange(1, 40))[:len(cases)]
    sel = lambda x, t: x[t]  # noqa: E731
    cu1 = np.concatenate([[0], np.cumsum([P for P, _ in cases])])
    cu2 = np.concatenate([[0], np.cumsum([C for _, C in cases])])
    o1, pool1 = R.paged_forward(sel(q, first), sel(k, first), sel(v, first), sel(g, first),
                                sel(beta, first), cu1, pool, idx, np.zeros(len(cases)))
    o2, pool2 = R.paged_forward(sel(q, second), sel(k, second), sel(v, second), sel(g, second),
                                sel(beta, second), cu2, pool1, idx, np.ones(len(cases)))
    assert rel_err(o1, o_ref[first]) < 1e-12 and rel_err(o2, o_ref[second]) < 1e-12
    assert rel_err(pool2[idx], h_ref) < 1e-12
    others = np.setdiff1d(np.arange(40), idx)
    assert np.array_equal(pool2[others], pool[others])


def test_paged_fresh_resumed_and_null_sequences():
    rng = np.random.default_rng(62)
    lens = [70, 5, 130, 64, 1]
    q, k, v, g, beta, cu, pool = _paged_case(rng, lens, H=2, HV=4, slots=10)
    idx = np.array([3, 0, 7, -1, 9])
    init = np.array([1, 1, 0, 1, 1])
    o, new = R.paged_forward(q, k, v, g, beta, cu, pool, idx, init)
    for n in range(len(lens)):
        t0, t1 = cu[n], cu[n + 1]
        start = pool[idx[n]:idx[n] + 1] if idx[n] > 0 and init[n] else None
        o_n, h_n = R.forward(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1], [0, t1 - t0],
                             start)
        assert np.array_equal(o[t0:t1], o_n), n
        if idx[n] > 0:
            assert np.array_equal(new[idx[n]], h_n[0]), n
    untouched = [s for s in range(10) if s not in (3, 7, 9)]
    assert np.array_equal(new[untouched], pool[untouched])
    # a fresh sequence does not depend on what its block held
    pool_b = pool.copy()
    pool_b[7] = 5.0
    o_b, new_b = R.paged_forward(q, k, v, g, beta, cu, pool_b, idx, init)
    assert np.array_equal(o_b, o) and np.array_equal(new_b[7], new[7])
    # no flags: every sequence with a block resumes
    o_all, _ = R.paged_forward(q, k, v, g, beta, cu, pool, idx, None)
    o_res, _ = R.paged_forward(q, k, v, g, beta, cu, pool, idx, np.ones(5))
    assert np.array_equal(o_all, o_res)


def test_paged_zero_length_sequences():
    rng = np.random.default_rng(63)
    q, k, v, g, beta, cu, pool = _paged_case(rng, [0, 9, 0], slots=6)
    o, new = R.paged_forward(q, k, v, g, beta, cu, pool, [2, 4, 5], [1, 1, 0])
    assert np.array_equal(new[2], pool[2])            # resumed, no tokens: unchanged
    assert np.array_equal(new[5], np.zeros_like(pool[5]))  # fresh, no tokens: zero state
    assert not np.array_equal(new[4], pool[4])


def test_paged_rejects_bad_active_indices():
    rng = np.random.default_rng(64)
    q, k, v, g, beta, cu, pool = _paged_case(rng, [3, 4], slots=6)
    with pytest.raises(ValueError):
        R.paged_forward(q, k, v, g, beta, cu, pool, [2, 2])
    with pytest.raises(ValueError):
        R.paged_forward(q, k, v, g, beta, cu, pool, [2, 6])
    R.paged_forward(q, k, v, g, beta, cu, pool, [0, 0])


# ---------------------------------------------------------------- transition (CP share)
def test_transition_reproduces_the_end_state_of_any_start_state():
    rng = np.random.default_rng(71)
    q, k, v, g, beta, cu, S0 = rand_inputs(rng, [5, 70, 0, 131], H=2, HV=4, K=8, V=6,
                                           g_scale=0.2)
    M, s = R.transition(q, k, v, g, beta, cu)
    _, hT = R.forward(q, k, v, g, beta, cu, S0)
    assert rel_err(np.einsum("nhvj,nhjk->nhvk", S0, M) + s, hT) < 1e-12
    _, hz = R.forward(q, k, v, g, beta, cu)
    assert np.array_equal(s, hz)
    assert np.array_equal(M[2], np.broadcast_to(np.eye(8), (4, 8, 8)))   # no tokens
    assert np.array_equal(s[2], np.zeros_like(s[2]))


def test_transition_equals_the_chunk_transition_product():
    """The product of the chunk maps e^gamma_L I - K_bwd^T W (the maxtext page,
    gdn_cp_m_scan commit) equals the token product, transposed to the S form."""
    rng = np.random.default_rng(72)
    q, k, v, g, beta, cu, _ = rand_inputs(rng, [150], H=1, HV=2, K=8, V=8, g_scale=0.2)
    M, _ = R.transition(q, k, v, g, beta, cu)
    qt, kh, vv = chunked._normed(q, k, v, 1, 2, None)
    for hv in range(2):
        Mh = np.eye(8)
        for c0 in range(0, 150, 64):
            c1 = min(c0 + 64, 150)
            m = chunked._chunk_terms(qt[c0:c1, hv], kh[c0:c1, hv], vv[c0:c1, hv], g[c0:c1, hv],
                                     beta[c0:c1, hv])
            Mh = (m["gL"] * np.eye(8) - m["Kbwd"].T @ m["W"]) @ Mh
        assert rel_err(Mh.T, M[0, hv]) < 1e-12


def test_transition_of_two_segments_composes():
    rng = np.random.default_rng(73)
    q, k, v, g, beta, cu, _ = rand_inputs(rng, [90], H=1, HV=2, K=6, V=5, g_scale=0.3)
    M, s = R.transition(q, k, v, g, beta, cu)
    a, b = slice(0, 37), slice(37, 90)
    M1, s1 = R.transition(q[a], k[a], v[a], g[a], beta[a], [0, 37])
    M2, s2 = R.transition(q[b], k[b], v[b], g[b], beta[b], [0, 53])
    assert rel_err(M1[0] @ M2[0], M[0]) < 1e-12
    assert rel_err(np.einsum("hvj,hjk->hvk", s1[0], M2[0]) + s2[0], s[0]) < 1e-12


def test_transition_without_writes_is_pure_decay():
    rng = np.random.default_rng(74)
    q, k, v, g, beta, cu, _ = rand_inputs(rng, [40], H=1, HV=3, K=4, V=4)
    M, s = R.transition(q, k, v, g, np.zeros_like(beta), cu)
    for hv in range(3):
        assert rel_err(M[0, hv], np.exp(g[:, hv].sum()) * np.eye(4)) < 1e-12
    assert np.array_equal(s, np.zeros_like(s))
