"""Chunk forms of the gated delta rule in fp64, used only to pin the oracle.

TEST INFRASTRUCTURE ONLY: the tests compare these independent formulations
with the token recurrence of ``recurrence.py``; neither is used by the
product path.

Convention here (the chunk papers' one): per sequence and value head the
state is h = S^T, a K x V matrix. For a chunk of L tokens with start state h:
  gamma_i = g_1 + ... + g_i            (cumulative log-decay inside the chunk)
  A_ij    = beta_i e^(gamma_i - gamma_j) k_i . k_j     for i > j, else 0
  T       = (I + A)^-1                 (the UT / WY transform)
  W       = T diag(beta e^gamma) K,   U = T diag(beta) V
  D       = U - W h                    (the corrected values of the chunk)
  O       = diag(e^gamma) Q h + (tril(e^(gamma_i - gamma_j)) o Q K^T) D
  h_next  = e^gamma_L h + K_bwd^T D,   K_bwd = diag(e^(gamma_L - gamma)) K
The transition form h_next = M h + s with M = e^gamma_L I - K_bwd^T W and
s = K_bwd^T U is the chunk transition written on the maxtext page ("Qwen3.5-
397B RL trainer on 128 v7x", the commit that adds the gdn_cp_m_scan forward
transition product), and the reverse state recurrence
  dh <- e^gamma_L dh + Q_g^T dO - K_bg^T T^T (attn^T dO + K_bwd dh)
with Q_g = diag(e^gamma) Q, K_bg = diag(beta e^gamma) K and
attn = tril(e^(gamma_i - gamma_j)) o Q K^T is the backward form of the same
page's gdn_cp_dh_scan commit. The cake_gdn page (miles PR #3597, "What the
commits add") names the same pipeline: a WY pass, the forward state scan
and the output, and the dh scan in the backward.

Only e^(gamma_i - gamma_j) for i >= j and e^(gamma_i) alone are formed, so a
strong decay underflows to 0 instead of producing 0/0.
"""
import numpy as np
from scipy.linalg import solve_triangular

from .recurrence import l2norm


def _chunk_terms(Qc, Kc, Vc, gc, bc):
    """Per-chunk matrices for one value head. Qc, Kc [L, K]; Vc [L, V]; gc, bc [L]."""
    L = gc.shape[0]
    gam = np.cumsum(gc)
    diff = gam[:, None] - gam[None, :]
    low_incl = np.tril(np.ones((L, L), dtype=bool))
    decay = np.exp(np.where(low_incl, diff, -np.inf))          # tril incl. diagonal
    A = np.tril(bc[:, None] * decay * (Kc @ Kc.T), -1)
    Tm = solve_triangular(np.eye(L) + A, np.eye(L), lower=True, unit_diagonal=True)
    W = Tm @ ((bc * np.exp(gam))[:, None] * Kc)
    U = Tm @ (bc[:, None] * Vc)
    attn = decay * (Qc @ Kc.T)
    Kbwd = np.exp(gam[-1] - gam)[:, None] * Kc
    return dict(gam=gam, Tm=Tm, W=W, U=U, attn=attn, Kbwd=Kbwd,
                Qg=np.exp(gam)[:, None] * Qc, Kbg=(bc * np.exp(gam))[:, None] * Kc,
                gL=np.exp(gam[-1]))


def _normed(q, k, v, H, HV, scale):
    hmap = np.arange(HV) // (HV // H)
    K = q.shape[2]
    if scale is None:
        scale = K ** -0.5
    return scale * l2norm(q)[:, hmap], l2norm(k)[:, hmap], np.asarray(v, np.float64)


def chunked_forward(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, chunk=64,
                    use_transition=False):
    """Chunk-form forward. Same arguments and results as recurrence.forward.

    With ``use_transition`` the state is advanced as h_next = M h + s
    instead of e^gamma_L h + K_bwd^T D.
    """
    T, H, K = np.shape(q)
    HV, V = np.shape(v)[1:]
    qt, kh, v = _normed(q, k, v, H, HV, scale)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.size - 1
    o = np.zeros((T, HV, V))
    hT = np.zeros((N, HV, V, K))
    for n in range(N):
        for hv in range(HV):
            h = np.zeros((K, V)) if h0 is None else np.asarray(h0, np.float64)[n, hv].T.copy()
            for c0 in range(cu[n], cu[n + 1], chunk):
                c1 = min(c0 + chunk, cu[n + 1])
                m = _chunk_terms(qt[c0:c1, hv], kh[c0:c1, hv], v[c0:c1, hv],
                                 g[c0:c1, hv], beta[c0:c1, hv])
                D = m["U"] - m["W"] @ h
                o[c0:c1, hv] = m["Qg"] @ h + m["attn"] @ D
                if use_transition:
                    M = m["gL"] * np.eye(K) - m["Kbwd"].T @ m["W"]
                    s = m["Kbwd"].T @ m["U"]
                    h = M @ h + s
                else:
                    h = m["gL"] * h + m["Kbwd"].T @ D
            hT[n, hv] = h.T
    return o, hT


def chunked_dh0(q, k, v, g, beta, cu_seqlens, do, dhT=None, scale=None, chunk=64):
    """dh0 [N, HV, V, K] from the reverse chunk recurrence of the backward.

    Only the state gradient: the recurrence needs the forward's chunk matrices
    but not its states.
    """
    T, H, K = np.shape(q)
    HV, V = np.shape(v)[1:]
    qt, kh, v = _normed(q, k, v, H, HV, scale)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    do = np.asarray(do, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.size - 1
    dh0 = np.zeros((N, HV, V, K))
    for n in range(N):
        starts = list(range(cu[n], cu[n + 1], chunk))
        for hv in range(HV):
            dh = np.zeros((K, V)) if dhT is None else np.asarray(dhT, np.float64)[n, hv].T.copy()
            for c0 in reversed(starts):
                c1 = min(c0 + chunk, cu[n + 1])
                m = _chunk_terms(qt[c0:c1, hv], kh[c0:c1, hv], v[c0:c1, hv],
                                 g[c0:c1, hv], beta[c0:c1, hv])
                dO = do[c0:c1, hv]
                dh = (m["gL"] * dh + m["Qg"].T @ dO
                      - m["Kbg"].T @ m["Tm"].T @ (m["attn"].T @ dO + m["Kbwd"] @ dh))
            dh0[n, hv] = dh.T
    return dh0
