"""Tree-structured WY form of the gated delta rule, fp64, with a LAPACK triangular solve.

Used only as an independent check of the oracle (the oracle walks the
recurrence token by token; this module never does).  Derivation, for one
(sequence, head), with anc*(n) the root-to-n path including n and anc(n) the
same path without n:

  gamma_n = prod_{j in anc*(n)} alpha_j
  S_n     = gamma_n S_root + sum_{j in anc*(n)} (gamma_n/gamma_j) k_j u_j^T        (T1)
  o_n     = gamma_n S_root^T q_n + sum_{j in anc*(n)} (gamma_n/gamma_j)(q_n.k_j) u_j   (T2)
  (I + A) U = diag(beta) (V - diag(gamma) K S_root),
  A[n, j] = beta_n (gamma_n/gamma_j)(k_n.k_j) for j in anc(n), else 0                (T3)

TreeWY's abstract describes exactly this shape: one triangular solve gives every
draft node's output, and the accepted state is rebuilt from a small
pseudo-value matrix U.  In scalar-decay mode A = 0 and U = V.
"""
import numpy as np
import scipy.linalg


def _ancestors(par):
    N = len(par)
    anc = np.zeros((N, N), dtype=bool)        # anc[n, j]: j on the root-to-n path, n included
    for n in range(N):
        anc[n, n] = True
        if par[n] >= 0:
            anc[n] |= anc[par[n]]
    return anc


def wy_head(mode, par, q, k, v, alpha, beta, S_root):
    """o [N, dv], U [N, dv] and per-node states [N, dk, dv] of one (sequence, head)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S_root = np.asarray(S_root, np.float64)
    alpha = np.asarray(alpha, np.float64)
    N = len(par)
    anc = _ancestors(par)
    loga = np.log(alpha)
    g = anc.astype(np.float64) @ loga                 # g_n = sum of log alpha over anc*(n)
    gamma = np.exp(g)
    decay = np.exp(g[:, None] - g[None, :]) * anc     # gamma_n / gamma_j on anc*(n)
    strict = anc & ~np.eye(N, dtype=bool)
    if mode == 0:
        beta = np.asarray(beta, np.float64)
        A = beta[:, None] * decay * (k @ k.T) * strict
        rhs = beta[:, None] * (v - gamma[:, None] * (k @ S_root))
        U = scipy.linalg.solve_triangular(np.eye(N) + A, rhs, lower=True, unit_diagonal=True)
    else:
        U = v.copy()
    P = decay * (q @ k.T)
    o = gamma[:, None] * (q @ S_root) + P @ U
    states = gamma[:, None, None] * S_root[None] + np.einsum("nj,jr,jc->nrc", decay, k, U)
    return o, U, states
