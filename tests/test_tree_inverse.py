"""The identity the blocked verification kernel solves with, checked in fp64
on the CPU: for a tree, T = (I + A)^-1 with A[n, j] = beta_n D(j->n) (k_n.k_j)
on strict ancestors j of n (TreeWY abstract's system) is nonzero only where j
is on n's root path, and its rows follow
    T[n, e_s] = - sum_{t=1..s} A[n, e_t] T[e_t, e_s]
over n's path e_0 = n, e_1 = parent(n), ...; equally, row n alone solves
x (I + A) = e_n on the path: x_0 = 1, x_s = - sum_{t<s} x_t A[e_t, e_s], where
A[e_t, e_s] is entry s - t of e_t's own row (the node-by-node form the
resident matrix-core path uses).  Then U = T R and
o_n = gamma_n QS_n + sum_s W[n, e_s] R_{e_s} with
    W[n, e_s] = sum_{t<=s} D(e_t->n) (q_n.k_{e_t}) T[e_t, e_s]."""
import numpy as np
import pytest


def _tree(rng, N, forest):
    par = np.full(N, -1)
    for i in range(1, N):
        if not (forest and rng.random() < 0.2):
            par[i] = rng.integers(0, i)
    return par


def _path(par, n):
    p = []
    while n >= 0:
        p.append(n)
        n = par[n]
    return p  # e_0 = n, e_1 = parent, ...


@pytest.mark.parametrize("seed,N,forest", [(0, 12, False), (1, 30, True), (2, 45, False)])
def test_inverse_is_path_supported_and_follows_the_recurrence(seed, N, forest):
    rng = np.random.default_rng(seed)
    par = _tree(rng, N, forest)
    d = 6
    k = rng.standard_normal((N, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((N, d))
    alpha = rng.uniform(0.8, 1.0, N)
    beta = rng.uniform(0.1, 0.9, N)

    def D(j, n):  # product of alpha over the path nodes after j, down to n
        p = _path(par, n)
        return float(np.prod([alpha[e] for e in p[:p.index(j)]]))

    A = np.zeros((N, N))
    on_path = np.zeros((N, N), bool)
    for n in range(N):
        p = _path(par, n)
        on_path[n, p] = True
        for j in p[1:]:
            A[n, j] = beta[n] * D(j, n) * (k[n] @ k[j])
    T = np.linalg.inv(np.eye(N) + A)
    assert np.abs(T[~on_path]).max() < 1e-12          # nonzero only on root paths
    for n in range(N):                                 # the row recurrence
        p = _path(par, n)
        for s in range(1, len(p)):
            rec = -sum(A[n, p[t]] * T[p[t], p[s]] for t in range(1, s + 1))
            assert abs(T[n, p[s]] - rec) < 1e-12
    for n in range(N):                                 # row n alone, node by node
        p = _path(par, n)
        x = [1.0]
        for s in range(1, len(p)):
            # A[e_t, e_s] read as entry s - t of e_t's own path row
            x.append(-sum(x[t] * A[p[t], _path(par, p[t])[s - t]] for t in range(s)))
        assert np.allclose(x, [T[n, e] for e in p], atol=1e-12)
    # outputs through T match a direct solve
    R = rng.standard_normal((N, 4))
    U = np.linalg.solve(np.eye(N) + A, R)
    assert np.allclose(T @ R, U, atol=1e-12)
    for n in range(N):
        p = _path(par, n)
        Pc = [D(e, n) * (q[n] @ k[e]) for e in p]
        direct = sum(Pc[t] * U[p[t]] for t in range(len(p)))
        W = [sum(Pc[t] * T[p[t], p[s]] for t in range(s + 1)) for s in range(len(p))]
        via_w = sum(W[s] * R[p[s]] for s in range(len(p)))
        assert np.allclose(via_w, direct, atol=1e-12)
