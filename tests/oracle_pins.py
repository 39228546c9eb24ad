"""Pins that tie the fp64 oracle to something other than itself.

Each pin_* function raises AssertionError when the oracle disagrees with a
closed form, a brute-force computation, an invariant or the page-4 worked
example.  tests/test_oracle.py runs them; tests/test_oracle_mutants.py plants
plausible mistakes in the oracle and checks that some pin catches each one.
"""
import json
import os

import numpy as np

import oracle
from oracle import tree_oracle as T
from wy_reference import wy_head

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _random_tree(rng, N, max_depth=None, forest=False):
    par = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=int)
    for i in range(1, N):
        cand = [j for j in range(i) if max_depth is None or depth[j] < max_depth]
        if forest and rng.random() < 0.2:
            continue
        par[i] = cand[rng.integers(len(cand))]
        depth[i] = depth[par[i]] + 1
    return par


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _head_inputs(rng, N, dk, dv, normalize=True):
    q = rng.standard_normal((N, dk))
    k = rng.standard_normal((N, dk))
    if normalize:
        q, k = _unit(q), _unit(k)
    v = rng.standard_normal((N, dv))
    alpha = rng.uniform(0.8, 1.0, N)
    beta = rng.uniform(0.0, 1.0, N)
    S = 0.3 * rng.standard_normal((dk, dv))
    return q, k, v, alpha, beta, S


# ------------------------------------------------------------------ page 4

def pin_page4_worked_example():
    """Scalar decay on the page-4 three-branch tree: a2 and c3 match the printed closed forms."""
    g = _load("page4_worked_example.json")
    names = g["nodes"]
    par = np.array(g["parents"])
    rng = np.random.default_rng(4)
    N, d = len(names), 5
    lam = 0.93
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    S_root = rng.standard_normal((d, d))
    alpha = np.full(N, lam)
    _, _, states = T.verify_head(T.SCALAR_DECAY, par, q, k, v, alpha, None, S_root)
    for node, form in g["closed_forms"].items():
        want = lam ** form["S_root"] * S_root
        for term, power in form.items():
            if term == "S_root":
                continue
            i = names.index(term)
            want = want + lam ** power * np.outer(k[i], v[i])
        n = names.index(node)
        assert np.allclose(states[n], want, rtol=0, atol=1e-12), node
        got = T.commit_head(T.SCALAR_DECAY, par, n, k, v, alpha, None, S_root)
        assert np.allclose(got, want, rtol=0, atol=1e-12), node
        assert np.allclose(states[n].T @ q[n], want.T @ q[n], rtol=0, atol=1e-12)
    for node, path in g["accepted_branch_path"].items():
        assert T.node_path(par, names.index(node)) == [names.index(x) for x in path]


def pin_scalar_closed_form_random():
    """General scalar-decay closed form on random trees and forests:
    S_n = lam^len(n) S_root + sum_{i on path} lam^(len(n)-len(i)) k_i v_i^T
    (the reading of the page-4 tree formula that its worked examples fix)."""
    rng = np.random.default_rng(11)
    for trial in range(6):
        N = int(rng.integers(1, 14))
        par = _random_tree(rng, N, forest=trial % 2 == 1)
        d = 4
        lam = rng.uniform(0.5, 1.0)
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        S_root = rng.standard_normal((d, d))
        o, U, states = T.verify_head(T.SCALAR_DECAY, par, q, k, v, np.full(N, lam), None, S_root)
        # lengths from a parent-pointer closure computed here, not from the oracle
        length = np.ones(N, dtype=int)
        onpath = np.eye(N, dtype=bool)
        for n in range(N):
            if par[n] >= 0:
                length[n] = length[par[n]] + 1
                onpath[n] |= onpath[par[n]]
        for n in range(N):
            want = lam ** length[n] * S_root
            for i in np.flatnonzero(onpath[n]):
                want = want + lam ** (length[n] - length[i]) * np.outer(k[i], v[i])
            assert np.allclose(states[n], want, rtol=0, atol=1e-11)
            assert np.allclose(o[n], want.T @ q[n], rtol=0, atol=1e-11)
            assert np.array_equal(U[n], v[n])


# ------------------------------------------------------------- tree index

def pin_index_golden():
    g = _load("index_7node.json")
    par = np.array([g["parents"]], dtype=np.int32)
    depth, anc, status = T.tree_index(par)
    assert status[0] == 0
    assert depth[0].tolist() == g["depth"]
    for n, want in enumerate(g["ancestors_inclusive"]):
        bits = int(anc[0, n, 0])
        assert [j for j in range(64) if bits >> j & 1] == want
    path, st = T.accepted_paths(par, np.array([6]))
    assert st[0] == 0
    assert path[0].tolist() == g["path_of_6"] + [-1] * (7 - len(g["path_of_6"]))
    leaves = sorted(set(range(7)) - set(p for p in g["parents"] if p >= 0))
    assert leaves == g["leaves"]


def pin_index_transitive_closure():
    """Ancestor bitsets equal the reflexive-transitive closure of the parent
    relation (boolean matrix powers); depth = popcount - 1."""
    rng = np.random.default_rng(5)
    for N in (1, 2, 7, 40, 64, 65, 100, 128):
        par = _random_tree(rng, N, forest=N % 2 == 0)
        P = np.zeros((N, N), dtype=np.int64)
        for i, p in enumerate(par):
            if p >= 0:
                P[i, p] = 1
        R = np.eye(N, dtype=np.int64)
        M = np.eye(N, dtype=np.int64)
        for _ in range(N):
            M = np.minimum(M @ P, 1)
            R = np.maximum(R, M)
        depth, anc, status = T.tree_index(par[None])
        assert status[0] == 0
        W = (N + 63) // 64
        assert anc.shape == (1, N, W)
        for n in range(N):
            got = [j for j in range(N) if int(anc[0, n, j // 64]) >> (j % 64) & 1]
            assert got == list(np.flatnonzero(R[n])), (N, n)
            assert depth[0, n] == len(got) - 1


def pin_index_bad_rows():
    """Rows with a parent outside [-1, i-1] are flagged, valid rows are not."""
    par = np.array([[-1, 0, 1], [-1, 2, 0], [0, -1, -1], [-1, -2, 0], [-1, 0, 0]], dtype=np.int32)
    _, _, status = T.tree_index(par)
    assert status.tolist() == [0, 1, 1, 1, 0]
    _, st = T.accepted_paths(par, np.array([2, 0, 0, 0, 3]))
    assert st.tolist() == [0, 1, 1, 1, 2]


# ---------------------------------------------------------- gated delta rule

def pin_one_hot_keys():
    """Keys that are unit basis vectors turn the gated delta rule into per-row
    exponential moving averages: row c <- alpha (1 - beta) S[c] + beta v for the
    keyed row c, every other row <- alpha S[r].  Dyadic alpha, beta and small
    integer values make every step exact in fp64, so equality is exact."""
    rng = np.random.default_rng(3)
    N, dk, dv = 9, 4, 3
    par = np.array([-1, 0, 1, 1, 0, 4, -1, 6, 2])
    rows = rng.integers(0, dk, N)
    k = np.eye(dk)[rows]
    q = rng.integers(-2, 3, (N, dk)).astype(float)
    v = rng.integers(-4, 5, (N, dv)).astype(float)
    alpha = rng.choice([0.5, 0.75, 1.0], N)
    beta = rng.choice([0.0, 0.25, 0.5, 1.0], N)
    S_root = rng.integers(-4, 5, (dk, dv)).astype(float)
    o, U, states = T.verify_head(T.GDN, par, q, k, v, alpha, beta, S_root)
    for n in range(N):
        path = []
        j = n
        while j >= 0:
            path.insert(0, j)
            j = par[j]
        S = S_root.copy()
        for j in path:
            prev_row = S[rows[j]].copy()
            S = alpha[j] * S
            S[rows[j]] = alpha[j] * (1 - beta[j]) * prev_row + beta[j] * v[j]
        assert np.array_equal(states[n], S), n
        assert np.array_equal(o[n], S.T @ q[n]), n
        p = par[n]
        Sp = S_root if p < 0 else states[p]
        # u_n = beta (v - alpha * keyed row of the parent state)
        assert np.array_equal(U[n], beta[n] * (v[n] - alpha[n] * Sp[rows[n]])), n


def pin_delta_write():
    """alpha = beta = 1 with unit keys: the state returns exactly v_n for key k_n."""
    rng = np.random.default_rng(8)
    N, d = 12, 6
    par = _random_tree(rng, N)
    q, k, v, _, _, S = _head_inputs(rng, N, d, d)
    _, _, states = T.verify_head(T.GDN, par, q, k, v, np.ones(N), np.ones(N), S)
    for n in range(N):
        assert np.allclose(states[n].T @ k[n], v[n], rtol=0, atol=1e-12)


def pin_beta_zero():
    """beta = 0: pure decay, U is exactly zero."""
    rng = np.random.default_rng(9)
    N, d = 10, 5
    par = _random_tree(rng, N, forest=True)
    q, k, v, alpha, _, S = _head_inputs(rng, N, d, d)
    o, U, states = T.verify_head(T.GDN, par, q, k, v, alpha, np.zeros(N), S)
    assert np.all(U == 0)
    gamma = np.ones(N)
    for n in range(N):
        gamma[n] = alpha[n] * (1.0 if par[n] < 0 else gamma[par[n]])
        assert np.allclose(states[n], gamma[n] * S, rtol=1e-13, atol=0)
        assert np.allclose(o[n], gamma[n] * (S.T @ q[n]), rtol=1e-13, atol=1e-15)


def pin_chain_is_decode():
    """A chain tree gives what a token-by-token decode loop gives."""
    rng = np.random.default_rng(10)
    N, dk, dv = 8, 6, 5
    q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv)
    par = np.arange(-1, N - 1)
    o, U, states = T.verify_head(T.GDN, par, q, k, v, alpha, beta, S_root)
    S = S_root.copy()
    for t in range(N):
        S = alpha[t] * (S - beta[t] * np.outer(k[t], k[t] @ S)) + beta[t] * np.outer(k[t], v[t])
        assert np.allclose(states[t], S, rtol=0, atol=1e-13)
        assert np.allclose(o[t], S.T @ q[t], rtol=0, atol=1e-13)


def pin_union_of_chains():
    """Brute force on small trees: decode each root-to-leaf path as its own
    chain; every node gets the same o, u and state on every path through it."""
    rng = np.random.default_rng(12)
    for mode in (T.GDN, T.SCALAR_DECAY):
        N, dk, dv = 11, 4, 3
        par = _random_tree(rng, N, forest=True)
        q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv)
        o, U, states = T.verify_head(mode, par, q, k, v, alpha, beta, S_root)
        children = {p for p in par if p >= 0}
        for leaf in [n for n in range(N) if n not in children]:
            path = []
            j = leaf
            while j >= 0:
                path.insert(0, j)
                j = par[j]
            L = len(path)
            oc, Uc, Sc = T.verify_head(mode, np.arange(-1, L - 1), q[path], k[path], v[path],
                                       alpha[path], beta[path], S_root)
            for pos, n in enumerate(path):
                assert np.array_equal(oc[pos], o[n])
                assert np.array_equal(Uc[pos], U[n])
                assert np.array_equal(Sc[pos], states[n])


def pin_relabel_invariance():
    """Another topological numbering of the same tree permutes the results and
    changes no value (each node only sees its own path)."""
    rng = np.random.default_rng(13)
    N, dk, dv = 12, 5, 4
    par = _random_tree(rng, N, forest=True)
    q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv)
    o, U, states = T.verify_head(T.GDN, par, q, k, v, alpha, beta, S_root)
    # random topological order: repeatedly pick a random node whose parent is placed
    placed, order = set(), []
    while len(order) < N:
        ready = [n for n in range(N) if n not in placed and (par[n] < 0 or par[n] in placed)]
        n = ready[rng.integers(len(ready))]
        order.append(n)
        placed.add(n)
    new_of = {old: i for i, old in enumerate(order)}
    par2 = np.array([-1 if par[old] < 0 else new_of[par[old]] for old in order])
    o2, U2, s2 = T.verify_head(T.GDN, par2, q[order], k[order], v[order], alpha[order],
                               beta[order], S_root)
    assert np.array_equal(o2, o[order])
    assert np.array_equal(U2, U[order])
    assert np.array_equal(s2, states[order])


def pin_commit_consistency():
    """The committed state is the accepted node's verified state; its read-out is o_a."""
    rng = np.random.default_rng(14)
    N, dk, dv = 9, 5, 6
    par = _random_tree(rng, N)
    q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv)
    o, U, states = T.verify_head(T.GDN, par, q, k, v, alpha, beta, S_root)
    for a in range(N):
        S = T.commit_head(T.GDN, par, a, k, v, alpha, beta, S_root)
        assert np.allclose(S, states[a], rtol=0, atol=1e-13)
        assert np.allclose(S.T @ q[a], o[a], rtol=0, atol=1e-13)


def pin_pseudo_value_identity():
    """Every node's state is its parent's state decayed plus the rank-1 term k_n u_n^T."""
    rng = np.random.default_rng(15)
    for mode in (T.GDN, T.SCALAR_DECAY):
        N, dk, dv = 10, 5, 4
        par = _random_tree(rng, N, forest=True)
        q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv)
        _, U, states = T.verify_head(mode, par, q, k, v, alpha, beta, S_root)
        for n in range(N):
            Sp = S_root if par[n] < 0 else states[par[n]]
            assert np.allclose(states[n], alpha[n] * Sp + np.outer(k[n], U[n]), rtol=0, atol=1e-13)


def pin_wy_derivation():
    """Tree WY form solved with LAPACK's triangular solve equals the token walk."""
    rng = np.random.default_rng(16)
    for mode in (T.GDN, T.SCALAR_DECAY):
        for trial in range(4):
            N = int(rng.integers(2, 30))
            par = _random_tree(rng, N, forest=trial == 3)
            dk, dv = 8, 6
            q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv, normalize=mode == T.GDN)
            o, U, states = T.verify_head(mode, par, q, k, v, alpha, beta, S_root)
            o2, U2, s2 = wy_head(mode, par, q, k, v, alpha, beta, S_root)
            scale = max(1.0, np.abs(o).max())
            assert np.abs(o - o2).max() <= 1e-11 * scale
            assert np.abs(U - U2).max() <= 1e-11 * max(1.0, np.abs(U).max())
            assert np.abs(states - s2).max() <= 1e-11 * max(1.0, np.abs(states).max())


def pin_zero_state_single_node():
    """From a zero root state one token gives S = beta k v^T and o = beta (q.k) v."""
    rng = np.random.default_rng(17)
    dk, dv = 7, 5
    q, k, v, alpha, beta, _ = _head_inputs(rng, 1, dk, dv)
    o, U, states = T.verify_head(T.GDN, np.array([-1]), q, k, v, alpha, beta, np.zeros((dk, dv)))
    assert np.allclose(states[0], beta[0] * np.outer(k[0], v[0]), rtol=0, atol=1e-15)
    assert np.allclose(o[0], beta[0] * (q[0] @ k[0]) * v[0], rtol=0, atol=1e-15)
    assert np.allclose(U[0], beta[0] * v[0], rtol=0, atol=1e-15)


def pin_linearity():
    """Scaling S_root and V together scales o, U and the committed state."""
    rng = np.random.default_rng(18)
    N, dk, dv = 9, 4, 4
    par = _random_tree(rng, N)
    q, k, v, alpha, beta, S_root = _head_inputs(rng, N, dk, dv)
    o, U, states = T.verify_head(T.GDN, par, q, k, v, alpha, beta, S_root)
    c = -2.5
    o2, U2, s2 = T.verify_head(T.GDN, par, q, k, c * v, alpha, beta, c * S_root)
    assert np.allclose(o2, c * o, rtol=1e-13, atol=1e-14)
    assert np.allclose(U2, c * U, rtol=1e-13, atol=1e-14)
    assert np.allclose(s2, c * states, rtol=1e-13, atol=1e-14)


def pin_batched_matches_heads():
    """The batched entry points lay out each (sequence, head) as the per-head ones."""
    rng = np.random.default_rng(19)
    B, N, H, dk, dv = 2, 6, 3, 4, 5
    par = np.stack([_random_tree(rng, N) for _ in range(B)])
    q = rng.standard_normal((B, N, H, dk))
    k = _unit(rng.standard_normal((B, N, H, dk)))
    v = rng.standard_normal((B, N, H, dv))
    alpha = rng.uniform(0.8, 1, (B, N, H))
    beta = rng.uniform(0, 1, (B, N, H))
    S = rng.standard_normal((B, H, dk, dv))
    acc = np.array([N - 1, 2])
    o, U, st = T.verify(T.GDN, par, q, k, v, alpha, beta, S)
    Sn, st2 = T.commit(T.GDN, par, acc, k, v, alpha, beta, S)
    assert st.tolist() == [0, 0] and st2.tolist() == [0, 0]
    for b in range(B):
        for h in range(H):
            ob, Ub, states = T.verify_head(T.GDN, par[b], q[b, :, h], k[b, :, h], v[b, :, h],
                                           alpha[b, :, h], beta[b, :, h], S[b, h])
            assert np.array_equal(o[b, :, h], ob)
            assert np.array_equal(U[b, h], Ub)
            assert np.allclose(Sn[b, h], states[acc[b]], rtol=0, atol=1e-13)


ALL_PINS = [pin_page4_worked_example, pin_scalar_closed_form_random, pin_index_golden,
            pin_index_transitive_closure, pin_index_bad_rows, pin_one_hot_keys, pin_delta_write,
            pin_beta_zero, pin_chain_is_decode, pin_union_of_chains, pin_relabel_invariance,
            pin_commit_consistency, pin_pseudo_value_identity, pin_wy_derivation,
            pin_zero_state_single_node, pin_linearity, pin_batched_matches_heads]
