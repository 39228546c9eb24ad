"""Pins that tie the tree-attention oracle to something other than itself.

Each pin_* raises AssertionError when oracle.tree_attention disagrees with a
closed form, an independent matrix formulation or an invariant.
tests/test_oracle_attention.py runs them and plants plausible mistakes in the
oracle to check that some pin catches each one.
"""
import numpy as np

from oracle import tree_attention as A


def _tree(rng, N, forest=False, max_depth=None):
    par = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=int)
    for i in range(1, N):
        if forest and rng.random() < 0.25:
            continue
        cand = [j for j in range(i) if max_depth is None or depth[j] < max_depth]
        par[i] = cand[rng.integers(len(cand))]
        depth[i] = depth[par[i]] + 1
    return par


def _inputs(rng, B, N, Hq, Hkv, D, P_max, forest=False):
    par = np.stack([_tree(rng, N, forest=forest) for _ in range(B)])
    q = rng.standard_normal((B, N, Hq, D))
    kc = rng.standard_normal((B, Hkv, P_max, D))
    vc = rng.standard_normal((B, Hkv, P_max, D))
    kt = rng.standard_normal((B, N, Hkv, D))
    vt = rng.standard_normal((B, N, Hkv, D))
    plen = rng.integers(0, P_max + 1, size=B)
    return par, q, kc, vc, plen, kt, vt


def _closure(par):
    """Inclusive ancestor matrix M[n, j] = (j on n's root path), by boolean
    matrix powers of the parent relation (no path walking)."""
    N = len(par)
    Pm = np.zeros((N, N), dtype=bool)
    for i, p in enumerate(par):
        if p >= 0:
            Pm[i, p] = True
    M = np.eye(N, dtype=bool)
    step = Pm.copy()
    for _ in range(N):
        M |= step
        step = (step.astype(int) @ Pm.astype(int)) > 0
    return M


def _matrix_attention(par, q, kc, vc, plen, kt, vt, scale):
    """Masked softmax attention in matrix form over all keys at once, with the
    key/value heads repeated for the query heads."""
    B, N, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, N, Hq, vc.shape[3]))
    for b in range(B):
        M = _closure(par[b])
        P = int(plen[b])
        for hq in range(Hq):
            kv = hq // G
            Kall = np.concatenate([kc[b, kv, :P], kt[b, :, kv]], axis=0)   # [P + N, D]
            Vall = np.concatenate([vc[b, kv, :P], vt[b, :, kv]], axis=0)
            S = scale * q[b, :, hq] @ Kall.T                                 # [N, P + N]
            mask = np.concatenate([np.ones((N, P), bool), M], axis=1)
            S = np.where(mask, S, -np.inf)
            W = np.exp(S - S.max(axis=1, keepdims=True))
            W /= W.sum(axis=1, keepdims=True)
            o[b, :, hq] = W @ Vall
    return o


def pin_attn_matrix_form():
    """Random forests, grouped heads, ragged prefixes (some empty): equal to the
    matrix form with a transitive-closure mask."""
    rng = np.random.default_rng(1)
    args = _inputs(rng, B=3, N=9, Hq=4, Hkv=2, D=5, P_max=6, forest=True)
    args[4][0] = 0
    o, st = A.tree_attention(*args, scale=0.7)
    assert not st.any()
    ref = _matrix_attention(*args, scale=0.7)
    assert np.allclose(o, ref, rtol=0, atol=1e-12), np.abs(o - ref).max()


def pin_attn_lone_roots():
    """No prefix and every node a root: each node sees only its own key, so its
    output is its own value, whatever the query."""
    rng = np.random.default_rng(2)
    B, N, Hq, Hkv, D = 2, 5, 2, 1, 4
    par = np.full((B, N), -1, np.int32)
    _, q, kc, vc, _, kt, vt = _inputs(rng, B, N, Hq, Hkv, D, 3)
    o, _ = A.tree_attention(par, q, kc, vc, np.zeros(B, int), kt, vt, scale=1.3)
    for hq in range(Hq):
        assert np.allclose(o[:, :, hq], vt[:, :, 0], rtol=0, atol=1e-14)


def pin_attn_zero_query_is_mean():
    """q = 0: every visible key gets the same weight, so o is the mean of the
    visible values (prefix entries plus path nodes, counted by hand)."""
    rng = np.random.default_rng(3)
    par = np.array([[-1, 0, 0, 1, 3, -1, 5]], np.int32)
    _, _, kc, vc, _, kt, vt = _inputs(rng, 1, 7, 1, 1, 3, 4)
    q = np.zeros((1, 7, 1, 3))
    o, _ = A.tree_attention(par, q, kc, vc, np.array([2]), kt, vt, scale=1.0)
    seen = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 1, 3], 4: [0, 1, 3, 4], 5: [5], 6: [5, 6]}
    for n, path in seen.items():
        mean = (vc[0, 0, :2].sum(axis=0) + vt[0, path, 0].sum(axis=0)) / (2 + len(path))
        assert np.allclose(o[0, n, 0], mean, rtol=0, atol=1e-14), n


def pin_attn_chain_is_causal():
    """A chain with no prefix is ordinary causal attention over the chain."""
    rng = np.random.default_rng(4)
    N, D = 6, 4
    par = np.arange(-1, N - 1, dtype=np.int32)[None]
    _, q, kc, vc, _, kt, vt = _inputs(rng, 1, N, 1, 1, D, 2)
    o, _ = A.tree_attention(par, q, kc, vc, np.array([0]), kt, vt, scale=0.5)
    S = 0.5 * q[0, :, 0] @ kt[0, :, 0].T
    S[np.triu_indices(N, 1)] = -np.inf
    W = np.exp(S - S.max(axis=1, keepdims=True))
    W /= W.sum(axis=1, keepdims=True)
    assert np.allclose(o[0, :, 0], W @ vt[0, :, 0], rtol=0, atol=1e-13)


def pin_attn_one_hot_selects():
    """Orthogonal keys and a query far along one of them: the output tends to
    that key's value (weights of the others fall as exp(-scale * gap))."""
    rng = np.random.default_rng(5)
    D = 6
    par = np.array([[-1, 0, 1]], np.int32)
    kc = np.eye(D)[None, None, :3]                # prefix keys e0, e1, e2
    vc = rng.standard_normal((1, 1, 3, D))
    kt = np.eye(D)[None, 3:6, None]               # tree keys e3, e4, e5
    vt = rng.standard_normal((1, 3, 1, D))
    q = np.zeros((1, 3, 1, D))
    q[0, 2, 0, 1] = 1.0                           # node 2 points at prefix key e1
    o, _ = A.tree_attention(par, q, kc, vc, np.array([3]), kt, vt, scale=60.0)
    assert np.allclose(o[0, 2, 0], vc[0, 0, 1], rtol=0, atol=1e-20)


def pin_attn_score_shift():
    """Adding one vector u with q.u = c to every key shifts every score by
    scale * c, which softmax ignores."""
    rng = np.random.default_rng(6)
    args = list(_inputs(rng, B=2, N=5, Hq=2, Hkv=1, D=4, P_max=3))
    par, q = args[0], args[1]
    q[..., 0] = 0.0                                # every query orthogonal to e0
    u = np.zeros(4)
    u[0] = 5.0
    o1, _ = A.tree_attention(*args, scale=0.8)
    args2 = list(args)
    args2[2] = args[2] + u
    args2[5] = args[5] + u
    o2, _ = A.tree_attention(*args2, scale=0.8)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)


def pin_attn_grouped_heads():
    """Grouped query heads equal plain multi-head attention with each key/value
    head repeated for its group."""
    rng = np.random.default_rng(7)
    par, q, kc, vc, plen, kt, vt = _inputs(rng, B=2, N=6, Hq=6, Hkv=2, D=3, P_max=4)
    o1, _ = A.tree_attention(par, q, kc, vc, plen, kt, vt, scale=1.1)
    rep = lambda x, ax: np.repeat(x, 3, axis=ax)  # noqa: E731
    o2, _ = A.tree_attention(par, q, rep(kc, 1), rep(vc, 1), plen, rep(kt, 2), rep(vt, 2), scale=1.1)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14)
    # and the group of query head 5 is key/value head 1, not 5 % 2
    K, V = A.visible_keys(0, 3, 1, par[0], kc, vc, plen, kt, vt)
    assert np.allclose(o1[0, 3, 5], A.softmax_attend(q[0, 3, 5], K, V, 1.1), rtol=0, atol=1e-14)


def pin_attn_bad_parents():
    rng = np.random.default_rng(8)
    par, q, kc, vc, plen, kt, vt = _inputs(rng, B=2, N=4, Hq=1, Hkv=1, D=2, P_max=2)
    par[1, 2] = 3
    o, st = A.tree_attention(par, q, kc, vc, plen, kt, vt, scale=1.0)
    assert st.tolist() == [0, 1]
    assert not o[1].any() and o[0].any()


ALL_PINS = [pin_attn_matrix_form, pin_attn_lone_roots, pin_attn_zero_query_is_mean,
            pin_attn_chain_is_causal, pin_attn_one_hot_selects, pin_attn_score_shift,
            pin_attn_grouped_heads, pin_attn_bad_parents]
