"""fp64 CPU oracle for tree-masked full attention (the attention layers of a
hybrid model during tree verification).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg call it.  It shares
no code with the GPU path.

What it computes is the plain definition:

* Model (Twig abstract; Bole abstract): the model interleaves full-attention
  layers, which keep a key/value cache of the committed context, with
  recurrent linear-attention layers; verification runs one forward over every
  node of the draft tree.
* Visibility (read here from the tree semantics the pages give the recurrent
  layers, Bole auto-summary worked example and Twig abstract: a draft node's
  state is the recurrence along its own root-to-node path): draft node n sees
  the committed context (the first prefix_len[b] cache entries) and the draft
  nodes on its root path, itself included, and nothing else.  Nodes with
  parent -1 hang directly off the committed context.
* Attention (the standard scaled-dot-product form; the pages do not print it):
  o = sum_j softmax_j(scale q.k_j) v_j over the visible keys, with grouped
  query heads: query head hq reads key/value head hq // (Hq / Hkv).

Every function here is checked by tests/oracle_pins_attention.py against
closed forms, brute force and invariants; none is left "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .tree_oracle import STATUS_BAD_PARENTS, node_path, parents_valid


def softmax_attend(q, K, V, scale):
    """softmax(scale K q) V for one query: q [D], K [L, D], V [L, Dv] -> [Dv] (fp64).

    The largest score is subtracted before exponentiating (exact in real
    arithmetic, keeps exp finite)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


def visible_keys(b, n, kvh, parents_b, k_cache, v_cache, prefix_len, k_tree, v_tree):
    """Keys and values node n of sequence b sees through key/value head kvh:
    the committed prefix, then its root path (root side first, n last)."""
    P = int(prefix_len[b])
    path = node_path(parents_b, n)
    K = np.concatenate([k_cache[b, kvh, :P], k_tree[b, path, kvh]], axis=0)
    V = np.concatenate([v_cache[b, kvh, :P], v_tree[b, path, kvh]], axis=0)
    return K, V


def tree_attention(parents, q, k_cache, v_cache, prefix_len, k_tree, v_tree, scale,
                   seqs=None, heads=None):
    """Outputs of every draft node through one attention layer.

    parents [B, N]; q [B, N, Hq, D]; k_cache, v_cache [B, Hkv, P_max, D]
    (entries past prefix_len[b] are never read); prefix_len [B];
    k_tree, v_tree [B, N, Hkv, D] (the draft tokens' own keys and values).
    Returns o [B, N, Hq, D] float64 and status [B] (1 for invalid parents; that
    row's outputs stay 0).  `seqs`/`heads` restrict the work (query heads).
    """
    parents = np.asarray(parents)
    B, N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, N, Hq, v_cache.shape[3]))
    status = np.zeros(B, dtype=np.int32)
    for b in (range(B) if seqs is None else seqs):
        if not parents_valid(parents[b]):
            status[b] = STATUS_BAD_PARENTS
            continue
        for n in range(N):
            for hq in (range(Hq) if heads is None else heads):
                K, V = visible_keys(b, n, hq // G, parents[b], k_cache, v_cache, prefix_len,
                                    k_tree, v_tree)
                o[b, n, hq] = softmax_attend(q[b, n, hq], K, V, scale)
    return o, status
