"""fp64 CPU oracle for tree speculative verification through a recurrent
linear-attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg call it.  It shares
no code with the GPU path.

What it computes is the plain definition, not the fast method:

* Recurrence (Bole auto-summary, "核心公式" section, first formula): scalar-decay
  linear attention updates a d_k x d_v state as  S_t = lam * S_{t-1} + k_t v_t^T.
* Gated delta rule (TreeWY abstract; the pages name it without printing it, so
  the standard Gated DeltaNet form is read here):
      S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.
* Tree (Bole auto-summary, "具体技术细节示例" worked example; Twig abstract):
  a draft node's state is the recurrence applied along its root-to-node path,
  starting from the root state S_root; nodes with parent -1 hang directly off
  S_root (the example's three branches a/b/c do).
* Output of node n: o_n = S_n^T q_n, read from the state after node n's own
  update.
* Pseudo-value of node n (TreeWY abstract: a small pseudo-value matrix stands in
  for per-node states; the per-token factor reading of the Bole summary's
  reconstruction formula):
      u_n = beta_n (v_n - alpha_n S_parent^T k_n)   (gated delta rule)
      u_n = v_n                                      (scalar decay)
  so that in both modes S_n = alpha_n S_parent + k_n u_n^T.
* Commit (Twig abstract "reconstructs only the accepted state"; Bole summary's
  reconstruction formula and its c3 example): the accepted node's state, got by
  walking its path from S_root one token at a time.

Pins: every function here is checked by tests/test_oracle.py against closed
forms and brute force (see that file).  No function is left "parity unpinned".
"""
from __future__ import annotations

import numpy as np

GDN = 0
SCALAR_DECAY = 1

STATUS_OK = 0
STATUS_BAD_PARENTS = 1
STATUS_BAD_ACCEPTED = 2


# ----------------------------------------------------------------- tree index

def parents_valid(par) -> bool:
    """A tree row is valid when every parent index is -1 or an earlier node."""
    par = np.asarray(par)
    return bool(all(-1 <= int(p) <= i - 1 for i, p in enumerate(par)))


def node_path(par, n):
    """Root-side-first list of the nodes on the path to n, n included."""
    path = []
    j = int(n)
    while j >= 0:
        path.append(j)
        j = int(par[j])
    path.reverse()
    return path


def tree_index(parents):
    """Depth and inclusive-ancestor bitsets of every node.

    parents: [B, N] ints.  Returns depth [B, N] int32 (a node with parent -1 has
    depth 0), anc [B, N, ceil(N/64)] uint64 with bit j%64 of word j//64 set when
    node j lies on the root-to-n path (n itself included), and status [B] int32
    (1 for a row whose parents are not all in [-1, i-1]; that row's depth and
    anc are left zero).
    """
    parents = np.asarray(parents)
    B, N = parents.shape
    W = (N + 63) // 64
    depth = np.zeros((B, N), dtype=np.int32)
    anc = np.zeros((B, N, W), dtype=np.uint64)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if not parents_valid(parents[b]):
            status[b] = STATUS_BAD_PARENTS
            continue
        for n in range(N):
            path = node_path(parents[b], n)
            depth[b, n] = len(path) - 1
            for j in path:
                anc[b, n, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return depth, anc, status


def accepted_paths(parents, accepted):
    """Root-side-first path of each accepted node, padded with -1 to length N.

    Returns path [B, N] int32 and status [B] int32 (1 bad parents, 2 accepted
    index outside [0, N); such rows are all -1).
    """
    parents = np.asarray(parents)
    B, N = parents.shape
    out = np.full((B, N), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if not parents_valid(parents[b]):
            status[b] = STATUS_BAD_PARENTS
            continue
        a = int(accepted[b])
        if not 0 <= a < N:
            status[b] = STATUS_BAD_ACCEPTED
            continue
        p = node_path(parents[b], a)
        out[b, :len(p)] = p
    return out, status


# ---------------------------------------------------------- one token's update

def gdn_step(S, k, v, alpha, beta):
    """Gated delta rule for one token: returns (new state, pseudo-value u).

    S_new = alpha (I - beta k k^T) S + beta k v^T, with (I - beta k k^T) S
    written as S - beta k (k^T S);  u = beta (v - alpha S^T k).
    """
    kS = k @ S                      # k^T S, a d_v row
    S_new = alpha * (S - beta * np.outer(k, kS)) + beta * np.outer(k, v)
    u = beta * (v - alpha * kS)
    return S_new, u


def scalar_step(S, k, v, alpha):
    """Scalar-decay linear attention for one token: S_new = alpha S + k v^T, u = v."""
    return alpha * S + np.outer(k, v), v.copy()


def _step(mode, S, k, v, alpha, beta):
    if mode == GDN:
        return gdn_step(S, k, v, alpha, beta)
    return scalar_step(S, k, v, alpha)


# --------------------------------------------------------------- verification

def verify_head(mode, parents_b, q, k, v, alpha, beta, S_root):
    """All nodes of one (sequence, head).

    parents_b [N]; q, k [N, dk]; v [N, dv]; alpha, beta [N] (beta unused in
    scalar mode); S_root [dk, dv].  Returns o [N, dv], U [N, dv] and the per-node
    states [N, dk, dv], all float64.  Nodes are visited in index order, which is
    topological because every parent precedes its child.
    """
    N = len(parents_b)
    S_root = np.asarray(S_root, dtype=np.float64)
    dk, dv = S_root.shape
    states = np.zeros((N, dk, dv))
    o = np.zeros((N, dv))
    U = np.zeros((N, dv))
    for n in range(N):
        p = int(parents_b[n])
        S_par = S_root if p < 0 else states[p]
        b_n = 0.0 if beta is None else float(beta[n])
        states[n], U[n] = _step(mode, S_par, np.asarray(k[n], np.float64),
                                np.asarray(v[n], np.float64), float(alpha[n]), b_n)
        o[n] = states[n].T @ np.asarray(q[n], np.float64)
    return o, U, states


def verify(mode, parents, q, k, v, alpha, beta, S_root, heads=None, seqs=None):
    """Per-node outputs and pseudo-values of a batch.

    Shapes as the library takes them: q, k [B, N, H, dk]; v [B, N, H, dv];
    alpha, beta [B, N, H]; parents [B, N]; S_root [B, H, dk, dv].
    Returns o [B, N, H, dv], U [B, H, N, dv] (float64) and status [B].
    `seqs`/`heads` restrict the work to those indices (other entries stay 0).
    """
    parents = np.asarray(parents)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((B, N, H, dv))
    U = np.zeros((B, H, N, dv))
    status = np.zeros(B, dtype=np.int32)
    for b in (range(B) if seqs is None else seqs):
        if not parents_valid(parents[b]):
            status[b] = STATUS_BAD_PARENTS
            continue
        for h in (range(H) if heads is None else heads):
            ob, Ub, _ = verify_head(mode, parents[b], q[b, :, h], k[b, :, h], v[b, :, h],
                                    alpha[b, :, h], None if beta is None else beta[b, :, h],
                                    S_root[b, h])
            o[b, :, h] = ob
            U[b, h] = Ub
    return o, U, status


# --------------------------------------------------------------------- commit

def commit_head(mode, parents_b, accepted, k, v, alpha, beta, S_root):
    """State after the accepted node of one (sequence, head), by walking its path."""
    S = np.asarray(S_root, dtype=np.float64).copy()
    for j in node_path(parents_b, accepted):
        b_j = 0.0 if beta is None else float(beta[j])
        S, _ = _step(mode, S, np.asarray(k[j], np.float64), np.asarray(v[j], np.float64),
                     float(alpha[j]), b_j)
    return S


def commit(mode, parents, accepted, k, v, alpha, beta, S_root, heads=None, seqs=None):
    """Committed states [B, H, dk, dv] float64 and status [B] (1 bad parents, 2 bad accepted)."""
    parents = np.asarray(parents)
    B, N, H, dk = k.shape
    dv = v.shape[3]
    out = np.zeros((B, H, dk, dv))
    status = np.zeros(B, dtype=np.int32)
    for b in (range(B) if seqs is None else seqs):
        if not parents_valid(parents[b]):
            status[b] = STATUS_BAD_PARENTS
            continue
        a = int(accepted[b])
        if not 0 <= a < N:
            status[b] = STATUS_BAD_ACCEPTED
            continue
        for h in (range(H) if heads is None else heads):
            out[b, h] = commit_head(mode, parents[b], a, k[b, :, h], v[b, :, h], alpha[b, :, h],
                                    None if beta is None else beta[b, :, h], S_root[b, h])
    return out, status
