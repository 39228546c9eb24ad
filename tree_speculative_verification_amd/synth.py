"""Seeded synthetic draft trees and layer inputs for tree verification.

This module only draws inputs: tree shapes, accepted nodes, q/k/v, gates and the
root state. It holds none of the verification arithmetic, so the GPU path, the
fp64 checker and the benchmark can all take their inputs from it.

The workloads follow the shapes that the Twig/Bole and TreeWY pages talk
about (hybrid models whose linear-attention layers carry a d_k x d_v state,
draft trees of a few dozen to ~128 nodes, batch-wide verification), plus one
wider tree of the kind the pages say the method makes affordable:

  1  gated delta rule, fp32, B=1 H=1 d=16, the 7-node tree [-1,0,0,1,1,2,3], accepted 6
  2  scalar decay (S = lam*S + k v^T, the page-4 closed form), fp32, B=4 H=8 d=64,
     15-node random tree of depth <= 5, accepted = deepest leaf
  3  gated delta rule, bf16 q/k/v, B=8 H=32 d=128, 8-node chain, accepted = random prefix
  4  gated delta rule, bf16 q/k/v, B=32 H=32 d=128, 64-node random tree
     (depth <= 8, <= 4 children), accepted uniform over nodes
  5  gated delta rule, bf16 q/k/v, B=128 H=64 d=128, 128-node wide tree
     (root fan-out 16, depth <= 10, <= 8 children), accepted uniform over leaves
  6  gated delta rule, bf16 q/k/v, B=16 H=32 d=128, 512-node wide tree
     (root fan-out 32, depth <= 12, <= 8 children), accepted uniform over leaves

Draw order per call is fixed: trees, accepted, q, k, v, alpha (or its log), beta,
S_root, all from one numpy PCG64 generator.  bf16 values are produced by
round-to-nearest-even from fp32 and handed to both sides as the same values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GDN = 0
SCALAR_DECAY = 1
F32 = 0
BF16 = 1


@dataclasses.dataclass
class TreeBatch:
    """Host arrays for one verification call.

    q, k: [B, N, H, dk] float32 (bf16-representable when dtype == BF16)
    v:    [B, N, H, dv] float32 (same)
    alpha, beta: [B, N, H] float32 (beta is None in scalar-decay mode)
    parents: [B, N] int32, parents[b, i] in [-1, i-1]
    accepted: [B] int32
    S_root: [B, H, dk, dv] float32
    """

    cfg: int
    mode: int
    dtype: int
    parents: np.ndarray
    accepted: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: Optional[np.ndarray]
    S_root: np.ndarray

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def N(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def dk(self):
        return self.q.shape[3]

    @property
    def dv(self):
        return self.v.shape[3]

    def select(self, bs, hs) -> "TreeBatch":
        """Sub-batch with sequences `bs` and heads `hs` (lists of indices)."""
        bs = np.asarray(bs)
        hs = np.asarray(hs)
        return TreeBatch(
            cfg=self.cfg, mode=self.mode, dtype=self.dtype,
            parents=self.parents[bs].copy(), accepted=self.accepted[bs].copy(),
            q=self.q[bs][:, :, hs].copy(), k=self.k[bs][:, :, hs].copy(),
            v=self.v[bs][:, :, hs].copy(),
            alpha=self.alpha[bs][:, :, hs].copy(),
            beta=None if self.beta is None else self.beta[bs][:, :, hs].copy(),
            S_root=self.S_root[bs][:, hs].copy())


CONFIGS = {
    1: dict(mode=GDN, dtype=F32, B=1, H=1, N=7, d=16),
    2: dict(mode=SCALAR_DECAY, dtype=F32, B=4, H=8, N=15, d=64),
    3: dict(mode=GDN, dtype=BF16, B=8, H=32, N=8, d=128),
    4: dict(mode=GDN, dtype=BF16, B=32, H=32, N=64, d=128),
    5: dict(mode=GDN, dtype=BF16, B=128, H=64, N=128, d=128),
    6: dict(mode=GDN, dtype=BF16, B=16, H=32, N=512, d=128),
}

CONFIG_NAMES = {
    1: "gdn-f32 B1 H1 N7 d16 fixed tree",
    2: "scalar-decay-f32 B4 H8 N15 d64 random tree depth<=5",
    3: "gdn-bf16 B8 H32 N8 d128 chain",
    4: "gdn-bf16 B32 H32 N64 d128 random tree depth<=8 fanout<=4",
    5: "gdn-bf16 B128 H64 N128 d128 wide tree rootfan16 depth<=10 fanout<=8",
    6: "gdn-bf16 B16 H32 N512 d128 wide tree rootfan32 depth<=12 fanout<=8",
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- tree shapes

def depths_of(parents: np.ndarray) -> np.ndarray:
    """Depth of each node of one topologically ordered tree (parent -1 -> depth 0)."""
    d = np.zeros(len(parents), dtype=np.int64)
    for i, p in enumerate(parents):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def random_tree(rng, N, max_depth, max_children, first_parent=0, fixed_root_children=0):
    """One topologically ordered tree: node 0 is the root (parent -1).

    Nodes 1..fixed_root_children hang off node 0.  Every later node i picks its
    parent uniformly among the nodes j in [first_parent, i) whose depth is below
    max_depth and which have fewer than max_children children.
    """
    par = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int64)
    nchild = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        if i <= fixed_root_children:
            p = 0
        else:
            cand = [j for j in range(first_parent, i)
                    if depth[j] < max_depth and nchild[j] < max_children]
            if not cand:
                raise RuntimeError("no eligible parent; tree limits too tight")
            p = cand[rng.integers(len(cand))]
        par[i] = p
        depth[i] = depth[p] + 1
        nchild[p] += 1
    return par


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _normal(rng, shape, dtype):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(cfg: int, seed: Optional[int] = None, B: Optional[int] = None,
                H: Optional[int] = None) -> TreeBatch:
    """Inputs of workload `cfg` (1..6); `seed` defaults to the workload number.

    B and H may be reduced (the per-sequence draws keep their order, so a
    smaller B gives the first sequences of a bigger one only for the trees and
    accepted nodes, not for the value tensors).
    """
    c = CONFIGS[cfg]
    rng = np.random.default_rng(cfg if seed is None else seed)
    B = c["B"] if B is None else B
    H = c["H"] if H is None else H
    N, d = c["N"], c["d"]

    # trees
    if cfg == 1:
        parents = np.tile(np.array([-1, 0, 0, 1, 1, 2, 3], dtype=np.int32), (B, 1))
    elif cfg == 2:
        parents = np.stack([random_tree(rng, N, max_depth=5, max_children=N) for _ in range(B)])
    elif cfg == 3:
        parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    elif cfg == 4:
        parents = np.stack([random_tree(rng, N, max_depth=8, max_children=4) for _ in range(B)])
    elif cfg == 5:
        parents = np.stack([random_tree(rng, N, max_depth=10, max_children=8, first_parent=1,
                                        fixed_root_children=16) for _ in range(B)])
    else:
        parents = np.stack([random_tree(rng, N, max_depth=12, max_children=8, first_parent=1,
                                        fixed_root_children=32) for _ in range(B)])
    parents = parents.astype(np.int32)

    # accepted nodes
    if cfg == 1:
        accepted = np.full(B, 6, dtype=np.int32)
    elif cfg == 2:
        acc = []
        for b in range(B):
            dep = depths_of(parents[b])
            acc.append(int(np.flatnonzero(dep == dep.max())[0]))  # smallest index among deepest
        accepted = np.array(acc, dtype=np.int32)
    elif cfg == 3:
        accepted = (rng.integers(1, N + 1, size=B) - 1).astype(np.int32)
    elif cfg == 4:
        accepted = rng.integers(0, N, size=B).astype(np.int32)
    else:
        acc = []
        for b in range(B):
            has_child = np.zeros(N, dtype=bool)
            has_child[parents[b][parents[b] >= 0]] = True
            leaves = np.flatnonzero(~has_child)
            acc.append(int(leaves[rng.integers(len(leaves))]))
        accepted = np.array(acc, dtype=np.int32)

    shape_qk = (B, N, H, d)
    q = _normal(rng, shape_qk, np.float32)
    k = _normal(rng, shape_qk, np.float32)
    v = _normal(rng, shape_qk, np.float32)
    if c["mode"] == GDN:
        q = _unit_rows(q)
        k = _unit_rows(k)
    if cfg == 1:
        alpha = rng.uniform(0.9, 1.0, size=(B, N, H)).astype(np.float32)
    elif cfg == 2:
        lam = rng.uniform(0.9, 0.99, size=H).astype(np.float32)
        alpha = np.ascontiguousarray(np.broadcast_to(lam[None, None, :], (B, N, H)))
    else:
        g = rng.uniform(-0.1, 0.0, size=(B, N, H))
        alpha = np.exp(g).astype(np.float32)
    beta = None
    if c["mode"] == GDN:
        beta = rng.uniform(0.0, 1.0, size=(B, N, H)).astype(np.float32)
    S_root = (0.1 * rng.standard_normal(size=(B, H, d, d), dtype=np.float32)).astype(np.float32)

    if c["dtype"] == BF16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)

    return TreeBatch(cfg=cfg, mode=c["mode"], dtype=c["dtype"], parents=parents,
                     accepted=accepted, q=q, k=k, v=v, alpha=alpha, beta=beta, S_root=S_root)


def make_custom(parents, accepted, H, dk, dv, mode=GDN, dtype=F32, seed=0,
                normalize=True, alpha_range=(0.9, 1.0), S_scale=0.1) -> TreeBatch:
    """Inputs for a caller-chosen tree (used by edge-case tests).

    parents: [B, N] int array, accepted: [B] int array.
    """
    parents = np.asarray(parents, dtype=np.int32)
    if parents.ndim == 1:
        parents = parents[None]
    accepted = np.asarray(accepted, dtype=np.int32).reshape(-1)
    B, N = parents.shape
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, N, H, dk), np.float32)
    k = _normal(rng, (B, N, H, dk), np.float32)
    v = _normal(rng, (B, N, H, dv), np.float32)
    if normalize:
        q, k = _unit_rows(q), _unit_rows(k)
    alpha = rng.uniform(alpha_range[0], alpha_range[1], size=(B, N, H)).astype(np.float32)
    beta = rng.uniform(0, 1, size=(B, N, H)).astype(np.float32) if mode == GDN else None
    S_root = (S_scale * rng.standard_normal(size=(B, H, dk, dv), dtype=np.float32)).astype(np.float32)
    if dtype == BF16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return TreeBatch(cfg=0, mode=mode, dtype=dtype, parents=parents, accepted=accepted,
                     q=q, k=k, v=v, alpha=alpha, beta=beta, S_root=S_root)


@dataclasses.dataclass
class AttnBatch:
    """Host arrays for one tree_attention call (bf16-representable float32).

    parents [B, N]; q [B, N, Hq, D]; k_cache, v_cache [B, Hkv, P_max, D];
    prefix_len [B] int32; k_tree, v_tree [B, N, Hkv, D]; scale.
    """

    parents: np.ndarray
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    prefix_len: np.ndarray
    k_tree: np.ndarray
    v_tree: np.ndarray
    scale: float


# The attention workload: the 64-node trees of workload 4 through a
# full-attention layer with grouped query heads and a ragged committed context.
ATTN_CONFIG = dict(B=32, N=64, Hq=32, Hkv=8, D=128, P_max=4096)
ATTN_NAME = ("tree-attention-bf16 B32 N64 Hq32 Hkv8 D128 prefix U[2048,4096] "
             "random tree depth<=8 fanout<=4")


def make_attention_inputs(seed: int = 7, B: Optional[int] = None, N: Optional[int] = None,
                          Hq: Optional[int] = None, Hkv: Optional[int] = None,
                          D: Optional[int] = None, P_max: Optional[int] = None,
                          parents: Optional[np.ndarray] = None,
                          prefix_len: Optional[np.ndarray] = None) -> AttnBatch:
    """Seeded inputs for tree_attention (defaults: the attention workload).

    Draw order: trees (depth <= 8, <= 4 children, as workload 4), prefix
    lengths (uniform in [P_max/2, P_max]), q, k_cache, v_cache, k_tree, v_tree,
    all N(0, 1) rounded to bf16; scale = 1/sqrt(D).
    """
    c = ATTN_CONFIG
    B = c["B"] if B is None else B
    N = c["N"] if N is None else N
    Hq = c["Hq"] if Hq is None else Hq
    Hkv = c["Hkv"] if Hkv is None else Hkv
    D = c["D"] if D is None else D
    P_max = c["P_max"] if P_max is None else P_max
    rng = np.random.default_rng(seed)
    if parents is None:
        parents = np.stack([random_tree(rng, N, max_depth=8, max_children=4) for _ in range(B)])
    parents = np.asarray(parents, dtype=np.int32)
    if prefix_len is None:
        prefix_len = rng.integers(P_max // 2, P_max + 1, size=B)
    prefix_len = np.asarray(prefix_len, dtype=np.int32)

    def g(shape):
        return round_bf16(rng.standard_normal(size=shape, dtype=np.float32))

    q = g((B, N, Hq, D))
    k_cache = g((B, Hkv, P_max, D))
    v_cache = g((B, Hkv, P_max, D))
    k_tree = g((B, N, Hkv, D))
    v_tree = g((B, N, Hkv, D))
    return AttnBatch(parents=parents, q=q, k_cache=k_cache, v_cache=v_cache,
                     prefix_len=prefix_len, k_tree=k_tree, v_tree=v_tree,
                     scale=float(1.0 / np.sqrt(D)))


def attention_to_torch(batch: AttnBatch, device="cuda"):
    """Device tensors of an AttnBatch (bf16 bit-exact copies, int32 indices)."""
    import torch

    def vals(x):
        bits = bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)

    return dict(q=vals(batch.q), k_cache=vals(batch.k_cache), v_cache=vals(batch.v_cache),
                prefix_len=i32(batch.prefix_len), k_tree=vals(batch.k_tree),
                v_tree=vals(batch.v_tree), parents=i32(batch.parents), scale=batch.scale)


def to_torch(batch: TreeBatch, device="cuda"):
    """Copies a batch to `device` as the tensors the library takes.

    q/k/v become float32 or bfloat16 (bit-exact: the host values are already
    bf16-representable); beta is None in scalar-decay mode.
    """
    import torch

    def vals(x):
        if batch.dtype == BF16:
            bits = bf16_bits(x).view(np.int16)
            return torch.from_numpy(bits).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    def f32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)

    return dict(q=vals(batch.q), k=vals(batch.k), v=vals(batch.v), alpha=f32(batch.alpha),
                beta=f32(batch.beta),
                parents=torch.from_numpy(np.ascontiguousarray(batch.parents, np.int32)).to(device),
                accepted=torch.from_numpy(np.ascontiguousarray(batch.accepted, np.int32)).to(device),
                S_root=f32(batch.S_root), mode=batch.mode)
