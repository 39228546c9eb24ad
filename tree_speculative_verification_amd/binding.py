"""ctypes binding of libtreeverify.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; torch is used
here only to allocate device memory and to name the current HIP stream.
Importing this module loads the library and raises if it has not been built
(`python -m tree_speculative_verification_amd.build`); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtreeverify.so")

TV_F32, TV_BF16 = 0, 1
TV_GDN, TV_SCALAR_DECAY = 0, 1
TV_ALGO_AUTO, TV_ALGO_LEVEL, TV_ALGO_MFMA, TV_ALGO_BLOCKED = 0, 1, 2, 3
TV_MAX_NODES = 512
TV_MAX_NODES_SNAPSHOT = 128

SYMBOLS = ["tree_verify", "tree_verify_algo", "tree_commit", "tree_index", "tree_verify_snapshot",
           "tree_commit_snapshot", "tree_commit_verify", "tree_attention", "tv_status_string",
           "tv_version"]


class TreeVerifyError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what} returned {code}: {status_string(code)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m tree_speculative_verification_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.tree_verify.argtypes = [I] * 7 + [P] * 10 + [P]
    lib.tree_verify.restype = I
    lib.tree_verify_algo.argtypes = [I] * 7 + [P] * 10 + [I, P]
    lib.tree_verify_algo.restype = I
    lib.tree_commit.argtypes = [I] * 6 + [P] * 9 + [P]
    lib.tree_commit.restype = I
    lib.tree_index.argtypes = [I, I, P, P, P, P, P]
    lib.tree_index.restype = I
    lib.tree_verify_snapshot.argtypes = [I] * 7 + [P] * 10 + [P]
    lib.tree_verify_snapshot.restype = I
    lib.tree_commit_snapshot.argtypes = [I] * 5 + [P] * 6 + [P]
    lib.tree_commit_snapshot.restype = I
    lib.tree_commit_verify.argtypes = [I] * 8 + [P] * 9 + [P] * 9 + [P]
    lib.tree_commit_verify.restype = I
    lib.tree_attention.argtypes = [I] * 7 + [P] * 7 + [ctypes.c_float] + [P] * 3
    lib.tree_attention.restype = I
    lib.tv_status_string.argtypes = [I]
    lib.tv_status_string.restype = ctypes.c_char_p
    lib.tv_version.argtypes = []
    lib.tv_version.restype = I
    return lib


LIB = _load()


def status_string(code: int) -> str:
    return LIB.tv_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TV_F32
    if t.dtype == torch.bfloat16:
        return TV_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def verify(q, k, v, alpha, beta, parents, S_root, mode=TV_GDN, algo=TV_ALGO_AUTO,
           o=None, U=None, status=None, stream=None):
    """Per-node outputs o [B,N,H,dv] (q's dtype), pseudo-values U [B,H,N,dv] f32, status [B] i32."""
    B, N, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    dt = q.dtype
    _check(q, "q", (B, N, H, dk), dt, dev)
    _check(k, "k", (B, N, H, dk), dt, dev)
    _check(v, "v", (B, N, H, dv), dt, dev)
    _check(alpha, "alpha", (B, N, H), torch.float32, dev)
    if mode == TV_GDN or beta is not None:
        _check(beta, "beta", (B, N, H), torch.float32, dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    _check(S_root, "S_root", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, N, H, dv), dtype=dt, device=dev)
    if U is None:
        U = torch.empty((B, H, N, dv), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(o, "o", (B, N, H, dv), dt, dev)
    _check(U, "U", (B, H, N, dv), torch.float32, dev)
    _check(status, "status", (B,), torch.int32, dev)
    rc = LIB.tree_verify_algo(B, H, N, dk, dv, _dtype_code(q), mode, _ptr(q), _ptr(k), _ptr(v),
                              _ptr(alpha), _ptr(beta), _ptr(parents), _ptr(S_root), _ptr(o),
                              _ptr(U), _ptr(status), algo, _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_verify")
    return o, U, status


def commit(k, alpha, U, parents, accepted, S_root, S_out=None, path_out=None, status=None,
           inplace=False, stream=None):
    """Committed state S_out [B,H,dk,dv] f32, accepted path [B,N] i32, status [B] i32."""
    B, N, H, dk = k.shape
    dv = U.shape[3]
    dev = k.device
    _check(k, "k", (B, N, H, dk), k.dtype, dev)
    _check(alpha, "alpha", (B, N, H), torch.float32, dev)
    _check(U, "U", (B, H, N, dv), torch.float32, dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    _check(accepted, "accepted", (B,), torch.int32, dev)
    _check(S_root, "S_root", (B, H, dk, dv), torch.float32, dev)
    if S_out is None:
        S_out = S_root if inplace else torch.empty_like(S_root)
    if path_out is None:
        path_out = torch.empty((B, N), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(S_out, "S_out", (B, H, dk, dv), torch.float32, dev)
    _check(path_out, "path_out", (B, N), torch.int32, dev)
    _check(status, "status", (B,), torch.int32, dev)
    rc = LIB.tree_commit(B, H, N, dk, dv, _dtype_code(k), _ptr(k), _ptr(alpha), _ptr(U),
                         _ptr(parents), _ptr(accepted), _ptr(S_root), _ptr(S_out),
                         _ptr(path_out), _ptr(status), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_commit")
    return S_out, path_out, status


def index(parents, stream=None):
    """depth [B,N] i32, ancestor bitsets [B,N,ceil(N/64)] (uint64 bits in an int64 tensor), status."""
    B, N = parents.shape
    dev = parents.device
    _check(parents, "parents", (B, N), torch.int32, dev)
    W = (N + 63) // 64
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    anc = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = LIB.tree_index(B, N, _ptr(parents), _ptr(depth), _ptr(anc), _ptr(status), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_index")
    return depth, anc, status


def verify_snapshot(q, k, v, alpha, beta, parents, S_root, mode=TV_GDN, snapshots=None, o=None,
                    status=None, stream=None):
    """Per-node-snapshot baseline: o [B,N,H,dv], snapshots [B,H,N,dk,dv] f32, status [B]."""
    B, N, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    dt = q.dtype
    _check(q, "q", (B, N, H, dk), dt, dev)
    _check(k, "k", (B, N, H, dk), dt, dev)
    _check(v, "v", (B, N, H, dv), dt, dev)
    _check(alpha, "alpha", (B, N, H), torch.float32, dev)
    if mode == TV_GDN or beta is not None:
        _check(beta, "beta", (B, N, H), torch.float32, dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    _check(S_root, "S_root", (B, H, dk, dv), torch.float32, dev)
    if snapshots is None:
        snapshots = torch.empty((B, H, N, dk, dv), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((B, N, H, dv), dtype=dt, device=dev)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(snapshots, "snapshots", (B, H, N, dk, dv), torch.float32, dev)
    _check(o, "o", (B, N, H, dv), dt, dev)
    _check(status, "status", (B,), torch.int32, dev)
    rc = LIB.tree_verify_snapshot(B, H, N, dk, dv, _dtype_code(q), mode, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(alpha), _ptr(beta), _ptr(parents), _ptr(S_root),
                                  _ptr(snapshots), _ptr(o), _ptr(status), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_verify_snapshot")
    return o, snapshots, status


def commit_snapshot(snapshots, parents, accepted, S_out=None, path_out=None, status=None,
                    stream=None):
    """The baseline's commit: S_out [B,H,dk,dv] = the accepted node's snapshot; path, status."""
    B, H, N, dk, dv = snapshots.shape
    dev = snapshots.device
    _check(snapshots, "snapshots", (B, H, N, dk, dv), torch.float32, dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    _check(accepted, "accepted", (B,), torch.int32, dev)
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if path_out is None:
        path_out = torch.empty((B, N), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(S_out, "S_out", (B, H, dk, dv), torch.float32, dev)
    _check(path_out, "path_out", (B, N), torch.int32, dev)
    _check(status, "status", (B,), torch.int32, dev)
    rc = LIB.tree_commit_snapshot(B, H, N, dk, dv, _ptr(snapshots), _ptr(parents), _ptr(accepted),
                                  _ptr(S_out), _ptr(path_out), _ptr(status), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_commit_snapshot")
    return S_out, path_out, status


def commit_verify(k_prev, alpha_prev, U_prev, parents_prev, accepted_prev, S_in,
                  q, k, v, alpha, beta, parents, mode=TV_GDN, S_out=None, inplace=False,
                  path_out=None, commit_status=None, o=None, U=None, status=None, stream=None):
    """Previous step's commit fused into this step's verification.

    Returns (S_out, path_out, commit_status, o, U, status): the committed state
    [B,H,dk,dv] (the new tree's root), the previous accepted path [B,N_prev] and
    its status, then tree_verify's outputs for the new tree against S_out.
    """
    B, N, H, dk = q.shape
    Np = k_prev.shape[1]
    dv = v.shape[3]
    dev = q.device
    dt = q.dtype
    _check(k_prev, "k_prev", (B, Np, H, dk), dt, dev)
    _check(alpha_prev, "alpha_prev", (B, Np, H), torch.float32, dev)
    _check(U_prev, "U_prev", (B, H, Np, dv), torch.float32, dev)
    _check(parents_prev, "parents_prev", (B, Np), torch.int32, dev)
    _check(accepted_prev, "accepted_prev", (B,), torch.int32, dev)
    _check(S_in, "S_in", (B, H, dk, dv), torch.float32, dev)
    _check(q, "q", (B, N, H, dk), dt, dev)
    _check(k, "k", (B, N, H, dk), dt, dev)
    _check(v, "v", (B, N, H, dv), dt, dev)
    _check(alpha, "alpha", (B, N, H), torch.float32, dev)
    if mode == TV_GDN or beta is not None:
        _check(beta, "beta", (B, N, H), torch.float32, dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    if S_out is None:
        S_out = S_in if inplace else torch.empty_like(S_in)
    if path_out is None:
        path_out = torch.empty((B, Np), dtype=torch.int32, device=dev)
    if commit_status is None:
        commit_status = torch.empty((B,), dtype=torch.int32, device=dev)
    if o is None:
        o = torch.empty((B, N, H, dv), dtype=dt, device=dev)
    if U is None:
        U = torch.empty((B, H, N, dv), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(S_out, "S_out", (B, H, dk, dv), torch.float32, dev)
    _check(path_out, "path_out", (B, Np), torch.int32, dev)
    _check(commit_status, "commit_status", (B,), torch.int32, dev)
    _check(o, "o", (B, N, H, dv), dt, dev)
    _check(U, "U", (B, H, N, dv), torch.float32, dev)
    _check(status, "status", (B,), torch.int32, dev)
    rc = LIB.tree_commit_verify(B, H, Np, N, dk, dv, _dtype_code(q), mode, _ptr(k_prev),
                                _ptr(alpha_prev), _ptr(U_prev), _ptr(parents_prev),
                                _ptr(accepted_prev), _ptr(S_in), _ptr(S_out), _ptr(path_out),
                                _ptr(commit_status), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(parents), _ptr(o), _ptr(U), _ptr(status),
                                _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_commit_verify")
    return S_out, path_out, commit_status, o, U, status


def attention(q, k_cache, v_cache, prefix_len, k_tree, v_tree, parents, scale, o=None, status=None,
              stream=None):
    """Tree-masked attention: o [B,N,Hq,D] bf16 and status [B] i32 (tree_attention)."""
    B, N, Hq, D = q.shape
    Hkv, P_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    bf = torch.bfloat16
    _check(q, "q", (B, N, Hq, D), bf, dev)
    _check(k_cache, "k_cache", (B, Hkv, P_max, D), bf, dev)
    _check(v_cache, "v_cache", (B, Hkv, P_max, D), bf, dev)
    _check(prefix_len, "prefix_len", (B,), torch.int32, dev)
    _check(k_tree, "k_tree", (B, N, Hkv, D), bf, dev)
    _check(v_tree, "v_tree", (B, N, Hkv, D), bf, dev)
    _check(parents, "parents", (B, N), torch.int32, dev)
    if o is None:
        o = torch.empty((B, N, Hq, D), dtype=bf, device=dev)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(o, "o", (B, N, Hq, D), bf, dev)
    _check(status, "status", (B,), torch.int32, dev)
    rc = LIB.tree_attention(B, N, Hq, Hkv, D, P_max, TV_BF16, _ptr(q), _ptr(k_cache),
                            _ptr(v_cache), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree),
                            _ptr(parents), ctypes.c_float(scale), _ptr(o), _ptr(status),
                            _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tree_attention")
    return o, status
