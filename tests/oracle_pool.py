"""The fp64 oracle over many (sequence, head) slices of a batch, in worker processes.

Workers are spawned, not forked, so they never inherit a process that has
initialised the GPU; they import only numpy and the oracle.  Each task gets one
sequence's slice (the heads asked for), so the whole batch is never pickled.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

import oracle


def _workers(n_tasks):
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, cores or 1, n_tasks))


def _verify_commit(sub):
    o, U, st_v = oracle.verify(sub.mode, sub.parents, sub.q, sub.k, sub.v, sub.alpha, sub.beta,
                               sub.S_root)
    S, st_c = oracle.commit(sub.mode, sub.parents, sub.accepted, sub.k, sub.v, sub.alpha,
                            sub.beta, sub.S_root)
    return o, U, S, st_v, st_c


def _commit_then_verify(args):
    prev, cur = args
    S_mid, st_c = oracle.commit(prev.mode, prev.parents, prev.accepted, prev.k, prev.v, prev.alpha,
                                prev.beta, prev.S_root)
    o, U, st_v = oracle.verify(cur.mode, cur.parents, cur.q, cur.k, cur.v, cur.alpha, cur.beta,
                               S_mid)
    return o, U, S_mid, st_v, st_c


def _run(fn, tasks):
    """fn over tasks in spawned workers; in this process if a worker cannot start
    (e.g. a main module that spawn cannot re-import)."""
    if len(tasks) == 1:
        return [fn(tasks[0])]
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"  # one BLAS thread per worker (inherited at spawn)
    try:
        with cf.ProcessPoolExecutor(_workers(len(tasks)), mp_context=mp.get_context("spawn")) as ex:
            return list(ex.map(fn, tasks, timeout=600))
    except (cf.process.BrokenProcessPool, OSError):
        return [fn(t) for t in tasks]
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _gather(batch, pairs, results):
    """Results per task back into arrays shaped like the batch (unvisited slices stay 0)."""
    B, N, H, dk, dv = batch.B, batch.N, batch.H, batch.dk, batch.dv
    o = np.zeros((B, N, H, dv))
    U = np.zeros((B, H, N, dv))
    S = np.zeros((B, H, dk, dv))
    st_v = np.zeros(B, np.int32)
    st_c = np.zeros(B, np.int32)
    for (b, hs), (ob, Ub, Sb, sv, sc) in zip(pairs, results):
        hs = np.asarray(hs)
        o[b][:, hs] = ob[0]
        U[b, hs] = Ub[0]
        S[b, hs] = Sb[0]
        st_v[b] = sv[0]
        st_c[b] = sc[0]
    return dict(o=o, U=U, S=S, status_v=st_v, status_c=st_c)


def verify_commit(batch, pairs):
    """Oracle verify + commit for each (b, heads) in pairs; arrays shaped like the batch."""
    tasks = [batch.select([b], hs) for b, hs in pairs]
    return _gather(batch, pairs, _run(_verify_commit, tasks))


def commit_then_verify(prev, cur, pairs):
    """Oracle commit of the previous tree, then verify of the new one from that state."""
    tasks = [(prev.select([b], hs), cur.select([b], hs)) for b, hs in pairs]
    return _gather(cur, pairs, _run(_commit_then_verify, tasks))
