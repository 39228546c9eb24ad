#!/usr/bin/env python3
"""Verified tree nodes/s through one gated-delta-rule layer on one MI355X.

Workload: the 64-node tree (B=32 sequences, H=32 heads, d_k=d_v=128, bf16
q/k/v, fp32 state, a random 64-node draft tree per sequence, accepted node
uniform over nodes).  Inputs are seeded synthetic data, resident in HBM
before timing starts.

One step verifies one batch and commits one batch.  Two pipelines are timed:
  * fused (the headline): one tree_commit_verify launch per step, which
    commits an earlier batch's accepted path into its state and verifies
    this batch's tree against the result, reading the state once;
  * two-kernel: tree_verify + tree_commit per step.
Cold caches without flush kernels: R copies of the input set (>= 1 GB in all,
far above the 256 MB Infinity Cache and the L2s) are used in turn, and a
step's commit takes the batch verified two steps earlier, so every kernel
streams its operands from HBM, as it would with the rest of a model forward
between verify and commit.  Warm-up: at least W steps and at least 250 ms of
GPU time (the clocks ramp over the first tens of milliseconds, so a count
alone makes short runs read slow), then, before each timed loop, 30 ms of
that loop's own body.  K timed steps run between one pair of HIP events on
the launch stream (bracketed by device synchronizations).  ms_per_step is
that time / K; value = B*N / ms_per_step of the fused pipeline.  Per-kernel
durations for the roofline come from K back-to-back launches of each kernel
over the same ring.

Prints ONE JSON line.  Options: --steps K --warmup W --gpus 1 (only 1 is
supported: the path runs on one GPU) --workload {3,4,5,6} --no-cpu-baseline.
Workload 6 (512-node trees) runs the blocked verification kernel; its step is
tree_commit_verify's two launches (commit, then blocked verify), and the
roofline line reports the blocked verify kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from tree_speculative_verification_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
# worker processes of the CPU oracle baseline: the host share of one GPU
CPU_WORKER_CAP = 16
# warm-up: at least this much GPU time before the first timed launch (clocks ramp
# over the first tens of milliseconds), and this much per timed body before its loop
WARM_MS = 250.0
WARM_BODY_MS = 30.0
METRIC = "verified tree nodes/s per GDN layer (1 GPU) + % of HBM roofline"
_CSRC = "tree_speculative_verification_amd/csrc/"
KERNEL_SOURCES = {
    "verify": [_CSRC + "tv_verify_mfma.hip", _CSRC + "tv_device.h"],
    "fused": [_CSRC + "tv_verify_mfma.hip", _CSRC + "tv_device.h"],
    "commit": [_CSRC + "tv_commit.hip", _CSRC + "tv_device.h"],
}
KERNEL_SOURCES["attention"] = [_CSRC + "tv_attention.hip", _CSRC + "tv_device.h"]
# trees above 128 nodes: blocked verification, and commit + blocked verify as the step
KERNEL_SOURCES_LARGE = {
    "verify": [_CSRC + "tv_verify_blocked.hip", _CSRC + "tv_device.h"],
    "fused": [_CSRC + "tv_verify_blocked.hip", _CSRC + "tv_commit.hip", _CSRC + "tv_device.h"],
    "commit": [_CSRC + "tv_commit.hip", _CSRC + "tv_device.h"],
}
SMALL_TREE = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def path_lengths(parents, accepted):
    L = np.zeros(len(accepted), dtype=np.int64)
    for b, a in enumerate(accepted):
        n, c = int(a), 0
        while n >= 0:
            c += 1
            n = int(parents[b, n])
        L[b] = c
    return L


def algorithmic_bytes(bt):
    """Bytes each kernel must move at least once (inputs read, outputs written)."""
    B, N, H, dk, dv = bt.B, bt.N, bt.H, bt.dk, bt.dv
    s = 2 if bt.dtype == synth.BF16 else 4
    gates = 8 * N if bt.mode == synth.GDN else 4 * N
    verify_bh = 4 * dk * dv + N * (2 * dk + dv) * s + gates + N * dv * s + 4 * N * dv
    verify = B * H * verify_bh + B * (4 * N + 4)
    L = path_lengths(bt.parents, bt.accepted)
    commit = int(np.sum(H * (8 * dk * dv + L * (dk * s + 4 * dv + 4)))) + B * (4 * N + 4 + 4 + 4 * N)
    # fused: both, with the state read once (the commit's read is the verify's)
    fused = verify + commit - B * H * 4 * dk * dv
    return int(verify), int(commit), int(fused), L


def code_text(src):
    """C++ source without comments and with whitespace runs collapsed, so that
    comment-only edits keep a counter record valid and any code change does not."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # string or character literal, copied as is
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_sha(kind, large=False):
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES_LARGE if large else KERNEL_SOURCES)[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kind, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(f"{kind}_w{workload}")
    large = workload in synth.CONFIGS and synth.CONFIGS[workload]["N"] > SMALL_TREE
    if not r or r.get("source_sha") != sources_sha(kind, large):
        return None
    return r.get("bytes_per_launch")


# ------------------------------------------------------------ CPU baseline

_CPU_BATCH = None


def _oracle_seq(b):
    import oracle
    bt = _CPU_BATCH
    sub = bt.select([b], np.arange(bt.H))
    oracle.verify(sub.mode, sub.parents, sub.q, sub.k, sub.v, sub.alpha, sub.beta, sub.S_root)
    oracle.commit(sub.mode, sub.parents, sub.accepted, sub.k, sub.v, sub.alpha, sub.beta, sub.S_root)
    return b


def cpu_baseline(bt, max_seqs, reps):
    """The fp64 oracle (as it stands) over whole sequences, one process per core.

    Runs before the GPU is touched (the pool forks).  `reps` passes over the
    sequences.  Returns nodes/s scaled to the metric: sequences done * N / wall
    seconds.
    """
    global _CPU_BATCH
    import multiprocessing as mp
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    _CPU_BATCH = bt
    seqs = list(range(min(bt.B, max_seqs))) * reps
    avail = len(os.sched_getaffinity(0))
    cores = min(avail, CPU_WORKER_CAP, len(seqs))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        list(pool.imap_unordered(_oracle_seq, seqs))
    wall = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": len(seqs) * bt.N / wall, "unit": "nodes/s", "cores": cores,
            "cores_available": avail, "kind": "oracle",
            "sample": f"{len(seqs) // reps} of {bt.B} sequences x all {bt.H} heads of the same "
                      f"workload, {reps} passes (fp64 token-by-token path walk, verify + commit), "
                      f"wall {wall:.2f} s on {cores} worker processes ({avail} cores available "
                      f"to this process, at most {CPU_WORKER_CAP} used), 1 BLAS thread each; "
                      f"{cpu_model}"}


def warm_up(body, min_calls, min_ms):
    """Runs body(i) at least min_calls times and until min_ms of wall time has passed
    with the GPU busy (synchronizing every few calls); returns (calls, ms)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            body(i)
            i += 1
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        if i >= min_calls and ms >= min_ms:
            return i, ms


# ------------------------------------------------------ tree attention leg

MFMA_BF16_PEAK_TFLOPS = 2500.0
ATTN_METRIC = "verified tree nodes/s per full-attention layer (1 GPU) + % of HBM roofline"


def attention_work(bt):
    """Algorithmic bytes and flops of one tree_attention launch.

    Bytes: q and o, the prefix rows of both caches that are visible (each
    read once per key/value head), the tree's k and v rows, prefix_len and
    parents.  Flops: 4 D per (query row, visible key) (q.k and p v)."""
    B, N, Hq, D = bt.q.shape
    Hkv = bt.k_cache.shape[1]
    depth = np.stack([synth.depths_of(p) for p in bt.parents])          # [B, N]
    nbytes = (2 * B * N * Hq * D * 2 + int(bt.prefix_len.sum()) * Hkv * D * 2 * 2
              + B * N * Hkv * D * 2 * 2 + B * 4 + B * N * 4)
    keys = bt.prefix_len[:, None] + depth + 1                           # visible keys per node
    flops = 4 * D * Hq * int(keys.sum())
    return int(nbytes), int(flops)


_ATTN_BATCH = None


def _oracle_attn_seq(bh):
    from threadpoolctl import threadpool_limits

    from oracle import tree_attention as A
    threadpool_limits(1)  # one BLAS thread per worker process
    b, h = bh
    bt = _ATTN_BATCH
    A.tree_attention(bt.parents, bt.q, bt.k_cache, bt.v_cache, bt.prefix_len, bt.k_tree,
                     bt.v_tree, bt.scale, seqs=[b], heads=[h])


def attention_cpu_baseline(bt, pairs):
    """The fp64 oracle over `pairs` (sequence, query head) of the workload, one
    process per core; scaled to nodes/s of the whole layer (every head)."""
    global _ATTN_BATCH
    import multiprocessing as mp
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    _ATTN_BATCH = bt
    B, N, Hq, _ = bt.q.shape
    work = [(b, h) for b in range(B) for h in range(Hq)][:pairs]
    avail = len(os.sched_getaffinity(0))
    cores = min(avail, CPU_WORKER_CAP, len(work))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        list(pool.imap_unordered(_oracle_attn_seq, work))
    wall = time.perf_counter() - t0
    # one sequence's N nodes need all Hq heads: nodes/s = pairs * N / Hq / wall
    return {"value": len(work) * N / Hq / wall, "unit": "nodes/s", "cores": cores,
            "cores_available": avail, "kind": "oracle",
            "sample": f"{len(work)} (sequence, query head) pairs of the workload, all {N} nodes "
                      f"each (fp64 masked softmax per node), scaled to whole nodes (all {Hq} "
                      f"heads); wall {wall:.2f} s on {cores} worker processes"}


def attention_main(a):
    bt = synth.make_attention_inputs()
    cpu = None if a.no_cpu_baseline else attention_cpu_baseline(bt, a.cpu_attn_pairs)

    import torch
    from tree_speculative_verification_amd import binding as tvb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = synth.attention_to_torch(bt, dev)
    B, N, Hq, D = bt.q.shape
    set_bytes = sum(x.numel() * x.element_size() for x in base.values() if torch.is_tensor(x))
    R = max(2, -(-(1 << 30) // set_bytes))
    sets = [base] + [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
                     for _ in range(R - 1)]
    for t in sets:
        t["o"] = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
        t["st"] = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        t = sets[i % R]
        tvb.attention(t["q"], t["k_cache"], t["v_cache"], t["prefix_len"], t["k_tree"],
                      t["v_tree"], t["parents"], t["scale"], o=t["o"], status=t["st"],
                      stream=stream)

    warm_calls, warm_ms = warm_up(step, a.warmup, a.warmup_ms)
    if any(t["st"].any().item() for t in sets):
        raise RuntimeError("device status reported bad input rows")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    nbytes, flops = attention_work(bt)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": ATTN_METRIC, "value": round(B * N / (ms * 1e-3), 1), "unit": "nodes/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "warmup_done": {"calls": warm_calls, "ms": round(warm_ms, 1)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": synth.ATTN_NAME, "B": B, "N": N, "Hq": Hq,
                   "Hkv": bt.k_cache.shape[1], "D": D, "P_max": bt.k_cache.shape[2],
                   "mean_prefix": round(float(bt.prefix_len.mean()), 1),
                   "timing": f"HIP events around K launches on the launch stream; ring of {R} "
                             "input copies (>= 1 GB) so every launch reads cold caches"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("attention", "attn"),
                     "kernel": "tree_attention_kernel", "algorithmic_bytes": nbytes},
        "mfma": {"achieved_TFLOPs": round(tfs, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
                 "arithmetic_intensity_flop_per_byte": round(flops / nbytes, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# --------------------------------------------------------------- GPU timing

def copy_calibration():
    """A copy of known size: 256 MiB read + 256 MiB written per launch."""
    import torch
    nbytes = 1 << 28
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    big = torch.empty(1 << 28, device="cuda")
    for _ in range(3):
        big.sum()          # read-only pass over 1 GiB: evicts src and dst, leaves nothing dirty
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                           "launches": 3}}), flush=True)
    return 0


def snapshot_baseline(tvb, sets, R, bt, stream, timed, steps, ms_tree, snap_bytes):
    """The method the pages compare against, on the same GPU and inputs: verify by
    walking the nodes with a full per-node state snapshot, commit by copying the
    accepted node's snapshot.  One snapshot buffer (B H N d_k d_v floats) is shared
    by all steps; the input sets rotate as in the main timing."""
    import torch
    B, N, H, dk, dv = bt.B, bt.N, bt.H, bt.dk, bt.dv
    snaps = torch.empty((B, H, N, dk, dv), dtype=torch.float32, device=sets[0]["q"].device)

    def verify(i):
        t = sets[i % R]
        tvb.verify_snapshot(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["parents"],
                            t["S_root"], mode=bt.mode, snapshots=snaps, o=t["o"],
                            status=t["st_v"], stream=stream)

    def commit(i):
        t = sets[i % R]
        tvb.commit_snapshot(snaps, t["parents"], t["accepted"], S_out=t["S_out"],
                            path_out=t["path"], status=t["st_c"], stream=stream)

    def step(i):
        verify(i)
        commit(i)

    k = max(3, steps // 5)
    for i in range(2):
        step(i)
    ms_step, _ = timed(step, k)
    v_ms, _ = timed(verify, k)
    c_ms, _ = timed(commit, k)
    del snaps
    torch.cuda.empty_cache()
    return {"method": "sequential per-node state snapshots (verify walks the nodes in index order "
                      "and writes every node's full fp32 state; commit copies the accepted one)",
            "ms_per_step": round(ms_step, 4), "nodes_per_s": round(B * N / (ms_step * 1e-3), 1),
            "verify_us": round(v_ms * 1e3, 1), "commit_us": round(c_ms * 1e3, 1),
            "steps": k, "snapshot_bytes": snap_bytes,
            "speedup_tree_vs_snapshot": round(ms_step / ms_tree, 2)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-ms", type=float, default=WARM_MS,
                    help="least GPU time of warm-up before timing (0 for short profiled runs)")
    ap.add_argument("--workload", type=int, default=4, choices=[3, 4, 5, 6])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--cpu-reps", type=int, default=5,
                    help="passes of the CPU oracle over the sampled sequences")
    ap.add_argument("--no-snapshot-baseline", action="store_true",
                    help="skip timing the per-node-snapshot baseline kernels")
    ap.add_argument("--attention", action="store_true",
                    help="time tree_attention (the hybrid's full-attention layers) on its "
                         "workload instead of the verification pipeline")
    ap.add_argument("--cpu-attn-pairs", type=int, default=256,
                    help="(sequence, head) pairs of the attention oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device-to-device copy (three times, caches "
                         "evicted by a read-only pass before each), to scale rocprofv3's "
                         "FETCH_SIZE / WRITE_SIZE readings to bytes")
    a = ap.parse_args(argv)
    if a.copy_calibration:
        return copy_calibration()
    if a.gpus != 1:
        print(f"bench.py: --gpus {a.gpus} is not supported; this path runs on one GPU "
              "(every (sequence, head) is independent, so more GPUs only split the batch).",
              file=sys.stderr)
        return 2
    if int(os.environ.get("RANK", "0")) != 0:
        return 0
    if a.attention:
        return attention_main(a)

    bt = synth.make_inputs(a.workload)
    cpu = None if a.no_cpu_baseline else cpu_baseline(bt, a.cpu_seqs, a.cpu_reps)

    import torch
    from tree_speculative_verification_amd import binding as tvb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host = synth.to_torch(bt, "cpu")
    B, N, H, dk, dv = bt.B, bt.N, bt.H, bt.dk, bt.dv
    set_bytes = sum(x.numel() * x.element_size() for x in host.values() if torch.is_tensor(x))
    set_bytes += B * N * H * dv * host["q"].element_size() + 2 * B * H * N * dv * 4 + B * H * dk * dv * 4
    R = max(3, -(-(1 << 30) // set_bytes))
    sets = []
    for _ in range(R):
        t = {key: (x.to(dev) if torch.is_tensor(x) else x) for key, x in host.items()}
        t["o"] = torch.empty((B, N, H, dv), dtype=t["q"].dtype, device=dev)
        t["U"] = torch.empty((B, H, N, dv), dtype=torch.float32, device=dev)
        t["S_out"] = torch.empty_like(t["S_root"])
        t["st_v"] = torch.empty((B,), dtype=torch.int32, device=dev)
        t["st_c"] = torch.empty((B,), dtype=torch.int32, device=dev)
        t["path"] = torch.empty((B, N), dtype=torch.int32, device=dev)
        sets.append(t)
    stream = torch.cuda.current_stream()

    def verify(i):
        t = sets[i % R]
        tvb.verify(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["parents"], t["S_root"],
                   mode=bt.mode, o=t["o"], U=t["U"], status=t["st_v"], stream=stream)

    def commit(i):
        t = sets[i % R]
        tvb.commit(t["k"], t["alpha"], t["U"], t["parents"], t["accepted"], t["S_root"],
                   S_out=t["S_out"], path_out=t["path"], status=t["st_c"], stream=stream)

    def fused(i):
        p = sets[(i - 2) % R]
        t = sets[i % R]
        tvb.commit_verify(p["k"], p["alpha"], p["U"], p["parents"], p["accepted"], p["S_root"],
                          t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["parents"],
                          mode=bt.mode, S_out=t["S_out"], path_out=p["path"],
                          commit_status=p["st_c"], o=t["o"], U=t["U"], status=t["st_v"],
                          stream=stream)

    def timed(body, k):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(k):
            body(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k, (time.perf_counter() - w0) / k * 1e3

    for i in range(R):          # every set gets pseudo-values before its first commit
        verify(i)

    def step2(i):
        verify(i)
        commit(i - 2)

    def both(i):
        step2(i)
        fused(i)

    warm_calls, warm_ms = warm_up(both, a.warmup, a.warmup_ms)
    for t in sets:
        if t["st_v"].any().item() or t["st_c"].any().item():
            raise RuntimeError("device status reported bad input rows")

    body_ms = WARM_BODY_MS if a.warmup_ms > 0 else 0.0

    def timed_warm(body, k):
        """K timed launches of body, after WARM_BODY_MS of the same body."""
        warm_up(body, 1, body_ms)
        return timed(body, k)

    ms_step, wall_ms = timed_warm(fused, a.steps)
    ms_two, _ = timed_warm(step2, a.steps)
    tv_ms, _ = timed_warm(verify, a.steps)
    tc_ms, _ = timed_warm(commit, a.steps)

    base = None
    snap_bytes = B * H * N * dk * dv * 4
    large = N > SMALL_TREE
    if not a.no_snapshot_baseline and snap_bytes <= (64 << 30) and not large:
        base = snapshot_baseline(tvb, sets, R, bt, stream, timed, a.steps, ms_step, snap_bytes)

    value = B * N / (ms_step * 1e-3)
    vbytes, cbytes, fbytes, L = algorithmic_bytes(bt)
    kern = {}
    for name, ms, nbytes in (("fused", ms_step, fbytes), ("verify", tv_ms, vbytes),
                             ("commit", tc_ms, cbytes)):
        gbs = nbytes / (ms * 1e-3) / 1e9
        kern[name] = {"mean_us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
                      "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic(name, a.workload)}
    if large:
        kern["fused"]["entry"] = ("tree_commit_verify (trees above 128 nodes: commit, then the "
                                  "blocked verification, two launches per step)")
        kern["verify"]["kernel"] = "blocked verification (verify_blocked_kernel)"
        dom = "verify"
    else:
        kern["fused"]["entry"] = "tree_commit_verify (one launch per step)"
        dom = "fused"
    combined_gbs = (vbytes + cbytes) / (ms_two * 1e-3) / 1e9
    snap = B * H * N * dk * dv * 4
    u_only = B * H * N * dv * 4
    u_k_g = B * H * N * (4 * dv + (2 if bt.dtype == synth.BF16 else 4) * dk + 4)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 5),
        "warmup_done": {"calls": warm_calls, "ms": round(warm_ms, 1),
                        "per_body_ms": body_ms},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": synth.CONFIG_NAMES[a.workload], "B": B, "H": H, "N": N,
                   "d_k": dk, "d_v": dv, "qkv": "bf16", "state": "fp32", "layer": "gated delta rule",
                   "mean_path_len": round(float(L.mean()), 3),
                   "pipeline": ("tree_commit_verify per step: commit of the batch verified 2 "
                                "steps earlier, then the blocked verification of this batch"
                                if large else
                                "fused: one tree_commit_verify launch per step (commit of the "
                                "batch verified 2 steps earlier + verify of this batch)"),
                   "timing": f"HIP events around K steps on the launch stream; ring of {R} input "
                             "copies (>= 1 GB) so every kernel reads cold data; commit lags verify "
                             "by 2 steps"},
        "roofline": {"bound": "hbm", "achieved": kern[dom]["achieved_GBs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kern[dom]["frac"], "traffic": kern[dom]["traffic"],
                     "kernel": dom},
        "kernels": kern,
        "two_kernel_pipeline": {"ms_per_step": round(ms_two, 5),
                                "nodes_per_s": round(B * N / (ms_two * 1e-3), 1),
                                "achieved_GBs": round(combined_gbs, 1),
                                "frac": round(combined_gbs / HBM_PEAK_GBS, 4),
                                "algorithmic_bytes": vbytes + cbytes,
                                "fused_speedup": round(ms_two / ms_step, 3)},
        "wall_ms_per_step": round(wall_ms, 5),
        "transient_state_bytes": {"per_node_snapshots": snap, "U_only": u_only,
                                  "U_plus_K_and_gates": u_k_g,
                                  "ratio_snapshots_to_U": round(snap / u_only, 2),
                                  "ratio_snapshots_to_U_K_gates": round(snap / u_k_g, 2)},
        "cpu_baseline": cpu,
        "snapshot_baseline": base if not large else {
            "skipped": "the per-node-snapshot kernels take trees of at most 128 nodes "
                       f"(this batch would need {snap_bytes} bytes of snapshots)"},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
