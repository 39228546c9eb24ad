"""bench.py's host-side accounting, on the CPU: the single-GPU refusal, the
algorithmic bytes the roofline divides by, and when committed counter
traffic may be reported."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tree_speculative_verification_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_verify_bytes_at_the_64_node_workload():
    """Per (sequence, head): S_root read (4 d_k d_v), q k v read, alpha and
    beta, o written (bf16), U written (fp32); parents and the accepted index
    per sequence.  Written out term by term for B=32, H=32, N=64, d=128."""
    bt = synth.make_inputs(4)
    verify, commit, fused, L = bench.algorithmic_bytes(bt)
    per_state = 4 * 128 * 128 + 64 * (128 + 128 + 128) * 2 + 64 * 8 + 64 * 128 * 2 + 64 * 128 * 4
    assert per_state == 164_352
    assert verify == 32 * 32 * per_state + 32 * (4 * 64 + 4) == 168_304_768
    # the fused step reads the state once: verify + commit minus one state read
    assert fused == verify + commit - 32 * 32 * 4 * 128 * 128
    assert L.shape == (32,) and L.min() >= 1 and L.max() <= 9


def test_attention_bytes_and_flops():
    bt = synth.make_attention_inputs()
    nbytes, flops = bench.attention_work(bt)
    B, N, Hq, D = bt.q.shape
    Hkv = bt.k_cache.shape[1]
    assert (B, N, Hq, Hkv, D) == (32, 64, 32, 8, 128)
    assert nbytes == 448_524_416
    # every node sees its prefix and its own root path (depth + 1 tree keys)
    keys = sum(int(bt.prefix_len[b]) * N + int((synth.depths_of(bt.parents[b]) + 1).sum())
               for b in range(B))
    assert flops == 4 * D * Hq * keys
    assert abs(flops / 1e9 - 104.2) < 0.1


def test_counter_traffic_needs_matching_sources(tmp_path, monkeypatch):
    sha = bench.sources_sha("fused")
    rec = {"fused_w4": {"bytes_per_launch": 12345, "source_sha": sha}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("fused", 4) == 12345
    rec["fused_w4"]["source_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("fused", 4) is None
    assert bench.measured_traffic("verify", 4) is None  # no record
    # trees above 128 nodes are hashed over the blocked kernel's sources
    assert bench.sources_sha("verify", large=True) != bench.sources_sha("verify")


def test_code_text_ignores_comments_only():
    base = 'int f(int a) {\n  // note\n  return a + 1; /* why */\n}\nconst char* s = "x // y";\n'
    reworded = 'int f(int a) {\n  // a different note\n  return a + 1;   /* another */\n}\nconst char* s = "x // y";\n'
    assert bench.code_text(base) == bench.code_text(reworded)
    assert bench.code_text(base) != bench.code_text(base.replace("a + 1", "a + 2"))
    # text inside string literals is code, comment markers included
    assert bench.code_text(base) != bench.code_text(base.replace('"x // y"', '"x // z"'))
    assert '"x // y"' in bench.code_text(base)
