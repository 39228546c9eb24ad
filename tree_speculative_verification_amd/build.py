"""Builds libtreeverify.so (gfx950) in-tree with hipcc.

    python -m tree_speculative_verification_amd.build [--jobs N] [--verbose]

Objects go to tree_speculative_verification_amd/_build/, the library next to
this file.  Always recompiles every source.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtreeverify.so")
ARCH = "gfx950"

SOURCES = ["tv_api.cpp", "tv_commit.hip", "tv_verify_level.hip", "tv_verify_mfma.hip",
           "tv_snapshot.hip",
           "tv_verify_blocked.hip", "tv_attention.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in the generated code: plain scalar FMAs only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libtreeverify.so")
    return exe


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel the host pass failed to instantiate shows up here,
    # not as a load error later
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
