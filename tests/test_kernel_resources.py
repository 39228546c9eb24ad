"""Register, scratch and LDS use of every kernel in the built library, read
from the code object's metadata (no GPU needed).

The kernels' designs rest on these numbers: no spills or scratch anywhere,
and the hot kernels within the LDS and register budgets of the residency
each one is laid out for (workgroups per CU, waves per SIMD).  A change that
silently pushes one of them over (a spill, an LDS array that no longer lets
two workgroups share a CU) fails here instead of only showing up as a slower
benchmark.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(ROOT, "tree_speculative_verification_amd", "libtreeverify.so")
LLVM = "/opt/rocm/llvm/bin"
BUNDLER = os.path.join(LLVM, "clang-offload-bundler")
READELF = os.path.join(LLVM, "llvm-readelf")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

LDS_PER_CU = 160 * 1024
VGPRS_PER_SIMD_LANE = 512  # architected + accumulation registers, shared by a SIMD's waves
FIELDS = ("name", "vgpr_count", "agpr_count", "vgpr_spill_count", "sgpr_spill_count",
          "private_segment_fixed_size", "group_segment_fixed_size")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not (shutil.which("objcopy") and os.path.exists(BUNDLER) and os.path.exists(READELF)):
        pytest.skip("objcopy or the ROCm LLVM tools are not available")
    if not os.path.exists(LIB_PATH):
        from tree_speculative_verification_amd import build
        build.build()
    d = tmp_path_factory.mktemp("co")
    fatbin = d / "fatbin"
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fatbin}", LIB_PATH, str(d / "lib")],
                   check=True, capture_output=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in the library"
    out = {}
    for i, s in enumerate(starts):
        e = starts[i + 1] if i + 1 < len(starts) else len(data)
        bundle, co = d / f"b{i}", d / f"b{i}.co"
        bundle.write_bytes(data[s:e])
        subprocess.run([BUNDLER, "--unbundle", "--type=o", f"--input={bundle}", f"--targets={TARGET}",
                        f"--output={co}"], check=True, capture_output=True)
        notes = subprocess.run([READELF, "--notes", str(co)], check=True, capture_output=True,
                               text=True).stdout
        for block in notes.split("\n  - ")[1:]:
            rec = dict(re.findall(r"\.(%s):\s+(\S+)" % "|".join(FIELDS), block))
            if "name" in rec and "vgpr_count" in rec:
                out[rec["name"]] = {k: (v if k == "name" else int(v)) for k, v in rec.items()}
    assert out, "no kernel metadata found"
    return out


def _find(kernels, *parts):
    """The one kernel whose mangled name contains every part."""
    hits = [r for n, r in kernels.items() if all(p in n for p in parts)]
    assert len(hits) == 1, (parts, [h["name"] for h in hits])
    return hits[0]


def _vgprs(rec):
    return rec["vgpr_count"] + rec.get("agpr_count", 0)


def test_no_spills_or_scratch_anywhere(kernels):
    bad = [(n, r["vgpr_spill_count"], r["sgpr_spill_count"], r["private_segment_fixed_size"])
           for n, r in kernels.items()
           if r["vgpr_spill_count"] or r["sgpr_spill_count"] or r["private_segment_fixed_size"]]
    assert not bad


def test_every_entry_points_kernel_is_present(kernels):
    for stem in ("verify_mfma_kernel", "verify_blocked_kernel", "verify_level_kernel",
                 "commit_kernel", "index_kernel", "index_wide_kernel", "tree_attention_kernel",
                 "snapshot_verify_kernel", "snapshot_commit_kernel"):
        assert any(stem in n for n in kernels), stem


# (name parts, workgroups per CU the design relies on, waves per workgroup)
RESIDENCY = [
    (("verify_mfma_kernel", "ILi64ELi64ELb1ELb0E"), 3, 4),    # fused commit + verify, 64 nodes
    (("verify_mfma_kernel", "ILi64ELi64ELb0ELb1E"), 2, 4),    # verify, 64 nodes, one workgroup per state
    (("verify_mfma_kernel", "ILi32ELi128ELb1ELb0E"), 3, 4),   # fused, 32 nodes
    (("verify_mfma_kernel", "ILi32ELi128ELb0ELb0E"), 3, 4),   # verify, 32 nodes
    (("verify_mfma_kernel", "ILi128ELi64ELb1ELb1E"), 1, 8),   # fused, 128 nodes
    (("verify_mfma_kernel", "ILi128ELi64ELb0ELb1E"), 1, 8),   # verify, 128 nodes
    (("verify_blocked_kernel", "ItLb1E"), 1, 16),             # blocked verify, up to 512 nodes
    (("tree_attention_kernel",), 2, 4),                       # tree attention
]


@pytest.mark.parametrize("parts,per_cu,waves", RESIDENCY, ids=[" ".join(p) for p, _, _ in RESIDENCY])
def test_hot_kernels_fit_their_residency(kernels, parts, per_cu, waves):
    rec = _find(kernels, *parts)
    assert rec["group_segment_fixed_size"] * per_cu <= LDS_PER_CU
    waves_per_simd = -(-per_cu * waves // 4)
    # registers come in granules of 8 per lane
    budget = VGPRS_PER_SIMD_LANE // waves_per_simd // 8 * 8
    assert _vgprs(rec) <= min(budget, 512)
