"""The C ABI library loads, exports what include/tree_verify.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed:
every call here fails its host checks, so no device pointer is touched)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_verify.h")
LIB_PATH = os.path.join(ROOT, "tree_speculative_verification_amd", "libtreeverify.so")

TV_ERR_NULL, TV_ERR_DIMS, TV_ERR_HEAD_DIM, TV_ERR_MODE, TV_ERR_ALIAS, TV_ERR_ALGO = -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from tree_speculative_verification_amd import build
        build.build()
    L = ctypes.CDLL(LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.tree_verify.argtypes = [I] * 7 + [P] * 11
    L.tree_verify_algo.argtypes = [I] * 7 + [P] * 10 + [I, P]
    L.tree_commit.argtypes = [I] * 6 + [P] * 10
    L.tree_index.argtypes = [I, I] + [P] * 5
    L.tree_verify_snapshot.argtypes = [I] * 7 + [P] * 10 + [P]
    L.tree_commit_snapshot.argtypes = [I] * 5 + [P] * 6 + [P]
    L.tree_commit_verify.argtypes = [I] * 8 + [P] * 19
    L.tree_attention.argtypes = [I] * 7 + [P] * 7 + [ctypes.c_float] + [P] * 3
    L.tv_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected():
    assert declared_functions() == sorted(["tree_verify", "tree_verify_algo", "tree_commit",
                                           "tree_index", "tree_verify_snapshot",
                                           "tree_commit_snapshot", "tree_commit_verify",
                                           "tree_attention", "tv_status_string", "tv_version"])


def _doc_blocks():
    """Each declared function with the comment block right above its declaration."""
    text = open(HEADER).read()
    out = {}
    for m in re.finditer(r"/\*((?:(?!\*/).)*)\*/\s*((?:const\s+)?\w+\s*\*?\s*(\w+)\s*\()", text, flags=re.S):
        out[m.group(3)] = m.group(1)
    return out


def test_every_declaration_cites_its_passage():
    """Every entry point's comment names the page passage that defines it (the
    pages by title and section), or says that it is library bookkeeping."""
    blocks = _doc_blocks()
    pages = re.compile(r"(TreeWY|Twig|Bole)[^.]*(abstract|auto-summary|worked example|core formula|"
                       r"reconstruction formula)", flags=re.S | re.I)
    for name in declared_functions():
        assert name in blocks, f"{name} has no comment block"
        doc = blocks[name]
        assert pages.search(doc) or "Library bookkeeping" in doc or "cannot allocate" in doc, name


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_strings(lib):
    assert lib.tv_version() == 100
    for code in (0, 1, 2, 3, -1, -2, -3, -4, -5, -6, -107):
        s = lib.tv_status_string(code)
        assert s and s.decode() != "unknown code", code
    assert lib.tv_status_string(12345).decode() == "unknown code"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def _verify(lib, B=1, H=1, N=4, dk=16, dv=16, dtype=0, mode=0, nulls=(), algo=0,
            beta_null=False):
    ptrs = [None if i in nulls else FAKE for i in range(10)]
    if beta_null:
        ptrs[4] = None
    return lib.tree_verify_algo(B, H, N, dk, dv, dtype, mode, *ptrs, algo, None)


def test_verify_null_pointers(lib):
    for i in (0, 1, 2, 3, 5, 6, 7, 8):  # q k v alpha parents S_root o U
        assert _verify(lib, nulls=(i,), B=0) == TV_ERR_NULL


@pytest.mark.parametrize("B,H,N", [(0, 1, 4), (1, 0, 4), (1, 1, 0), (1, 1, 513), (-3, 1, 4),
                                   (1 << 30, 1 << 20, 128)])
def test_verify_bad_dims(lib, B, H, N):
    assert _verify(lib, B=B, H=H, N=N) == TV_ERR_DIMS


def test_verify_sequence_past_32bit_offsets(lib):
    """One sequence's N H d rows must stay addressable with 32-bit byte
    offsets: 512 nodes x 16384 heads x 128 x 4 bytes is just past 2^32."""
    assert _verify(lib, B=1, H=1 << 14, N=512, dk=128, dv=128, dtype=1) == TV_ERR_DIMS
    assert lib.tree_commit(1, 1 << 14, 512, 128, 128, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           None, None, None) == TV_ERR_DIMS


@pytest.mark.parametrize("dk,dv", [(8, 16), (16, 48), (256, 128), (0, 16)])
def test_verify_bad_head_dims(lib, dk, dv):
    assert _verify(lib, dk=dk, dv=dv) == TV_ERR_HEAD_DIM


def test_verify_bad_mode_dtype(lib):
    assert _verify(lib, dtype=2) == TV_ERR_MODE
    assert _verify(lib, mode=7) == TV_ERR_MODE
    assert _verify(lib, mode=0, beta_null=True) == TV_ERR_MODE


def test_verify_bad_algo(lib):
    assert _verify(lib, algo=9) == TV_ERR_ALGO
    assert _verify(lib, algo=2, dtype=0, dk=128, dv=128) == TV_ERR_ALGO   # fp32 has no MFMA path
    assert _verify(lib, algo=2, dtype=1, dk=64, dv=64) == TV_ERR_ALGO     # d != 128
    assert _verify(lib, algo=-1) == TV_ERR_ALGO
    # the register-path and level kernels take trees of at most 128 nodes
    assert _verify(lib, algo=2, dtype=1, dk=128, dv=128, N=129) == TV_ERR_ALGO
    assert _verify(lib, algo=1, N=129) == TV_ERR_ALGO


def test_commit_checks(lib):
    P = FAKE
    assert lib.tree_commit(1, 1, 4, 16, 16, 0, None, P, P, P, P, P, P, None, None, None) == TV_ERR_NULL
    assert lib.tree_commit(1, 1, 4, 16, 16, 0, P, P, P, P, None, P, P, None, None, None) == TV_ERR_NULL
    assert lib.tree_commit(1, 1, 513, 16, 16, 0, P, P, P, P, P, P, P, None, None, None) == TV_ERR_DIMS
    assert lib.tree_commit(1, 1, 4, 16, 24, 0, P, P, P, P, P, P, P, None, None, None) == TV_ERR_HEAD_DIM
    assert lib.tree_commit(1, 1, 4, 16, 16, 5, P, P, P, P, P, P, P, None, None, None) == TV_ERR_MODE
    # S_out starting 4 bytes into S_root: partial overlap
    s0 = ctypes.c_void_p(0x100000)
    s1 = ctypes.c_void_p(0x100004)
    assert lib.tree_commit(1, 1, 4, 16, 16, 0, P, P, P, P, P, s0, s1, None, None, None) == TV_ERR_ALIAS
    assert lib.tree_commit(1, 1, 4, 16, 16, 0, P, P, P, P, P, s1, s0, None, None, None) == TV_ERR_ALIAS


def test_index_checks(lib):
    P = FAKE
    assert lib.tree_index(1, 4, None, P, P, None, None) == TV_ERR_NULL
    assert lib.tree_index(1, 4, P, None, P, None, None) == TV_ERR_NULL
    assert lib.tree_index(0, 4, P, P, P, None, None) == TV_ERR_DIMS
    assert lib.tree_index(1, 513, P, P, P, None, None) == TV_ERR_DIMS


def test_snapshot_checks(lib):
    P = FAKE
    args = lambda **kw: [kw.get("B", 1), kw.get("H", 1), kw.get("N", 4), kw.get("dk", 16),
                         kw.get("dv", 16), kw.get("dtype", 0), kw.get("mode", 0)]
    ptrs = [P] * 9 + [None]   # q k v alpha beta parents S_root snapshots o, status = NULL
    assert lib.tree_verify_snapshot(*args(), *([None] + ptrs[1:]), None) == TV_ERR_NULL
    assert lib.tree_verify_snapshot(*args(), *(ptrs[:7] + [None] + ptrs[8:]), None) == TV_ERR_NULL
    assert lib.tree_verify_snapshot(*args(N=129), *ptrs, None) == TV_ERR_DIMS   # baseline: N <= 128
    assert lib.tree_verify_snapshot(*args(dv=48), *ptrs, None) == TV_ERR_HEAD_DIM
    assert lib.tree_verify_snapshot(*args(mode=3), *ptrs, None) == TV_ERR_MODE
    nob = ptrs[:4] + [None] + ptrs[5:]
    assert lib.tree_verify_snapshot(*args(), *nob, None) == TV_ERR_MODE   # GDN needs beta
    # B H N d_k d_v beyond 2^44 floats of snapshots
    assert lib.tree_verify_snapshot(*args(B=1 << 20, H=64, N=128, dk=128, dv=128), *ptrs, None) == TV_ERR_DIMS
    assert lib.tree_commit_snapshot(1, 1, 4, 16, 16, None, P, P, P, None, None, None) == TV_ERR_NULL
    assert lib.tree_commit_snapshot(1, 1, 4, 16, 16, P, P, None, P, None, None, None) == TV_ERR_NULL
    assert lib.tree_commit_snapshot(1, 1, 0, 16, 16, P, P, P, P, None, None, None) == TV_ERR_DIMS
    assert lib.tree_commit_snapshot(1, 1, 129, 16, 16, P, P, P, P, None, None, None) == TV_ERR_DIMS
    # S_out inside the snapshot buffer
    s0 = ctypes.c_void_p(0x100000)
    s1 = ctypes.c_void_p(0x100000 + 4 * 16 * 16)
    assert lib.tree_commit_snapshot(1, 1, 4, 16, 16, s0, P, P, s1, None, None, None) == TV_ERR_ALIAS


def test_commit_verify_checks(lib):
    P = FAKE
    # pointers: k_prev alpha_prev U_prev parents_prev accepted_prev S_in S_out path_out
    # commit_status | q k v alpha beta parents o U status | stream
    def call(ptrs=None, B=1, H=1, Np=4, N=4, dk=16, dv=16, dtype=0, mode=0, **over):
        p = [P] * 7 + [None, None] + [P] * 8 + [None] if ptrs is None else ptrs
        for i, v in over.items():
            p[int(i[1:])] = v
        return lib.tree_commit_verify(B, H, Np, N, dk, dv, dtype, mode, *p, None)
    for i in (0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12, 14, 15, 16):
        assert call(**{f"p{i}": None}) == TV_ERR_NULL, i
    assert call(p13=None, mode=0) == TV_ERR_MODE          # GDN needs beta
    assert call(Np=0) == TV_ERR_DIMS
    assert call(Np=513) == TV_ERR_DIMS
    assert call(N=513) == TV_ERR_DIMS
    assert call(dv=48) == TV_ERR_HEAD_DIM
    assert call(dtype=3) == TV_ERR_MODE
    assert call(mode=4) == TV_ERR_MODE
    # S_out partly over S_in
    assert call(p5=ctypes.c_void_p(0x100000), p6=ctypes.c_void_p(0x100004)) == TV_ERR_ALIAS
    # U (new, 4 nodes x 16 floats) over U_prev
    assert call(p2=ctypes.c_void_p(0x200000), p16=ctypes.c_void_p(0x200000 + 4 * 16 * 4 - 4)) == TV_ERR_ALIAS
    assert call(p2=ctypes.c_void_p(0x200000 + 4 * 16 * 4 - 4), p16=ctypes.c_void_p(0x200000)) == TV_ERR_ALIAS


def test_product_path_has_no_oracle_import():
    """The library package never reaches into the oracle (or any CPU fallback)."""
    pkg = os.path.join(ROOT, "tree_speculative_verification_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "tree_oracle" not in text, f


def test_attention_checks(lib):
    P = FAKE
    # B N Hq Hkv D P_max dtype | q kc vc plen kt vt parents | scale | o status stream
    def call(B=1, N=4, Hq=4, Hkv=2, D=128, Pm=8, dtype=1, scale=0.1, **over):
        p = [P] * 7 + [P, None, None]
        for i, v in over.items():
            p[int(i[1:])] = v
        return lib.tree_attention(B, N, Hq, Hkv, D, Pm, dtype, *p[:7], ctypes.c_float(scale), *p[7:])
    for i in (0, 3, 4, 5, 6, 7):           # q plen k_tree v_tree parents o
        assert call(**{f"p{i}": None}) == TV_ERR_NULL, i
    assert call(p1=None) == TV_ERR_NULL     # caches are required when P_max > 0
    assert call(p1=None, p2=None, Pm=0, B=0) == TV_ERR_DIMS   # allowed NULL, then the size check
    assert call(B=0) == TV_ERR_DIMS
    assert call(N=513) == TV_ERR_DIMS
    assert call(Hq=6, Hkv=4) == TV_ERR_DIMS  # Hq not a multiple of Hkv
    assert call(Pm=-1) == TV_ERR_DIMS
    assert call(D=64) == TV_ERR_HEAD_DIM
    assert call(dtype=0) == TV_ERR_MODE


def test_host_checks_under_address_and_ub_sanitizers(tmp_path):
    """tv_api.cpp built for the CPU alone (g++, no device code) with AddressSanitizer
    and UBSan, linked against launchers that only count calls: every entry point
    with good and bad arguments; bad ones must return their code and launch nothing."""
    import shutil
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    here = os.path.join(ROOT, "tests", "host_sanitize")
    exe = str(tmp_path / "abi_asan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "tree_speculative_verification_amd", "csrc"),
           os.path.join(ROOT, "tree_speculative_verification_amd", "csrc", "tv_api.cpp"),
           os.path.join(here, "stub_launchers.cpp"), os.path.join(here, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    # another preloaded library may come before the ASan runtime: allow that order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert r.stdout.startswith("ok:"), r.stdout
