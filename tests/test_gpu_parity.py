"""HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs."""
import functools

import numpy as np
import pytest

import oracle
import oracle_pool
from parity import TOL, compare, max_rel, run_gpu, run_oracle
from tree_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

LEVEL, MFMA = 1, 2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from tree_speculative_verification_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    torch.cuda.init()


@functools.lru_cache(maxsize=None)
def cfg_batch(cfg):
    return synth.make_inputs(cfg)


def _check(batch, gpu, ref, rows=None):
    ok, errs = compare(gpu, ref, batch.dtype, rows)
    assert ok, errs
    return errs


# ---------------------------------------------------------------- tree index

def _random_parents(rng, B, N, kind):
    par = np.full((B, N), -1, np.int32)
    for b in range(B):
        for i in range(1, N):
            if kind == "chain":
                par[b, i] = i - 1
            elif kind == "forest" and rng.random() < 0.25:
                par[b, i] = -1
            elif kind == "star":
                par[b, i] = 0
            else:
                par[b, i] = rng.integers(0, i)
    return par


@pytest.mark.parametrize("N", [1, 2, 7, 31, 63, 64, 65, 100, 127, 128])
@pytest.mark.parametrize("kind", ["random", "chain", "forest", "star"])
def test_index_bit_exact(N, kind):
    import torch

    from tree_speculative_verification_amd import binding as tvb
    rng = np.random.default_rng(N * 7 + len(kind))
    par = _random_parents(rng, 5, N, kind)
    if N > 2:
        par[1, N - 1] = N - 1       # self parent: invalid
        par[3, 1] = -2              # below -1: invalid
    depth, anc, st = tvb.index(torch.from_numpy(par).cuda())
    d_ref, a_ref, s_ref = oracle.tree_index(par)
    assert np.array_equal(st.cpu().numpy(), s_ref)
    assert np.array_equal(depth.cpu().numpy(), d_ref)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), a_ref)


# ------------------------------------------------------------- workloads

@pytest.mark.parametrize("cfg,algo", [(1, 0), (2, 0), (3, 0), (3, LEVEL)])
def test_small_configs(cfg, algo):
    bt = cfg_batch(cfg)
    gpu = run_gpu(bt, algo=algo)
    ref = run_oracle(bt)
    assert np.array_equal(gpu["path"], ref["path"])
    assert not gpu["status_v"].any() and not gpu["status_c"].any()
    _check(bt, gpu, ref)


def _sampled(cfg, nb, nh, seed):
    bt = cfg_batch(cfg)
    rng = np.random.default_rng(seed)
    bs = np.sort(rng.choice(bt.B, nb, replace=False))
    hs = np.sort(rng.choice(bt.H, nh, replace=False))
    return bt, bs, hs


@pytest.mark.parametrize("cfg,algo", [(4, 0), (4, LEVEL), (5, 0)])
def test_full_size_sampled(cfg, algo):
    """Full-size launch (as the benchmark runs it); oracle on sampled (sequence, head) slices."""
    bt, bs, hs = _sampled(cfg, 4, 3, seed=cfg * 10 + algo)
    gpu = run_gpu(bt, algo=algo)
    sub = bt.select(bs, hs)
    ref = run_oracle(sub)
    g = dict(o=gpu["o"][bs][:, :, hs], U=gpu["U"][bs][:, hs], S=gpu["S"][bs][:, hs])
    _check(sub, g, ref)
    # integer outputs for every sequence, checked against the oracle's walk
    path_ref, st_ref = oracle.accepted_paths(bt.parents, bt.accepted)
    assert np.array_equal(gpu["path"], path_ref)
    assert not gpu["status_v"].any() and not gpu["status_c"].any()


def test_full_size_every_state_64_node():
    """The 64-node workload at full size (B=32, H=32), as the benchmark launches it:
    every (sequence, head) state of the launch against the oracle (verify + commit)."""
    bt = cfg_batch(4)
    gpu = run_gpu(bt)
    ref = oracle_pool.verify_commit(bt, [(b, list(range(bt.H))) for b in range(bt.B)])
    assert not gpu["status_v"].any() and not gpu["status_c"].any()
    path_ref, _ = oracle.accepted_paths(bt.parents, bt.accepted)
    assert np.array_equal(gpu["path"], path_ref)
    _check(bt, gpu, ref)


def _diag(gpu, ref, pairs):
    """The listed (b, h) slices of both sides as [P, ..., 1, ...] arrays for compare()."""
    g = dict(o=np.stack([gpu["o"][b, :, h] for b, h in pairs])[:, :, None],
             U=np.stack([gpu["U"][b, h] for b, h in pairs])[:, None],
             S=np.stack([gpu["S"][b, h] for b, h in pairs])[:, None])
    r = dict(o=np.stack([ref["o"][b, :, h] for b, h in pairs])[:, :, None],
             U=np.stack([ref["U"][b, h] for b, h in pairs])[:, None],
             S=np.stack([ref["S"][b, h] for b, h in pairs])[:, None])
    return g, r


def test_full_size_every_sequence_128_node():
    """The 128-node workload at full size (B=128, H=64): every sequence, two heads
    each (h = b mod 64 and (7b + 3) mod 64), so every head and every residue of the
    launch's block index is checked against the oracle."""
    bt = cfg_batch(5)
    gpu = run_gpu(bt)
    heads = [sorted({b % bt.H, (7 * b + 3) % bt.H}) for b in range(bt.B)]
    ref = oracle_pool.verify_commit(bt, list(zip(range(bt.B), heads)))
    pairs = [(b, h) for b in range(bt.B) for h in heads[b]]
    g, r = _diag(gpu, ref, pairs)
    ok, errs = compare(g, r, bt.dtype)
    assert ok, errs
    assert not gpu["status_v"].any() and not gpu["status_c"].any()


# ------------------------------------------------------------- edge cases

def _custom(parents, accepted, H=2, dk=128, dv=128, mode=synth.GDN, dtype=synth.BF16, seed=0, **kw):
    return synth.make_custom(parents, accepted, H, dk, dv, mode=mode, dtype=dtype, seed=seed, **kw)


@pytest.mark.parametrize("N", [1, 7, 31, 33, 63, 65, 100, 128])
@pytest.mark.parametrize("algo", [MFMA, LEVEL])
def test_ragged_sizes(N, algo):
    rng = np.random.default_rng(N)
    par = _random_parents(rng, 3, N, "random")
    # rows 0, 1: shallow (register path solve); row 2: a 20-node chain at the top
    # so the MFMA kernel falls back to the level solve for that sequence only
    for i in range(1, N):
        par[0, i] = rng.integers(0, min(i, 8))
        par[2, i] = i - 1 if i <= 20 else rng.integers(0, i)
    acc = np.array([N - 1, 0, N // 2], np.int32)
    bt = _custom(par, acc, seed=N)
    gpu = run_gpu(bt, algo=algo)
    ref = run_oracle(bt)
    assert np.array_equal(gpu["path"], ref["path"])
    _check(bt, gpu, ref)


def test_deep_chain_takes_level_solve_inside_mfma_kernel():
    """A 128-node chain has 128-node paths, beyond the register solve."""
    N = 128
    par = np.arange(-1, N - 1, dtype=np.int32)[None].repeat(2, 0)
    bt = _custom(par, np.array([N - 1, 40], np.int32), H=2, seed=5, alpha_range=(0.97, 1.0))
    gpu = run_gpu(bt, algo=MFMA)
    ref = run_oracle(bt)
    assert np.array_equal(gpu["path"], ref["path"])
    _check(bt, gpu, ref)


def test_forest_page4_shape():
    """Three branches straight off S_root, as in the page-4 example, plus a longer one."""
    par = np.array([[-1, 0, -1, -1, 3, 4, -1, 6, 7, 8]], np.int32)
    for dtype, algo, d in [(synth.BF16, MFMA, 128), (synth.F32, LEVEL, 32)]:
        for mode in (synth.GDN, synth.SCALAR_DECAY):
            bt = _custom(par, np.array([5], np.int32), dk=d, dv=d, mode=mode, dtype=dtype,
                         normalize=mode == synth.GDN)
            gpu = run_gpu(bt, algo=algo)
            ref = run_oracle(bt)
            assert gpu["path"][0].tolist()[:3] == [3, 4, 5]
            _check(bt, gpu, ref)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
@pytest.mark.parametrize("mode", [synth.GDN, synth.SCALAR_DECAY])
def test_level_kernel_head_dims(dk, dv, mode):
    rng = np.random.default_rng(dk + dv)
    par = _random_parents(rng, 2, 20, "forest")
    bt = _custom(par, np.array([19, 3], np.int32), H=3, dk=dk, dv=dv, mode=mode,
                 dtype=synth.F32, normalize=mode == synth.GDN)
    gpu = run_gpu(bt, algo=LEVEL)
    ref = run_oracle(bt)
    _check(bt, gpu, ref)


def test_beta_zero_is_pure_decay():
    par = _random_parents(np.random.default_rng(3), 2, 40, "random")
    bt = _custom(par, np.array([39, 10], np.int32))
    bt.beta[:] = 0
    for algo in (MFMA, LEVEL):
        gpu = run_gpu(bt, algo=algo)
        assert np.all(gpu["U"] == 0)
        ref = run_oracle(bt)
        _check(bt, gpu, ref)


def test_scalar_mode_on_matrix_cores():
    par = _random_parents(np.random.default_rng(4), 3, 50, "random")
    for i in range(1, 50):
        par[:, i] = (i - 1) // 3
    bt = _custom(par, np.array([49, 20, 7], np.int32), mode=synth.SCALAR_DECAY, normalize=False,
                 alpha_range=(0.9, 0.99))
    gpu = run_gpu(bt, algo=MFMA)
    ref = run_oracle(bt)
    _check(bt, gpu, ref)
    # scalar mode: U is v exactly
    assert np.array_equal(gpu["U"], np.transpose(bt.v, (0, 2, 1, 3)))


def test_bad_rows_report_status_and_leave_others_exact():
    N = 20
    par = _random_parents(np.random.default_rng(6), 4, N, "random")
    par[1, 5] = 7          # parent after child
    acc = np.array([N - 1, 3, N + 4, -1], np.int32)   # rows 2, 3: accepted out of range
    bt = _custom(par, acc, H=2)
    for algo in (MFMA, LEVEL):
        gpu = run_gpu(bt, algo=algo)
        assert gpu["status_v"].tolist() == [0, 1, 0, 0]
        assert gpu["status_c"].tolist() == [0, 1, 2, 2]
        assert np.all(gpu["path"][1:] == -1)
        good = np.array([True, False, False, False])
        ref = run_oracle(bt)
        assert np.array_equal(gpu["path"][0], ref["path"][0])
        _check(bt, gpu, ref, rows=good)
        # verify outputs of rows with a good tree but a bad accepted index are still right
        okv = np.array([True, False, True, True])
        assert max_rel(gpu["o"][okv], ref["o"][okv], 0, 2) <= TOL[synth.BF16]["o"]
        assert max_rel(gpu["U"][okv], ref["U"][okv], 0, 1) <= TOL[synth.BF16]["U"]


def test_commit_in_place_matches():
    bt = cfg_batch(3)
    a = run_gpu(bt)
    b = run_gpu(bt, inplace=True)
    assert np.array_equal(a["S"], b["S"])


def test_repeat_runs_bitwise_identical():
    bt = cfg_batch(4).select(np.arange(8), np.arange(8))
    a = run_gpu(bt)
    b = run_gpu(bt)
    for key in ("o", "U", "S", "path"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("N", [8, 32, 40, 64, 96, 128])
def test_node_tile_shapes_agree_with_level_solver(N):
    """Each node-count bucket of the matrix-core kernel against the level-scheduled
    kernel and the oracle on the same inputs."""
    rng = np.random.default_rng(100 + N)
    par = _random_parents(rng, 2, N, "random")
    bt = _custom(par, np.array([N - 1, N // 3], np.int32), H=4, seed=N)
    a = run_gpu(bt, algo=MFMA)
    b = run_gpu(bt, algo=LEVEL)
    ref = run_oracle(bt)
    _check(bt, a, ref)
    _check(bt, b, ref)


@pytest.mark.parametrize("cfg,B,H", [(4, 6, 5), (4, 3, 1), (4, 32, 8), (2, 4, 8), (3, 8, 32)])
def test_commit_alone_with_oracle_pseudo_values(cfg, B, H):
    """Feed the oracle's U (rounded to fp32) to the commit kernel: isolates
    tree_commit.  The shapes cover state counts whose row tiles fill whole
    runs of eight XCD groups, a ragged tail of them, and fewer tiles than
    one run, at d = 128 (32-row tiles) and d = 64."""
    import torch

    from tree_speculative_verification_amd import binding as tvb
    bt = cfg_batch(cfg).select(np.arange(B), np.arange(H))
    o_ref, U_ref, _ = oracle.verify(bt.mode, bt.parents, bt.q, bt.k, bt.v, bt.alpha, bt.beta, bt.S_root)
    S_ref, _ = oracle.commit(bt.mode, bt.parents, bt.accepted, bt.k, bt.v, bt.alpha, bt.beta, bt.S_root)
    t = synth.to_torch(bt)
    U = torch.from_numpy(U_ref.astype(np.float32)).cuda()
    S, path, st = tvb.commit(t["k"], t["alpha"], U, t["parents"], t["accepted"], t["S_root"])
    torch.cuda.synchronize()
    assert not st.cpu().numpy().any()
    assert max_rel(S.cpu().numpy(), S_ref, 0, 1) <= 1e-5
