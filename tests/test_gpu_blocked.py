"""Trees beyond 128 nodes and deep trees: the blocked solve (TV_ALGO_BLOCKED), the
commit and the tree index at up to 512 nodes, through the C ABI, against the fp64
oracle on the same seeded inputs."""
import numpy as np
import pytest

import oracle
from parity import TOL, compare, max_rel, run_gpu, run_oracle
from tree_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

AUTO, LEVEL, MFMA, BLOCKED = 0, 1, 2, 3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from tree_speculative_verification_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    torch.cuda.init()


def _chain(n):
    return np.arange(-1, n - 1, dtype=np.int32)


def _random(rng, n, depth, fan, root_fan=0):
    return synth.random_tree(rng, n, max_depth=depth, max_children=fan,
                             first_parent=1 if root_fan else 0,
                             fixed_root_children=root_fan).astype(np.int32)


def _batch(par, H=2, d=128, mode=synth.GDN, dtype=synth.BF16, seed=0, acc=None):
    par = np.atleast_2d(np.asarray(par, np.int32))
    if acc is None:
        acc = np.full(par.shape[0], par.shape[1] - 1, np.int32)
    return synth.make_custom(par, acc, H, d, d, mode=mode, dtype=dtype, seed=seed)


def _check(bt, algo=AUTO, rows=None):
    g = run_gpu(bt, algo=algo)
    r = run_oracle(bt)
    assert np.array_equal(g["path"], r["path"])
    assert np.array_equal(g["status_v"], r["status_v"])
    assert np.array_equal(g["status_c"], r["status_c"])
    ok, errs = compare(g, r, bt.dtype, rows)
    assert ok, errs
    return g, errs


@pytest.mark.parametrize("N", [129, 200, 256, 333, 512])
def test_wide_bf16_matches_oracle(N):
    """Wide random trees past 128 nodes: matrix-core contraction, several chunks,
    ragged last node tile."""
    rng = np.random.default_rng(N)
    par = np.stack([_random(rng, N, 12, 8, root_fan=16) for _ in range(2)])
    _check(_batch(par, seed=N))


def test_wide_workload_sampled():
    """The 512-node workload in the launch shape the benchmark times (B=16, H=32),
    sampled (sequence, head) pairs against the oracle."""
    import torch

    from tree_speculative_verification_amd import binding as tvb
    bt = synth.make_inputs(6)
    t = synth.to_torch(bt)
    o, U, st = tvb.verify(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["parents"],
                          t["S_root"], mode=bt.mode)
    torch.cuda.synchronize()
    assert not st.cpu().numpy().any()
    bs, hs = [0, 7, 15], [0, 19, 31]
    o_ref, U_ref, _ = oracle.verify(bt.mode, bt.parents, bt.q, bt.k, bt.v, bt.alpha, bt.beta,
                                    bt.S_root, heads=hs, seqs=bs)
    sub = np.ix_(bs, hs)
    o_g = o.float().cpu().numpy()[bs][:, :, hs]
    tol = TOL[synth.BF16]
    assert max_rel(U.cpu().numpy()[sub], U_ref[sub], 0, 1) <= tol["U"]
    assert max_rel(o_g, o_ref[bs][:, :, hs], 0, 2) <= tol["o"]


@pytest.mark.parametrize("N", [130, 300, 512])
def test_deep_chain(N):
    """A chain of N nodes: N levels, N(N+1)/2 path entries over many chunks."""
    _check(_batch(np.stack([_chain(N)] * 2), H=1, seed=N))


@pytest.mark.parametrize("N,dtype,d", [(77, synth.BF16, 128), (78, synth.BF16, 128),
                                       (52, synth.F32, 64), (53, synth.F32, 64)])
def test_resident_limit(N, dtype, d):
    """Chains whose N(N+1)/2 path entries sit just inside and just outside what
    LDS holds (3040 entries with bf16 inputs, 1400 with fp32): inside, the
    inverse of I + A is built level by level over the whole chain and each
    column block is one gather; outside, the chunked level solve."""
    par = np.stack([_chain(N), np.full(N, -1, np.int32)])  # a chain, and N lone roots
    _check(_batch(par, H=2, d=d, dtype=dtype, seed=N), algo=BLOCKED)


@pytest.mark.parametrize("N,depth", [(400, 120), (256, 40)])
def test_deep_random(N, depth):
    rng = np.random.default_rng(N + depth)
    par = np.stack([_random(rng, N, depth, 2) for _ in range(2)])
    _check(_batch(par, seed=depth))


@pytest.mark.parametrize("N", [1, 8, 40, 64, 100, 128])
@pytest.mark.parametrize("kind", ["random", "chain"])
def test_blocked_on_small_trees(N, kind):
    """Forced onto trees the other kernels take: same results as the oracle and
    as the matrix-core path."""
    rng = np.random.default_rng(N)
    par = np.stack([_chain(N) if kind == "chain" else _random(rng, N, 8, 4) for _ in range(2)])
    bt = _batch(par, seed=N + 1)
    g, _ = _check(bt, algo=BLOCKED)
    g2 = run_gpu(bt, algo=MFMA)
    assert max_rel(g["U"], g2["U"], 0, 1) <= 1e-3
    assert max_rel(g["o"], g2["o"], 0, 2) <= 2e-2


def test_scalar_decay_bf16():
    rng = np.random.default_rng(5)
    par = np.stack([_random(rng, 300, 10, 6, root_fan=8) for _ in range(2)])
    _check(_batch(par, mode=synth.SCALAR_DECAY, seed=5))


@pytest.mark.parametrize("d,dtype,mode", [(64, synth.F32, synth.GDN), (16, synth.F32, synth.GDN),
                                          (32, synth.BF16, synth.GDN),
                                          (128, synth.F32, synth.SCALAR_DECAY)])
def test_other_shapes(d, dtype, mode):
    """fp32 FMA contraction and generic Gram dots (fp32, or d != 128)."""
    rng = np.random.default_rng(d + dtype)
    par = np.stack([_random(rng, 180, 9, 5, root_fan=4), _chain(180)])
    _check(_batch(par, d=d, dtype=dtype, mode=mode, seed=d))


def test_bad_rows():
    """Bad parents (status 1) and a bad accepted index (status 2) in a 300-node
    batch; the good rows are still within tolerance."""
    rng = np.random.default_rng(9)
    good = _random(rng, 300, 10, 6, root_fan=8)
    bad = good.copy()
    bad[200] = 250                     # parent after the node
    par = np.stack([good, bad, good])
    bt = _batch(par, seed=9, acc=np.array([299, 5, 300], np.int32))
    g = run_gpu(bt)
    r = run_oracle(bt)
    assert list(g["status_v"]) == [0, 1, 0]
    assert list(g["status_c"]) == [0, 1, 2]
    assert np.array_equal(g["path"], r["path"])
    ok, errs = compare(g, r, bt.dtype, rows=np.array([True, False, False]))
    assert ok, errs
    # row 2 verifies fine (only its accepted index is bad)
    assert max_rel(g["o"][[2]], r["o"][[2]], 0, 2) <= TOL[synth.BF16]["o"]


@pytest.mark.parametrize("N", [129, 255, 256, 257, 512])
@pytest.mark.parametrize("kind", ["random", "chain", "forest"])
def test_index_wide_bit_exact(N, kind):
    import torch

    from tree_speculative_verification_amd import binding as tvb
    rng = np.random.default_rng(N + len(kind))
    par = np.full((4, N), -1, np.int32)
    for b in range(4):
        for i in range(1, N):
            if kind == "chain":
                par[b, i] = i - 1
            elif kind == "forest" and rng.random() < 0.2:
                par[b, i] = -1
            else:
                par[b, i] = rng.integers(0, i)
    par[1, N - 1] = N - 1               # self parent: invalid
    par[3, 200 if N > 200 else 100] = -3
    depth, anc, st = tvb.index(torch.from_numpy(par).cuda())
    d_ref, a_ref, s_ref = oracle.tree_index(par)
    assert np.array_equal(st.cpu().numpy(), s_ref)
    assert np.array_equal(depth.cpu().numpy(), d_ref)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), a_ref)


@pytest.mark.parametrize("Np,N", [(300, 64), (64, 300), (512, 512)])
def test_commit_verify_large_trees(Np, N):
    """tree_commit_verify with a tree above 128 nodes runs commit then the blocked
    verification; both against the oracle."""
    import torch

    from tree_speculative_verification_amd import binding as tvb
    rng = np.random.default_rng(Np * 3 + N)
    par_p = np.stack([_random(rng, Np, 12, 8, root_fan=8) for _ in range(2)])
    par_c = np.stack([_random(rng, N, 12, 8, root_fan=8) for _ in range(2)])
    acc = np.array([Np - 1, Np // 2], np.int32)
    prev = _batch(par_p, seed=Np, acc=acc)
    cur = _batch(par_c, seed=N + 7)
    t0, t1 = synth.to_torch(prev), synth.to_torch(cur)
    _, U_prev, _ = tvb.verify(t0["q"], t0["k"], t0["v"], t0["alpha"], t0["beta"], t0["parents"],
                              t0["S_root"], mode=prev.mode)
    S_out, path, cst, o, U, st = tvb.commit_verify(
        t0["k"], t0["alpha"], U_prev, t0["parents"], t0["accepted"], t0["S_root"].clone(),
        t1["q"], t1["k"], t1["v"], t1["alpha"], t1["beta"], t1["parents"], mode=cur.mode)
    torch.cuda.synchronize()
    S_mid, cst_ref = oracle.commit(prev.mode, prev.parents, prev.accepted, prev.k, prev.v,
                                   prev.alpha, prev.beta, prev.S_root)
    path_ref, _ = oracle.accepted_paths(prev.parents, prev.accepted)
    o_ref, U_ref, st_ref = oracle.verify(cur.mode, cur.parents, cur.q, cur.k, cur.v, cur.alpha,
                                         cur.beta, S_mid)
    assert np.array_equal(path.cpu().numpy(), path_ref)
    assert np.array_equal(cst.cpu().numpy(), cst_ref) and np.array_equal(st.cpu().numpy(), st_ref)
    tol = TOL[synth.BF16]
    assert max_rel(S_out.cpu().numpy(), S_mid, 0, 1) <= tol["S"]
    assert max_rel(U.cpu().numpy(), U_ref, 0, 1) <= tol["U"]
    assert max_rel(o.float().cpu().numpy(), o_ref, 0, 2) <= tol["o"]


@pytest.mark.parametrize("kind", ["resident", "chunked"])
def test_repeatable_bit_for_bit(kind):
    """The same inputs twice give bit-identical outputs: every LDS region the
    kernel reuses across phases and column blocks (the staged S block, the R
    rows, the entries, the inverse formed in place) is ordered by its
    barriers, with no race that could change a result between runs."""
    rng = np.random.default_rng(99)
    if kind == "resident":
        par = np.stack([_random(rng, 512, 12, 8, root_fan=32) for _ in range(3)])
    else:
        par = np.stack([_chain(300), _random(rng, 300, 120, 2), _chain(300)])
    bt = _batch(par, H=4, seed=99)
    g1 = run_gpu(bt, algo=BLOCKED)
    g2 = run_gpu(bt, algo=BLOCKED)
    for key in ("o", "U", "S", "path", "status_v"):
        assert np.array_equal(g1[key], g2[key]), key
