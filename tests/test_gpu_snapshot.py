"""Per-node-snapshot baseline kernels (through the C ABI) against the fp64 oracle.

The oracle's per-node states are its token-by-token path walk (pinned against
the explicit commit walk in the oracle pins), so the snapshots, the outputs and
the committed state are all checked against the same definition as the
tree-structured path.
"""
import numpy as np
import pytest

import oracle
from parity import TOL, max_rel
from tree_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from tree_speculative_verification_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    torch.cuda.init()


def _run(bt):
    import torch

    from tree_speculative_verification_amd import binding as tvb
    t = synth.to_torch(bt, "cuda")
    o, snaps, st_v = tvb.verify_snapshot(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                                         t["parents"], t["S_root"], mode=bt.mode)
    S, path, st_c = tvb.commit_snapshot(snaps, t["parents"], t["accepted"])
    torch.cuda.synchronize()
    return dict(o=o.float().cpu().numpy(), snaps=snaps.cpu().numpy(), S=S.cpu().numpy(),
                path=path.cpu().numpy(), st_v=st_v.cpu().numpy(), st_c=st_c.cpu().numpy())


def _reference(bt, bs=None, hs=None):
    """Oracle o, per-node states and committed states for sequences bs x heads hs."""
    bs = range(bt.B) if bs is None else bs
    hs = range(bt.H) if hs is None else hs
    o = np.zeros((len(bs), bt.N, len(hs), bt.dv))
    st = np.zeros((len(bs), len(hs), bt.N, bt.dk, bt.dv))
    for i, b in enumerate(bs):
        for j, h in enumerate(hs):
            ob, _, sb = oracle.verify_head(bt.mode, bt.parents[b], bt.q[b, :, h], bt.k[b, :, h],
                                           bt.v[b, :, h], bt.alpha[b, :, h],
                                           None if bt.beta is None else bt.beta[b, :, h],
                                           bt.S_root[b, h])
            o[i, :, j] = ob
            st[i, j] = sb
    return o, st


def _check(bt, g, bs=None, hs=None):
    bsl = slice(None) if bs is None else bs
    o_ref, st_ref = _reference(bt, bs, hs)
    go = g["o"][bsl] if hs is None else g["o"][bsl][:, :, hs]
    gs = g["snaps"][bsl] if hs is None else g["snaps"][bsl][:, hs]
    tol = TOL[bt.dtype]
    assert max_rel(go, o_ref, 0, 2) <= tol["o"]
    # every node's snapshot, held to the state tolerance
    assert max_rel(gs, st_ref, 0, 1) <= tol["S"]
    # the commit is the accepted node's snapshot, bit for bit
    acc = bt.accepted[bsl] if bs is not None else bt.accepted
    for i in range(gs.shape[0]):
        for j in range(gs.shape[1]):
            b = i if bs is None else bs[i]
            h = j if hs is None else hs[j]
            assert np.array_equal(g["S"][b, h], g["snaps"][b, h, int(acc[i])])
    path_ref, st = oracle.accepted_paths(bt.parents, bt.accepted)
    assert np.array_equal(g["path"], path_ref)
    assert np.array_equal(g["st_c"], st)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_snapshot_small_configs(cfg):
    bt = synth.make_inputs(cfg)
    g = _run(bt)
    assert not g["st_v"].any()
    _check(bt, g)


def test_snapshot_64_node_tree_sampled():
    """The 64-node workload at a reduced batch (the full one needs 4.3 GB of snapshots)."""
    bt = synth.make_inputs(4, B=4, H=4)
    g = _run(bt)
    assert not g["st_v"].any()
    _check(bt, g, bs=np.array([0, 3]), hs=np.array([1, 2]))


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 16)])
def test_snapshot_head_dims(dk, dv):
    rng = np.random.default_rng(dk + dv)
    N = 12
    par = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, N)]], np.int32)
    bt = synth.make_custom(par, np.array([N - 1], np.int32), 3, dk, dv, mode=synth.GDN,
                           dtype=synth.F32, seed=5)
    g = _run(bt)
    _check(bt, g)


def test_snapshot_matches_tree_path():
    """Same outputs as tree_verify on the same inputs (both within tolerance of each other)."""
    import torch

    from tree_speculative_verification_amd import binding as tvb
    bt = synth.make_inputs(4, B=2, H=8)
    t = synth.to_torch(bt, "cuda")
    o1, _, _ = tvb.verify(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["parents"], t["S_root"],
                          mode=bt.mode)
    o2, _, _ = tvb.verify_snapshot(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["parents"],
                                   t["S_root"], mode=bt.mode)
    torch.cuda.synchronize()
    assert max_rel(o1.float().cpu().numpy(), o2.float().cpu().numpy(), 0, 2) <= 2e-2


def test_snapshot_bad_rows():
    par = np.array([[-1, 0, 1, 2], [-1, 0, 3, 1], [-1, 0, 0, 1], [-1, -1, 1, 2]], np.int32)
    acc = np.array([3, 2, 7, -1], np.int32)
    bt = synth.make_custom(par, acc, 2, 16, 16, mode=synth.GDN, dtype=synth.F32, seed=3)
    g = _run(bt)
    assert list(g["st_v"]) == [0, 1, 0, 0]
    assert list(g["st_c"]) == [0, 1, 2, 2]
    assert (g["path"][1] == -1).all() and (g["path"][2] == -1).all() and (g["path"][3] == -1).all()
    ok = np.array([0])
    _check(bt.select(ok, np.arange(2)), dict(o=g["o"][ok], snaps=g["snaps"][ok], S=g["S"][ok],
                                              path=g["path"][ok], st_c=g["st_c"][ok]))
