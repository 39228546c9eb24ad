"""The seeded input generator: determinism, tree shapes and acceptance rules per workload."""
import numpy as np
import pytest

from tree_speculative_verification_amd import synth


def _depths(par):
    d = np.zeros(len(par), int)
    for i, p in enumerate(par):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_deterministic(cfg):
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg)
    for f in ("parents", "accepted", "q", "k", "v", "alpha", "S_root"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = synth.make_inputs(cfg, seed=99)
    assert not np.array_equal(a.q, c.q)


def test_shapes_and_trees():
    for cfg, spec in synth.CONFIGS.items():
        if cfg >= 5:
            bt = synth.make_inputs(cfg, B=4, H=2)
            B, H = 4, 2
        else:
            bt = synth.make_inputs(cfg)
            B, H = spec["B"], spec["H"]
        N, d = spec["N"], spec["d"]
        assert bt.q.shape == (B, N, H, d) and bt.v.shape == (B, N, H, d)
        assert bt.S_root.shape == (B, H, d, d) and bt.alpha.shape == (B, N, H)
        assert (bt.beta is None) == (spec["mode"] == synth.SCALAR_DECAY)
        for b in range(B):
            par = bt.parents[b]
            assert par[0] == -1 and all(-1 <= p < i for i, p in enumerate(par))
            dep = _depths(par)
            kids = np.bincount(par[par >= 0], minlength=N)
            a = bt.accepted[b]
            assert 0 <= a < N
            if cfg == 1:
                assert par.tolist() == [-1, 0, 0, 1, 1, 2, 3] and a == 6
            if cfg == 2:
                assert dep.max() <= 5
                assert a == np.flatnonzero(dep == dep.max())[0]
            if cfg == 3:
                assert par.tolist() == list(range(-1, N - 1))
            if cfg == 4:
                assert dep.max() <= 8 and kids.max() <= 4
            if cfg == 5:
                assert kids[0] == 16 and list(par[1:17]) == [0] * 16
                assert dep.max() <= 10 and kids[1:].max() <= 8
                assert kids[a] == 0   # a leaf
            if cfg == 6:
                assert kids[0] == 32 and list(par[1:33]) == [0] * 32
                assert dep.max() <= 12 and kids[1:].max() <= 8
                assert kids[a] == 0
        if spec["dtype"] == synth.BF16:
            for x in (bt.q, bt.k, bt.v):
                assert not np.any(x.view(np.uint32) & 0xFFFF)
        if spec["mode"] == synth.GDN:
            nk = np.linalg.norm(bt.k.astype(np.float64), axis=-1)
            assert np.all(np.abs(nk - 1) < 1e-2)
            assert np.all(bt.alpha > 0) and np.all(bt.alpha <= 1)
            assert np.all(bt.beta >= 0) and np.all(bt.beta <= 1)


def test_round_bf16_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8)], np.float32)
    assert synth.round_bf16(x).tolist() == [1.0, 1.0 + 2 ** -6, 1.0, -1.0]
