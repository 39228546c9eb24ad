"""tree_attention (tree-masked full attention with a committed cache) through the
C ABI, against the fp64 oracle on the same seeded inputs."""
import numpy as np
import pytest

from oracle import tree_attention as A
from parity import max_rel
from tree_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

TOL_O = 2e-2   # bf16 q/k/v/o, as the verification outputs


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from tree_speculative_verification_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    torch.cuda.init()


def _run(bt, prefix_len=None, null_cache=False):
    import torch

    from tree_speculative_verification_amd import binding as tvb
    t = synth.attention_to_torch(bt)
    if prefix_len is not None:
        t["prefix_len"] = torch.tensor(prefix_len, dtype=torch.int32, device="cuda")
    o, st = tvb.attention(t["q"], t["k_cache"], t["v_cache"], t["prefix_len"], t["k_tree"],
                          t["v_tree"], t["parents"], t["scale"])
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), st.cpu().numpy()


def _check(bt, o, seqs=None, heads=None, plen=None):
    ref, st = A.tree_attention(bt.parents, bt.q, bt.k_cache, bt.v_cache,
                               bt.prefix_len if plen is None else plen, bt.k_tree, bt.v_tree,
                               bt.scale, seqs=seqs, heads=heads)
    bs = np.arange(bt.q.shape[0]) if seqs is None else np.asarray(seqs)
    hs = np.arange(bt.q.shape[2]) if heads is None else np.asarray(heads)
    err = max_rel(o[bs][:, :, hs], ref[bs][:, :, hs], 0, 2)
    assert err <= TOL_O, err
    return err, st


def _rand_tree(rng, N, depth=8, fan=4):
    return synth.random_tree(rng, N, max_depth=depth, max_children=fan).astype(np.int32)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 2), (4, 4), (16, 2)])
def test_small_matches_oracle(Hq, Hkv):
    """Group sizes 4, 3, 1 and 8; ragged prefixes including 0 and P_max."""
    rng = np.random.default_rng(Hq * 10 + Hkv)
    par = np.stack([_rand_tree(rng, 17) for _ in range(3)])
    bt = synth.make_attention_inputs(seed=Hq + Hkv, B=3, N=17, Hq=Hq, Hkv=Hkv, P_max=100,
                                     parents=par, prefix_len=np.array([0, 37, 100]))
    o, st = _run(bt)
    assert not st.any()
    _check(bt, o)


@pytest.mark.parametrize("kind", ["chain", "star", "forest"])
def test_tree_shapes(kind):
    N = 64
    rng = np.random.default_rng(len(kind))
    if kind == "chain":
        par = np.arange(-1, N - 1, dtype=np.int32)
    elif kind == "star":
        par = np.zeros(N, np.int32)
        par[0] = -1
    else:
        par = _rand_tree(rng, N)
        par[rng.random(N) < 0.2] = -1
    bt = synth.make_attention_inputs(seed=3, B=2, N=N, Hq=8, Hkv=2, P_max=70,
                                     parents=np.stack([par, par]), prefix_len=np.array([70, 5]))
    o, _ = _run(bt)
    _check(bt, o)


@pytest.mark.parametrize("N", [1, 31, 129, 300, 512])
def test_sizes_and_ragged_row_blocks(N):
    """Node counts that leave ragged 32-row tiles and 128-row blocks; trees past
    128 nodes (ancestor words beyond the fourth), up to the largest tree."""
    rng = np.random.default_rng(N)
    par = np.stack([_rand_tree(rng, N, depth=40, fan=3) for _ in range(2)])
    bt = synth.make_attention_inputs(seed=N, B=2, N=N, Hq=12, Hkv=4, P_max=64, parents=par,
                                     prefix_len=np.array([64, 33]))
    o, _ = _run(bt)
    _check(bt, o)


def test_largest_chain():
    """A 512-node chain: the last node sees all 16 tree tiles and its query
    block spans the last ancestor words."""
    N = 512
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (2, 1))
    bt = synth.make_attention_inputs(seed=5, B=2, N=N, Hq=8, Hkv=4, P_max=96, parents=par,
                                     prefix_len=np.array([96, 0]))
    o, st = _run(bt)
    assert not st.any()
    _check(bt, o)


def test_no_cache():
    """P_max = 0: only the tree (caches of zero length)."""
    rng = np.random.default_rng(11)
    par = np.stack([_rand_tree(rng, 20) for _ in range(2)])
    bt = synth.make_attention_inputs(seed=11, B=2, N=20, Hq=4, Hkv=2, P_max=0, parents=par,
                                     prefix_len=np.array([0, 0]))
    o, _ = _run(bt)
    _check(bt, o)


def test_sharp_softmax():
    """Scores of several hundred: the running maximum must rescale correctly."""
    rng = np.random.default_rng(12)
    par = np.stack([_rand_tree(rng, 40) for _ in range(2)])
    bt = synth.make_attention_inputs(seed=12, B=2, N=40, Hq=4, Hkv=1, P_max=200, parents=par,
                                     prefix_len=np.array([200, 150]))
    bt.scale = 4.0
    o, _ = _run(bt)
    _check(bt, o)


def test_bad_rows():
    """Bad parents (status 1) and a prefix length past P_max (status 3, clamped);
    the clamped row still matches the oracle at the clamped length."""
    rng = np.random.default_rng(13)
    good = _rand_tree(rng, 12)
    bad = good.copy()
    bad[7] = 9
    bt = synth.make_attention_inputs(seed=13, B=3, N=12, Hq=4, Hkv=2, P_max=40,
                                     parents=np.stack([good, bad, good]),
                                     prefix_len=np.array([40, 10, 10]))
    o, st = _run(bt, prefix_len=[40, 10, 55])
    assert list(st) == [0, 1, 3]
    _check(bt.__class__(**{**bt.__dict__}), o, seqs=[0, 2], plen=np.array([40, 10, 40]))


def test_workload_sampled():
    """The attention workload at full size (B=32, N=64, Hq=32, Hkv=8, prefixes
    of 2048-4096), sampled (sequence, head) pairs against the oracle."""
    bt = synth.make_attention_inputs()
    o, st = _run(bt)
    assert not st.any()
    _check(bt, o, seqs=[0, 17, 31], heads=[0, 5, 31])


def test_repeatable_bit_for_bit():
    """The same inputs twice give bit-identical outputs (the double-buffered
    key/value tiles are ordered by their barriers)."""
    rng = np.random.default_rng(21)
    par = np.stack([_rand_tree(rng, 100) for _ in range(2)])
    bt = synth.make_attention_inputs(seed=21, B=2, N=100, Hq=8, Hkv=2, P_max=700, parents=par,
                                     prefix_len=np.array([700, 389]))
    o1, s1 = _run(bt)
    o2, s2 = _run(bt)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_one_round_pairing_every_output():
    """A grid of exactly 512 workgroups (64 sequences x 8 key/value heads x 1
    query block) takes the ordering that pairs long and short prefixes on a
    CU: every output checked, with prefix lengths that tie, reach 0 and
    reach P_max."""
    rng = np.random.default_rng(31)
    B, N = 64, 16
    par = np.stack([_rand_tree(rng, N) for _ in range(B)])
    plen = rng.integers(0, 97, size=B)
    plen[:6] = [0, 96, 96, 40, 40, 40]
    bt = synth.make_attention_inputs(seed=31, B=B, N=N, Hq=8, Hkv=8, P_max=96, parents=par,
                                     prefix_len=plen)
    o, st = _run(bt)
    assert not st.any()
    _check(bt, o)


@pytest.mark.parametrize("B,Hkv,N,Hq", [
    (48, 8, 16, 8),    # 384 workgroups, one round: some CUs run one, some a pair
    (8, 8, 16, 8),     # 64 workgroups, fewer than the CUs
    (36, 4, 70, 8),    # 288 workgroups of two query blocks each
    (128, 8, 16, 8),   # 1024 workgroups, several rounds: heaviest first
    (40, 2, 200, 8),   # 560 workgroups of seven query blocks each
    (260, 1, 8, 2),    # more sequences than the in-kernel ranking holds: plain order
])
def test_work_order_every_output(B, Hkv, N, Hq):
    """Grids on every branch of the work order (one round with and without
    pairs, several rounds, unranked): every output checked, with prefix
    lengths that tie, reach 0 and reach P_max."""
    rng = np.random.default_rng(B + N)
    par = np.stack([_rand_tree(rng, N) for _ in range(B)])
    plen = rng.integers(0, 97, size=B)
    plen[:6] = [0, 96, 96, 40, 40, 40]
    bt = synth.make_attention_inputs(seed=B, B=B, N=N, Hq=Hq, Hkv=Hkv, P_max=96, parents=par,
                                     prefix_len=plen)
    o, st = _run(bt)
    assert not st.any()
    _check(bt, o)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_scale_sign_and_zero(scale):
    """A negative scale (applied with q negated), a zero scale (every visible
    key weighted alike) and a large one, against the oracle."""
    rng = np.random.default_rng(41)
    par = np.stack([_rand_tree(rng, 40) for _ in range(3)])
    bt = synth.make_attention_inputs(seed=41, B=3, N=40, Hq=8, Hkv=2, P_max=80, parents=par,
                                     prefix_len=np.array([80, 33, 0]))
    bt = bt.__class__(**{**bt.__dict__, "scale": scale})
    o, st = _run(bt)
    assert not st.any()
    _check(bt, o)
