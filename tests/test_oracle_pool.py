"""The worker-pool runner of the oracle gives the same arrays as the plain calls."""
import numpy as np

import oracle_pool
from parity import run_oracle
from tree_speculative_verification_amd import synth


def test_pool_matches_plain_oracle():
    bt = synth.make_inputs(4, B=5, H=3)
    pairs = [(b, [0, 1, 2]) for b in range(bt.B)]
    got = oracle_pool.verify_commit(bt, pairs)
    ref = run_oracle(bt)
    for key in ("o", "U", "S", "status_v", "status_c"):
        assert np.array_equal(got[key], ref[key]), key


def test_pool_commit_then_verify_and_partial_heads():
    prev = synth.make_inputs(4, B=3, H=4)
    cur = synth.make_inputs(4, seed=104, B=3, H=4)
    got = oracle_pool.commit_then_verify(prev, cur, [(0, [1]), (1, [0, 3]), (2, [2])])
    import oracle
    S_mid, _ = oracle.commit(prev.mode, prev.parents, prev.accepted, prev.k, prev.v, prev.alpha,
                             prev.beta, prev.S_root)
    o, U, _ = oracle.verify(cur.mode, cur.parents, cur.q, cur.k, cur.v, cur.alpha, cur.beta, S_mid)
    for b, hs in [(0, [1]), (1, [0, 3]), (2, [2])]:
        assert np.array_equal(got["S"][b, hs], S_mid[b, hs])
        assert np.array_equal(got["o"][b][:, hs], o[b][:, hs])
        assert np.array_equal(got["U"][b, hs], U[b, hs])
    assert not got["S"][0, 0].any()   # heads not asked for stay zero
