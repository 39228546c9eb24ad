"""The tree-attention oracle against its pins, and plausible mistakes planted in it
(on the CPU) that some pin must catch."""
import numpy as np
import pytest

import oracle_pins_attention as P
from oracle import tree_attention as A
from oracle import tree_oracle as T


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


_attend = A.softmax_attend
_visible = A.visible_keys


def m_no_scale(q, K, V, scale):
    return _attend(q, K, V, 1.0)


def m_unnormalized(q, K, V, scale):
    s = scale * (np.asarray(K, float) @ np.asarray(q, float))
    return np.exp(s - s.max()) @ np.asarray(V, float)


def m_keys_as_values(q, K, V, scale):
    return _attend(q, K, K, scale)


def m_drop_prefix(b, n, kvh, parents_b, kc, vc, plen, kt, vt):
    return _visible(b, n, kvh, parents_b, kc, vc, np.zeros_like(plen), kt, vt)


def m_prefix_one_long(b, n, kvh, parents_b, kc, vc, plen, kt, vt):
    return _visible(b, n, kvh, parents_b, kc, vc, np.minimum(np.asarray(plen) + 1, kc.shape[2]), kt, vt)


def m_path_without_self(b, n, kvh, parents_b, kc, vc, plen, kt, vt):
    K, V = _visible(b, n, kvh, parents_b, kc, vc, plen, kt, vt)
    return (K[:-1], V[:-1]) if len(K) > 1 else (K, V)


def m_whole_tree(b, n, kvh, parents_b, kc, vc, plen, kt, vt):
    P_ = int(plen[b])
    return (np.concatenate([kc[b, kvh, :P_], kt[b, :, kvh]]),
            np.concatenate([vc[b, kvh, :P_], vt[b, :, kvh]]))


def m_parent_path(b, n, kvh, parents_b, kc, vc, plen, kt, vt):
    p = int(parents_b[n])
    return _visible(b, p if p >= 0 else n, kvh, parents_b, kc, vc, plen, kt, vt)


ATTEND_MUTANTS = [m_no_scale, m_unnormalized, m_keys_as_values]
VISIBLE_MUTANTS = [m_drop_prefix, m_prefix_one_long, m_path_without_self, m_whole_tree, m_parent_path]


def _caught():
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception:  # AssertionError, or a shape error the mistake causes
            return True
    return False


@pytest.mark.parametrize("mutant", ATTEND_MUTANTS, ids=lambda f: f.__name__)
def test_attend_mutant_caught(monkeypatch, mutant):
    monkeypatch.setattr(A, "softmax_attend", mutant)
    assert _caught()


@pytest.mark.parametrize("mutant", VISIBLE_MUTANTS, ids=lambda f: f.__name__)
def test_visible_mutant_caught(monkeypatch, mutant):
    monkeypatch.setattr(A, "visible_keys", mutant)
    assert _caught()


def test_wrong_group_caught(monkeypatch):
    """Query head hq read from key/value head hq % Hkv instead of hq // G."""
    def tree_attention(parents, q, kc, vc, plen, kt, vt, scale, seqs=None, heads=None):
        B, N, Hq, D = q.shape
        Hkv = kc.shape[1]
        o = np.zeros((B, N, Hq, vc.shape[3]))
        st = np.zeros(B, np.int32)
        for b in range(B):
            if not T.parents_valid(parents[b]):
                st[b] = 1
                continue
            for n in range(N):
                for hq in range(Hq):
                    K, V = A.visible_keys(b, n, hq % Hkv, parents[b], kc, vc, plen, kt, vt)
                    o[b, n, hq] = A.softmax_attend(q[b, n, hq], K, V, scale)
        return o, st
    monkeypatch.setattr(A, "tree_attention", tree_attention)
    assert _caught()


def test_unmutated_passes():
    assert not _caught()
