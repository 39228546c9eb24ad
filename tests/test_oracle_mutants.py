"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

A pin suite that lets a dropped term, a flipped sign, a transposed operand or an
off-by-one path through would not be pinning anything.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import tree_oracle as T

_gdn = T.gdn_step
_scalar = T.scalar_step
_path = T.node_path


def m_drop_beta_write(S, k, v, a, b):
    kS = k @ S
    return a * (S - b * np.outer(k, kS)) + np.outer(k, v), b * (v - a * kS)


def m_sign_flip(S, k, v, a, b):
    kS = k @ S
    return a * (S + b * np.outer(k, kS)) + b * np.outer(k, v), b * (v - a * kS)


def m_transposed(S, k, v, a, b):
    kS = S @ k
    return a * (S - b * np.outer(k, kS)) + b * np.outer(k, v), b * (v - a * kS)


def m_decay_after_write(S, k, v, a, b):
    kS = k @ S
    return a * (S - b * np.outer(k, kS) + b * np.outer(k, v)), b * (v - a * kS)


def m_u_without_alpha(S, k, v, a, b):
    kS = k @ S
    return a * (S - b * np.outer(k, kS)) + b * np.outer(k, v), b * (v - kS)


def m_u_without_beta(S, k, v, a, b):
    kS = k @ S
    return a * (S - b * np.outer(k, kS)) + b * np.outer(k, v), (v - a * kS)


def m_scalar_no_decay(S, k, v, a):
    return S + np.outer(k, v), v.copy()


def m_scalar_outer_swapped(S, k, v, a):
    return a * S + np.outer(v, k), v.copy()


def m_scalar_decay_write(S, k, v, a):
    return a * (S + np.outer(k, v)), v.copy()


def m_path_without_self(par, n):
    return _path(par, n)[:-1] or [int(n)]


def m_path_skips_grandparent(par, n):
    path = _path(par, n)
    return path[:-3] + path[-2:] if len(path) >= 3 else path


def m_path_duplicate_root(par, n):
    path = _path(par, n)
    return [path[0]] + path


GDN_MUTANTS = [m_drop_beta_write, m_sign_flip, m_transposed, m_decay_after_write,
               m_u_without_alpha, m_u_without_beta]
SCALAR_MUTANTS = [m_scalar_no_decay, m_scalar_outer_swapped, m_scalar_decay_write]
PATH_MUTANTS = [m_path_without_self, m_path_skips_grandparent, m_path_duplicate_root]


def _caught():
    """True when some pin fails its assertion.  Any other exception (a shape
    error on a non-square state, say) is not a catch: such a pin is skipped and
    the next one must find the mistake by its values."""
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            return True
        except Exception:  # noqa: BLE001  (crash, not a value check)
            continue
    return False


@pytest.mark.parametrize("mutant", GDN_MUTANTS, ids=lambda f: f.__name__)
def test_gdn_mutant_caught(monkeypatch, mutant):
    monkeypatch.setattr(T, "gdn_step", mutant)
    assert _caught()


@pytest.mark.parametrize("mutant", SCALAR_MUTANTS, ids=lambda f: f.__name__)
def test_scalar_mutant_caught(monkeypatch, mutant):
    monkeypatch.setattr(T, "scalar_step", mutant)
    assert _caught()


@pytest.mark.parametrize("mutant", PATH_MUTANTS, ids=lambda f: f.__name__)
def test_path_mutant_caught(monkeypatch, mutant):
    monkeypatch.setattr(T, "node_path", mutant)
    assert _caught()


def test_parent_state_output_caught(monkeypatch):
    """Reading o_n from the parent's state instead of node n's own state."""
    def verify_head(mode, parents_b, q, k, v, alpha, beta, S_root):
        N = len(parents_b)
        S_root = np.asarray(S_root, dtype=np.float64)
        states = np.zeros((N,) + S_root.shape)
        o = np.zeros((N, S_root.shape[1]))
        U = np.zeros((N, S_root.shape[1]))
        for n in range(N):
            p = int(parents_b[n])
            Sp = S_root if p < 0 else states[p]
            b_n = 0.0 if beta is None else float(beta[n])
            states[n], U[n] = T._step(mode, Sp, np.asarray(k[n], float), np.asarray(v[n], float),
                                      float(alpha[n]), b_n)
            o[n] = Sp.T @ np.asarray(q[n], float)
        return o, U, states
    monkeypatch.setattr(T, "verify_head", verify_head)
    assert _caught()


def test_unmutated_passes():
    assert not _caught()
