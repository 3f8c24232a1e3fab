"""Plausible mistakes planted in a copy of the oracle must each be caught by some pin (CPU only).

Every mutant is applied with monkeypatch to the oracle module for the duration of one test, so
the real oracle is untouched. A mutant that no pin rejects would mean the pins cannot tell that
mistake from the method.
"""
import numpy as np
import pytest

from oracle import gsi_oracle as orc
from tests import oracle_pins

_real = {name: getattr(orc, name) for name in ("residual", "residual_norms", "gate", "project",
                                              "precompute_image", "forward", "spectral_norm",
                                              "static_projection", "dense")}


def m_residual_sign(V, X, G=None):
    V = orc.as_f64(V); X = np.atleast_2d(orc.as_f64(X))
    G = _real["project"](V, X) if G is None else G
    return X + G @ V.T


def m_pythagorean(V, X, G=None):
    X = np.atleast_2d(orc.as_f64(X))
    G = _real["project"](V, X) if G is None else G
    return np.einsum("ti,ti->t", X, X) - np.einsum("tj,tj->t", G, G)


def m_gate_ties_fast(nr2, nx2, eps):
    return np.where(np.asarray(nr2) <= eps * eps * np.asarray(nx2), orc.FAST, orc.SLOW).astype(np.uint8)


def m_gate_inverted(nr2, nx2, eps):
    return (1 - _real["gate"](nr2, nx2, eps)).astype(np.uint8)


def m_gate_eps_not_squared(nr2, nx2, eps):
    return np.where(np.asarray(nr2) < eps * np.asarray(nx2), orc.FAST, orc.SLOW).astype(np.uint8)


def m_project_dropped_column(V, X):
    G = _real["project"](V, X)
    G[:, -1:] = 0.0
    return G


def m_project_reversed(V, X):
    return _real["project"](V, X)[:, ::-1]


def m_image_dropped_term(W, V):
    M = _real["precompute_image"](W, V)
    if M.shape[1] > 1:
        M[:, 0] = 0.0
    return M


def m_image_transposed_basis(W, V):
    W = orc.as_f64(W); V = orc.as_f64(V)
    return W @ V[::-1, :]


def m_forward_always_fast(W, V, X, eps, M=None):
    return _real["forward"](W, V, X, np.inf, M=M)


def m_forward_slow_uses_image(W, V, X, eps, M=None):
    out = _real["forward"](W, V, X, eps, M=M)
    Wf = orc.as_f64(W); Vf = orc.as_f64(V)
    Mf = Wf @ Vf if M is None else orc.as_f64(M)
    slow = out["gate"] == orc.SLOW
    out["y"][slow] = out["g"][slow] @ Mf.T
    return out


def m_forward_scaled(W, V, X, eps, M=None):
    out = _real["forward"](W, V, X, eps, M=M)
    fast = out["gate"] == orc.FAST
    out["y"][fast] *= 1.0 + 1e-6
    return out


def m_spectral_squared(W, **kw):
    return _real["spectral_norm"](W, **kw) ** 2


def m_static_is_dense(W, V, X, M=None):
    out = _real["static_projection"](W, V, X, M=M)
    out["y"] = _real["dense"](W, X)
    return out


def m_static_drops_column(W, V, X, M=None):
    Vf = orc.as_f64(V).copy()
    Vf[:, -1] = 0.0
    return _real["static_projection"](W, Vf, X, M=M)


def m_dense_drops_column(W, X):
    Xf = np.atleast_2d(orc.as_f64(X)).copy()
    Xf[:, -1] = 0.0
    return _real["dense"](W, Xf)


def m_dense_rounded(W, X):
    return _real["dense"](W, X) * (1.0 + 1e-9)


MUTANTS = {
    "static_is_dense": ("static_projection", m_static_is_dense),
    "static_drops_column": ("static_projection", m_static_drops_column),
    "dense_drops_column": ("dense", m_dense_drops_column),
    "dense_scaled": ("dense", m_dense_rounded),
    "residual_sign": ("residual", m_residual_sign),
    "pythagorean_shortcut": ("residual_norms", m_pythagorean),
    "gate_ties_fast": ("gate", m_gate_ties_fast),
    "gate_inverted": ("gate", m_gate_inverted),
    "gate_eps_not_squared": ("gate", m_gate_eps_not_squared),
    "project_dropped_column": ("project", m_project_dropped_column),
    "project_reversed": ("project", m_project_reversed),
    "image_dropped_term": ("precompute_image", m_image_dropped_term),
    "image_transposed_basis": ("precompute_image", m_image_transposed_basis),
    "forward_always_fast": ("forward", m_forward_always_fast),
    "forward_slow_uses_image": ("forward", m_forward_slow_uses_image),
    "forward_fast_scaled": ("forward", m_forward_scaled),
    "spectral_norm_squared": ("spectral_norm", m_spectral_squared),
}


def test_real_oracle_passes_every_pin():
    assert oracle_pins.failing_pins(orc) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = oracle_pins.failing_pins(orc)
    assert caught, f"mutant {name} passed every pin"
