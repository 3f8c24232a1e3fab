"""Plausible mistakes planted in a copy of the calibration oracle must each be caught by some
calibration pin (CPU only). Each mutant replaces one function of the module for one test."""
import math

import numpy as np
import pytest

from oracle import gsi_calibration as cal
from tests import calibration_pins

_real = {n: getattr(cal, n) for n in ("dgks_orthonormalize", "subspace_iteration", "calibrate_cascade",
                                     "exact_subspace", "principal_sines")}


def _gs(Y, passes, proj_against_y=False, normalise=True, inverted=False):
    Y = cal.as_f64(Y)
    d, k = Y.shape
    Q = np.zeros((d, k))
    twice = np.zeros(k, dtype=bool)
    for j in range(k):
        P = Y[:, :j] if proj_against_y else Q[:, :j]
        v = Y[:, j].copy()
        before = float(v @ v)
        v = v - P @ (P.T @ v)
        after = float(v @ v)
        need = after >= 0.5 * before if inverted else after < 0.5 * before
        if passes == 2 and need:
            twice[j] = True
            v = v - P @ (P.T @ v)
            after = float(v @ v)
        Q[:, j] = v / math.sqrt(after) if normalise else v
    return Q, twice


def m_single_pass(Y, eta=cal.DGKS_ETA):
    return _gs(Y, 1)


def m_project_against_inputs(Y, eta=cal.DGKS_ETA):
    return _gs(Y, 2, proj_against_y=True)


def m_no_normalise(Y, eta=cal.DGKS_ETA):
    return _gs(Y, 2, normalise=False)


def m_dgks_inverted(Y, eta=cal.DGKS_ETA):
    return _gs(Y, 2, inverted=True)


def m_no_product(A, Q0, n_iter):
    Q = cal.as_f64(Q0)
    for _ in range(n_iter):
        Q, _ = _real["dgks_orthonormalize"](Q)
    return Q


def m_shifted_product(A, Q0, n_iter):
    """Iterates with A^T A + c I (c the mean eigenvalue): same eigenvectors, slower convergence."""
    A = cal.as_f64(A)
    Q = cal.as_f64(Q0)
    c = float(np.sum(A * A)) / A.shape[1]
    for _ in range(n_iter):
        Q, _ = _real["dgks_orthonormalize"](A.T @ (A @ Q) + c * Q)
    return Q


def m_cascade_cold_every_layer(As, Omega, n_cold, n_warm):
    return [_real["subspace_iteration"](A, Omega, n_cold if i == 0 else n_warm) for i, A in enumerate(As)]


def m_trailing_eigenvectors(A, k):
    A = cal.as_f64(A)
    w, U = np.linalg.eigh(A.T @ A)
    return U[:, np.argsort(w)[:k]]


def m_cosines(U, V):
    s = np.linalg.svd(cal.as_f64(U).T @ cal.as_f64(V), compute_uv=False)
    return np.sort(s)[::-1]


MUTANTS = [
    ("dgks_orthonormalize", m_single_pass),
    ("dgks_orthonormalize", m_project_against_inputs),
    ("dgks_orthonormalize", m_no_normalise),
    ("dgks_orthonormalize", m_dgks_inverted),
    ("subspace_iteration", m_no_product),
    ("subspace_iteration", m_shifted_product),
    ("calibrate_cascade", m_cascade_cold_every_layer),
    ("exact_subspace", m_trailing_eigenvectors),
    ("principal_sines", m_cosines),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_calibration_mutant_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(cal, name, mutant)
    caught = []
    for pin in calibration_pins.ALL_PINS:
        try:
            pin(cal)
        except (AssertionError, ValueError, FloatingPointError, np.linalg.LinAlgError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects mutant {mutant.__name__}"
