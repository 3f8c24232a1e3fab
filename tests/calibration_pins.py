"""Pins that tie the fp64 calibration oracle to what the GSI summary and mathematics fix.

Each pin takes the oracle module as `cal` (so the mutation tests can hand in a broken copy) and
raises AssertionError when the oracle disagrees with an independent fact:

  Q1  Gram-Schmidt is the QR factorisation: on a well-conditioned Y, dgks_orthonormalize(Y)
      equals the Q of a library QR with diag(R) > 0, and Q^T Y is upper triangular with a
      positive diagonal                                             [textbook identity]
  Q2  DGKS keeps orthogonality where one Gram-Schmidt pass loses it: on a Y with condition number
      ~1e9 the result is orthonormal to 1e-12 and the second projection was taken  [DGKS 1976]
  Q3  exact rank k: when A = Z B^T (B orthonormal, d x k) one iteration from a Gaussian start
      gives span(B) exactly                                         [power iteration]
  Q4  convergence rate: on A with a known spectrum, tan of the largest principal angle to the
      leading eigenspace shrinks at least by lambda_{k+1}/lambda_k per iteration, and the result
      approaches the eigensolver's subspace                         [classical bound]
  Q5  the definition: exact_subspace equals the leading right singular vectors of an SVD and
      leaves the Eckart-Young residual sum_{i>k} sigma_i^2; principal_sines reproduces a planted
      angle                                                          [closed forms]
  Q6  depth cascade [GSI §2.3]: with layer l+1's subspace rotated by 25 degrees from layer l's
      (cosine 0.906 > 0.90), one warm iteration from layer l's basis lands within the one-step
      bound of the rotated angle, which a cold start with one iteration does not reach
"""
from __future__ import annotations

import math

import numpy as np


def _orthonormal(rng, d, n):
    q, r = np.linalg.qr(rng.standard_normal((d, n)))
    return q * np.sign(np.diag(r))


def _spectral_matrix(rng, n, d, sig):
    """A = U diag(sig) W^T with Haar-like orthonormal U (n x r), W (d x r)."""
    r = len(sig)
    U = _orthonormal(rng, n, r)
    Wm = _orthonormal(rng, d, r)
    return U @ np.diag(sig) @ Wm.T, Wm


def _tan_max(sines):
    s = float(np.max(sines))
    return s / math.sqrt(max(1.0 - s * s, 1e-300))


def pin_gram_schmidt_is_qr(cal):
    rng = np.random.default_rng(21)
    Y = rng.standard_normal((64, 16))
    Q, _ = cal.dgks_orthonormalize(Y)
    q, r = np.linalg.qr(Y)
    sgn = np.sign(np.diag(r))
    assert np.max(np.abs(Q - q * sgn)) < 1e-12, "Gram-Schmidt factor differs from QR"
    R = Q.T @ Y
    assert np.max(np.abs(np.tril(R, -1))) < 1e-12 and np.all(np.diag(R) > 0)
    assert np.max(np.abs(Q.T @ Q - np.eye(16))) < 1e-13


def pin_dgks_reorthogonalises(cal):
    rng = np.random.default_rng(22)
    d, k = 80, 20
    # nearly dependent columns: a well-conditioned basis times a triangular factor with a
    # geometric diagonal down to 1e-9
    B = _orthonormal(rng, d, k)
    T = np.triu(rng.standard_normal((k, k))) + np.diag(np.geomspace(1.0, 1e-9, k))
    Y = B @ T
    Q, twice = cal.dgks_orthonormalize(Y)
    assert np.max(np.abs(Q.T @ Q - np.eye(k))) < 1e-12, "orthogonality lost"
    assert twice.any(), "no column took the second projection"
    # Y's columns leave span(B) only by rounding (~1e-16), amplified by the 1e-9 scale of the
    # last columns
    assert np.max(cal.principal_sines(B, Q)) < 1e-6
    # span of the leading columns is kept column by column
    for j in (1, 5, 12):
        assert np.max(cal.principal_sines(Q[:, :j], _orthonormal_span(Y[:, :j]))) < 1e-6


def _orthonormal_span(Y):
    u, _, _ = np.linalg.svd(Y, full_matrices=False)
    return u


def pin_exact_rank_k(cal):
    rng = np.random.default_rng(23)
    n, d, k = 200, 96, 12
    B = _orthonormal(rng, d, k)
    A = rng.standard_normal((n, k)) @ B.T
    Q = cal.subspace_iteration(A, rng.standard_normal((d, k)), 1)
    assert np.max(np.abs(Q.T @ Q - np.eye(k))) < 1e-12
    assert np.max(cal.principal_sines(B, Q)) < 1e-10


def pin_convergence_rate(cal):
    rng = np.random.default_rng(24)
    n, d, k = 300, 120, 10
    sig = np.concatenate([np.linspace(20.0, 10.0, k), 5.0 * np.linspace(1.0, 0.2, d - k)])
    A, Wm = _spectral_matrix(rng, n, d, sig)
    lead = Wm[:, :k]
    ratio = (sig[k] / sig[k - 1]) ** 2          # lambda_{k+1} / lambda_k = 0.25
    Q0 = rng.standard_normal((d, k))
    t_prev = _tan_max(cal.principal_sines(lead, _orthonormal_span(Q0)))
    for q in range(1, 13):
        Q = cal.subspace_iteration(A, Q0, q)
        t = _tan_max(cal.principal_sines(lead, Q))
        assert t <= t_prev * ratio * (1 + 1e-9) + 1e-13, f"iteration {q}: tan {t} > {t_prev} * {ratio}"
        t_prev = t
    assert np.max(cal.principal_sines(cal.exact_subspace(A, k), Q)) < 1e-4


def pin_definition(cal):
    rng = np.random.default_rng(25)
    n, d, k = 150, 60, 8
    sig = np.sort(rng.uniform(0.5, 10.0, d))[::-1]
    sig[k:] *= 0.3
    A, Wm = _spectral_matrix(rng, n, d, sig)
    E = cal.exact_subspace(A, k)
    _, s, vt = np.linalg.svd(A, full_matrices=False)
    assert np.max(cal.principal_sines(vt[:k].T, E)) < 1e-10
    assert np.max(cal.principal_sines(Wm[:, :k], E)) < 1e-10
    assert abs(cal.residual_energy(A, E) - float(np.sum(s[k:] ** 2))) <= 1e-9 * float(np.sum(s ** 2))
    # a planted principal angle: span{e1 cos t + e2 sin t} against span{e1}
    t = 0.3
    U = np.zeros((5, 1)); U[0, 0] = 1.0
    V = np.zeros((5, 1)); V[0, 0] = math.cos(t); V[1, 0] = math.sin(t)
    assert abs(cal.principal_sines(U, V)[0] - math.sin(t)) < 1e-15


def pin_depth_cascade(cal):
    rng = np.random.default_rng(26)
    n, d, k = 400, 128, 16
    th = math.radians(25.0)
    V0 = _orthonormal(rng, d, k)
    Ufull = _orthonormal(rng, d, 3 * k)
    U = Ufull - V0 @ (V0.T @ Ufull)
    U = _orthonormal_span(U)[:, :k]
    V1 = V0 * math.cos(th) + U * math.sin(th)            # every principal angle 25 degrees
    assert np.allclose(cal.principal_sines(V0, V1), math.sin(th), atol=1e-12)

    def acts(V, noise):
        return rng.standard_normal((n, k)) @ np.diag(np.linspace(8.0, 4.0, k)) @ V.T + noise * rng.standard_normal((n, d))
    A1 = acts(V1, 0.3)
    E1 = cal.exact_subspace(A1, k)
    lam = np.sort(np.linalg.eigvalsh(A1.T @ A1))[::-1]
    ratio = lam[k] / lam[k - 1]
    t0 = _tan_max(cal.principal_sines(E1, V0))
    warm = cal.subspace_iteration(A1, V0, 1)
    t1 = _tan_max(cal.principal_sines(E1, warm))
    assert t1 <= t0 * ratio * (1 + 1e-9), f"warm step {t1} above the bound {t0 * ratio}"
    cold = cal.subspace_iteration(A1, rng.standard_normal((d, k)), 1)
    assert _tan_max(cal.principal_sines(E1, cold)) > t0 * ratio, "a cold step should not reach the warm bound"
    # the cascade helper starts layer 1 from layer 0's basis
    A0 = acts(V0, 0.3)
    Om = rng.standard_normal((d, k))
    Qs = cal.calibrate_cascade([A0, A1], Om, 6, 1)
    assert np.max(np.abs(Qs[1] - cal.subspace_iteration(A1, Qs[0], 1))) < 1e-12
    assert np.max(np.abs(Qs[0] - cal.subspace_iteration(A0, Om, 6))) < 1e-12


ALL_PINS = [pin_gram_schmidt_is_qr, pin_dgks_reorthogonalises, pin_exact_rank_k, pin_convergence_rate,
            pin_definition, pin_depth_cascade]
