"""Plain, slow, fp64 CPU oracle for calibrating GSI's activation bases with the depth cascade.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this module:
it is used by the tests and the benchmark's measurement of the calibration. It shares no code
with the HIP library and imports nothing from it.

Source: the technical summary "Gated Subspace Inference for transformer acceleration"
(gist.science, arXiv 2605.03109), section 2.3 (depth cascade and calibration), cited as
[GSI §2.3]. What the summary fixes: a layer's basis V_k is computed once, from one forward pass
over a representative calibration sequence; the activation subspaces of consecutive layers are
strongly aligned (mean cosine above 0.90 in the deeper layers), so the basis of layer l + 1 is
initialised from the basis of layer l and corrected with a few rank-1 (DGKS) updates instead of
a full SVD per layer; the cascade cuts the calibration cost by 96% [GSI §3 item 3].

Readings (the summary names the pieces, not the algorithm):
  C1  The activation subspace of a layer whose calibration activations are the rows of A (N x d)
      is the span of the k leading eigenvectors of A^T A. By the Eckart-Young theorem it is the
      k-dimensional subspace with the least total squared residual sum_t |x_t - V V^T x_t|^2 over
      the calibration tokens, the residual the gate measures [GSI §2.1-§2.2].
  C2  It is reached by subspace (block power) iteration  Q <- orth(A^T (A Q)).
  C3  orth is Gram-Schmidt over the columns in order: column j is projected against the
      orthonormal columns before it and normalised, one rank-1 extension of the factor per
      column. With the Daniel-Gragg-Kaufman-Stewart criterion: when that projection leaves less
      than eta = 1/sqrt(2) of the column's norm, the column is projected a second time.
  C4  First layer (cold start): Q0 is a d x k Gaussian draw, passed in; n_cold iterations.
  C5  Cascade: layer l + 1 starts from layer l's calibrated basis; n_warm (few) iterations.
  C6  The basis is returned as it comes out of the last orthonormalisation (no Rayleigh-Ritz
      rotation): the gate and y = M g depend on the span only.

numpy's matmul, eigh and svd are the only library primitives used as steps. Pins for every
function here live in tests/calibration_pins.py; none is unpinned.
"""
from __future__ import annotations

import math

import numpy as np

DGKS_ETA = 1.0 / math.sqrt(2.0)


def as_f64(a) -> np.ndarray:
    """Exact float64 copy of stored values (numpy array or torch CPU tensor)."""
    if hasattr(a, "detach"):
        import torch
        return a.detach().cpu().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def dgks_orthonormalize(Y, eta: float = DGKS_ETA):
    """Gram-Schmidt with DGKS reorthogonalisation over the columns of Y (d x k), in order [C3].

    Returns (Q, twice): Q (d x k) with orthonormal columns, span(Q[:, :j]) = span(Y[:, :j]) for
    every j, and `twice[j]` telling whether column j needed the second projection. Y must have
    full column rank (a column that projects to zero has no direction to normalise).
    """
    Y = as_f64(Y)
    if Y.ndim != 2 or Y.shape[1] > Y.shape[0]:
        raise ValueError(f"need a tall d x k matrix, got {Y.shape}")
    d, k = Y.shape
    Q = np.zeros((d, k))
    twice = np.zeros(k, dtype=bool)
    for j in range(k):
        P = Q[:, :j]
        v = Y[:, j].copy()
        before = float(v @ v)
        v = v - P @ (P.T @ v)
        after = float(v @ v)
        if after < eta * eta * before:
            twice[j] = True
            v = v - P @ (P.T @ v)
            after = float(v @ v)
        Q[:, j] = v / math.sqrt(after)
    return Q, twice


def subspace_iteration(A, Q0, n_iter: int) -> np.ndarray:
    """n_iter steps of Q <- orth(A^T (A Q)) from Q0 (d x k) [C2, C3]; A is N x d."""
    A = as_f64(A)
    Q = as_f64(Q0)
    if A.shape[1] != Q.shape[0]:
        raise ValueError(f"A {A.shape} and Q0 {Q.shape} do not chain")
    for _ in range(n_iter):
        Q, _ = dgks_orthonormalize(A.T @ (A @ Q))
    return Q


def calibrate_cascade(As, Omega, n_cold: int, n_warm: int) -> list:
    """Bases of consecutive layers [GSI §2.3]: layer 0 from the Gaussian start Omega (cold,
    n_cold iterations) [C4], every later layer from the previous layer's basis (n_warm) [C5]."""
    out = []
    Q = None
    for i, A in enumerate(As):
        Q = subspace_iteration(A, Omega if i == 0 else Q, n_cold if i == 0 else n_warm)
        out.append(Q)
    return out


def exact_subspace(A, k: int) -> np.ndarray:
    """The k leading eigenvectors of A^T A (d x k), the definition C1 written out with a
    symmetric eigensolver; columns in decreasing eigenvalue order."""
    A = as_f64(A)
    w, U = np.linalg.eigh(A.T @ A)
    return U[:, np.argsort(w)[::-1][:k]]


def principal_sines(U, V) -> np.ndarray:
    """Sines of the principal angles between span(U) and span(V) (orthonormal d x k each),
    largest first: the singular values of (I - U U^T) V."""
    U = as_f64(U)
    V = as_f64(V)
    s = np.linalg.svd(V - U @ (U.T @ V), compute_uv=False)
    return np.sort(np.clip(s, 0.0, 1.0))[::-1]


def residual_energy(A, V) -> float:
    """sum_t |x_t - V V^T x_t|^2 over the rows x_t of A, for orthonormal V."""
    A = as_f64(A)
    V = as_f64(V)
    R = A - (A @ V) @ V.T
    return float(np.sum(R * R))
