"""Plain, slow, fp64 CPU oracle for Gated Subspace Inference (GSI).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this module:
it is used by the tests, by the smoke check, and by the benchmark's CPU-baseline timing leg.
It shares no code with the HIP library and imports nothing from it.

Source: the technical summary "Gated Subspace Inference for transformer acceleration"
(gist.science, arXiv 2605.03109; Korean and Japanese editions, same content), cited below as
[GSI §n]. Every operand is the *stored* value (fp32 / fp16 / bf16 upcast exactly to float64);
all arithmetic is float64. numpy's matmul is the only library primitive used as a step.

Per linear layer with weight W (d_out x d), basis V (d x k) and token x (d):
  M   = W V                                      [GSI §2.1, the cached low-rank weight image]
  g   = V^T x                                    [GSI §2.1, projection onto the subspace]
  r   = x - V g,  nr2 = |r|^2,  nx2 = |x|^2      [GSI §2.1 decomposition x = V V^T x + r]
  rho = |r| / |x|                                [GSI §2.2 residual ratio]
  fast (gate 0) iff rho < eps, else slow (gate 1) [GSI §2.2]
  y   = M g if fast, W x if slow                 [GSI §2.2 fast and slow paths]

Readings where the summary is silent (each listed in the design notes):
  * |.| is the Euclidean norm.
  * The residual is formed explicitly against the stored V (which is not exactly orthonormal
    once rounded to fp16/bf16); 1 - |g|^2/|x|^2 is a different quantity and is not used.
  * rho < eps is tested as nr2 < eps^2 * nx2, in float64 like every other step (the summary
    fixes no precision for the test); ties go slow, x = 0 goes slow (0 < 0 is false), NaN/Inf go
    slow (comparisons with NaN are false).
  * The slow path returns W x directly (the summary's "full computation"), not M g + W r.

Parity pins for every function here live in tests/test_oracle_pins.py; none is unpinned.
"""
from __future__ import annotations

import numpy as np

FAST, SLOW = 0, 1


def as_f64(a) -> np.ndarray:
    """Exact float64 copy of stored values (numpy array or torch CPU tensor of any float dtype)."""
    if hasattr(a, "detach"):  # torch tensor: fp16/bf16/fp32 -> float64 is exact
        import torch
        return a.detach().cpu().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def precompute_image(W, V) -> np.ndarray:
    """M = W V (d_out x k), the low-rank weight image [GSI §2.1]."""
    W = as_f64(W)
    V = as_f64(V)
    if W.shape[1] != V.shape[0]:
        raise ValueError(f"W {W.shape} and V {V.shape} do not chain")
    return W @ V


def project(V, X) -> np.ndarray:
    """g_t = V^T x_t for each row x_t of X (T x d); returns G (T x k) [GSI §2.1]."""
    V = as_f64(V)
    X = np.atleast_2d(as_f64(X))
    return X @ V


def squared_norms(X) -> np.ndarray:
    """nx2_t = sum_i x_ti^2 for each token."""
    X = np.atleast_2d(as_f64(X))
    return np.einsum("ti,ti->t", X, X)


def residual(V, X, G=None) -> np.ndarray:
    """r_t = x_t - V g_t (T x d), the residual of the exact decomposition [GSI §2.1]."""
    V = as_f64(V)
    X = np.atleast_2d(as_f64(X))
    if G is None:
        G = project(V, X)
    return X - G @ V.T


def residual_norms(V, X, G=None) -> np.ndarray:
    """nr2_t = |r_t|^2 with r_t formed explicitly."""
    R = residual(V, X, G)
    return np.einsum("ti,ti->t", R, R)


def ratio(nr2, nx2) -> np.ndarray:
    """rho_t = |r_t| / |x_t| [GSI §2.2]; NaN where x_t = 0 (diagnostic only)."""
    nr2 = np.asarray(nr2, dtype=np.float64)
    nx2 = np.asarray(nx2, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.sqrt(nr2 / nx2)


def gate(nr2, nx2, eps) -> np.ndarray:
    """Per-token gate bits [GSI §2.2]: 0 = fast (rho < eps), 1 = slow (rho >= eps).

    rho < eps is taken as nr2 < eps^2 * nx2 (both sides non-negative, so the two forms agree for
    nx2 > 0 and the squared form needs no division), evaluated in float64.
    """
    nr2 = np.asarray(nr2, dtype=np.float64)
    nx2 = np.asarray(nx2, dtype=np.float64)
    e = float(eps)
    with np.errstate(invalid="ignore", over="ignore"):
        fast = nr2 < (e * e) * nx2
    return np.where(fast, FAST, SLOW).astype(np.uint8)


def forward(W, V, X, eps, M=None) -> dict:
    """One GSI linear layer over T tokens (rows of X) [GSI §2.1-§2.2].

    Returns y (T x d_out, float64), gate (uint8, 1 = slow), rho, g, nx2, nr2.
    M defaults to the float64 image W V of the stored W and V.
    """
    W = as_f64(W)
    V = as_f64(V)
    X = np.atleast_2d(as_f64(X))
    if M is None:
        M = precompute_image(W, V)
    else:
        M = as_f64(M)
    G = project(V, X)
    nx2 = squared_norms(X)
    nr2 = residual_norms(V, X, G)
    gb = gate(nr2, nx2, eps)
    T = X.shape[0]
    Y = np.empty((T, W.shape[0]), dtype=np.float64)
    fast = gb == FAST
    if fast.any():
        Y[fast] = G[fast] @ M.T          # y = M g  [GSI §2.2 fast path]
    if (~fast).any():
        Y[~fast] = X[~fast] @ W.T        # y = W x  [GSI §2.2 slow path]
    return {"y": Y, "gate": gb, "rho": ratio(nr2, nx2), "g": G, "nx2": nx2, "nr2": nr2}


def gate_only(V, X, eps) -> dict:
    """Gate decisions and their inputs without touching W (used on large stacks)."""
    V = as_f64(V)
    X = np.atleast_2d(as_f64(X))
    G = project(V, X)
    nx2 = squared_norms(X)
    nr2 = residual_norms(V, X, G)
    return {"gate": gate(nr2, nx2, eps), "rho": ratio(nr2, nx2), "g": G, "nx2": nx2, "nr2": nr2}


def spectral_norm(W, tol=1e-12, max_iter=100000, seed=0) -> float:
    """|W|_2 by power iteration on W^T W from a seeded start, until the relative change < tol.

    Used by the Theorem 4 check of [GSI §2.2]: per-token fast-path error <= |W|_2 eps |x|.
    """
    W = as_f64(W)
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(W.shape[1])
    v /= np.linalg.norm(v)
    lam = 0.0
    for _ in range(max_iter):
        u = W.T @ (W @ v)
        nu = np.linalg.norm(u)
        if nu == 0.0:
            return 0.0
        v = u / nu
        if abs(nu - lam) <= tol * nu:
            lam = nu
            break
        lam = nu
    return float(np.sqrt(lam))


def static_projection(W, V, X, M=None) -> dict:
    """Static projection [GSI §2.2, closing remark; §4 negative control]: every token takes the
    fast path, y = M g with g = V^T x, no gate. Returns y and g."""
    W = as_f64(W)
    V = as_f64(V)
    X = np.atleast_2d(as_f64(X))
    M = precompute_image(W, V) if M is None else as_f64(M)
    G = project(V, X)
    return {"y": G @ M.T, "g": G}


def dense(W, X) -> np.ndarray:
    """The unmodified linear map y = W x for every token (a site left outside the method)."""
    W = as_f64(W)
    X = np.atleast_2d(as_f64(X))
    return X @ W.T

