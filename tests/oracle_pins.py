"""Pins that tie the fp64 oracle to what the GSI summary and mathematics fix.

Each pin takes the oracle module as `orc` (so the mutation tests can hand in a deliberately broken
copy) and raises AssertionError when the oracle disagrees with an independent fact:

  P1  decomposition identity  M g + W r = W x                       [GSI §2.1]
  P2  x in span(V_k): g = z, rho = 0, fast, y = W x                  [GSI §2.1-§2.2]
  P3  x orthogonal to span(V_k): g = 0, rho = 1, slow, y = W x       [GSI §2.2 slow path]
  P4  eps = 0: every token slow, y = W x                             [GSI §2.2]
  P5  eps > 1: every nonzero token fast, y = static projection, computed through least squares
      (an independent route to the orthogonal projector)            [GSI §2.2, §4 negative control]
  P6  Theorem 4: |M g - W x| <= |W|_2 rho |x| <= |W|_2 eps |x| on fast tokens; tight when the
      residual lies on W's top right-singular vector; |W|_2 cross-checked against an SVD [GSI §2.2]
  P7  d = 8 brute force in exact rational arithmetic (Fractions), k = 0..8, plus a non-orthonormal
      stored basis where the explicit residual differs from 1 - |g|^2/|x|^2
  P8  exact ties go slow; x = 0, NaN and Inf go slow                 [GSI §2.2: slow iff rho >= eps]
  P9  per-token independence: T-row call equals T one-row calls       [GSI §2.2: per-token gate]
  P10 static projection: y = W P x with P the orthogonal projector onto span(V), computed through
      least squares; equal to the gated forward at eps > 1 on nonzero tokens [GSI §2.2, §4]
  P11 dense map: exact integer W x                                    [a site outside the method]
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _orthonormal(rng, d, n):
    q, r = np.linalg.qr(rng.standard_normal((d, n)))
    return q * np.sign(np.diag(r))


def _case(seed=0, d=48, k=12, d_out=40):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d_out, d)) / math.sqrt(d)
    Q = _orthonormal(rng, d, d)
    return rng, W, Q[:, :k], Q[:, k:]


def pin_decomposition(orc):
    rng, W, V, _ = _case(1)
    X = rng.standard_normal((9, V.shape[0]))
    M = orc.precompute_image(W, V)
    G = orc.project(V, X)
    R = orc.residual(V, X, G)
    lhs = G @ M.T + R @ W.T
    rhs = X @ W.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs)), "M g + W r != W x"
    # the residual carries exactly the part of x outside span(V): V^T r = 0
    assert np.max(np.abs(R @ V)) <= 1e-12 * np.max(np.abs(X)), "residual not orthogonal to V"


def pin_in_span(orc):
    rng, W, V, _ = _case(2)
    Z = rng.standard_normal((7, V.shape[1]))
    X = Z @ V.T
    out = orc.forward(W, V, X, 0.10)
    assert np.max(np.abs(out["g"] - Z)) <= 1e-12 * np.max(np.abs(Z)), "g != z for x = V z"
    assert np.all(out["rho"] <= 1e-14 * 10), "rho != 0 in span"
    assert np.all(out["gate"] == orc.FAST), "in-span token not fast"
    assert np.max(np.abs(out["y"] - X @ W.T)) <= 1e-12 * np.max(np.abs(X @ W.T)), "M g != W x in span"


def pin_orthogonal(orc):
    rng, W, V, C = _case(3)
    X = rng.standard_normal((6, C.shape[1])) @ C.T
    out = orc.forward(W, V, X, 0.99)
    assert np.max(np.abs(out["g"])) <= 1e-12 * np.max(np.abs(X)), "g != 0 for x orthogonal"
    assert np.all(np.abs(out["rho"] - 1.0) <= 1e-12), "rho != 1 for x orthogonal"
    assert np.all(out["gate"] == orc.SLOW), "orthogonal token not slow"
    assert np.max(np.abs(out["y"] - X @ W.T)) <= 1e-12 * np.max(np.abs(X @ W.T))


def _mixed_tokens(rng, V, C, n=16):
    z = rng.standard_normal((n, V.shape[1]))
    w = rng.standard_normal((n, C.shape[1]))
    s = np.geomspace(1e-3, 3.0, n)[:, None]
    return z @ V.T + s * (w @ C.T)


def pin_eps_zero(orc):
    rng, W, V, C = _case(4)
    X = _mixed_tokens(rng, V, C)
    out = orc.forward(W, V, X, 0.0)
    assert np.all(out["gate"] == orc.SLOW), "eps = 0 left a token fast"
    assert np.array_equal(out["y"], X @ W.T), "eps = 0 is not the dense product"


def pin_eps_above_one(orc):
    rng, W, V, C = _case(5)
    X = _mixed_tokens(rng, V, C)
    out = orc.forward(W, V, X, 1.5)
    assert np.all(out["gate"] == orc.FAST), "eps > 1 left a nonzero token slow"
    coef = np.linalg.lstsq(V, X.T, rcond=None)[0]        # argmin_c |V c - x|
    ref = (W @ (V @ coef)).T                             # W times the orthogonal projection of x
    assert np.max(np.abs(out["y"] - ref)) <= 1e-11 * np.max(np.abs(ref)), "eps > 1 is not static projection"


def pin_spectral_norm(orc):
    rng = np.random.default_rng(6)
    for shape in [(40, 48), (48, 40), (17, 17)]:
        W = rng.standard_normal(shape)
        ref = np.linalg.svd(W, compute_uv=False)[0]
        got = orc.spectral_norm(W)
        assert abs(got - ref) <= 1e-8 * ref, f"spectral norm {got} vs svd {ref}"


def pin_theorem4(orc):
    rng, W, V, C = _case(7)
    X = _mixed_tokens(rng, V, C, n=40)
    eps = 0.5
    out = orc.forward(W, V, X, eps)
    nw = orc.spectral_norm(W)
    fast = out["gate"] == orc.FAST
    assert fast.sum() >= 10
    err = np.linalg.norm(out["y"][fast] - X[fast] @ W.T, axis=1)
    nx = np.linalg.norm(X[fast], axis=1)
    assert np.all(err <= nw * out["rho"][fast] * nx * (1 + 1e-9)), "Theorem 4 (rho form) violated"
    assert np.all(err <= nw * eps * nx * (1 + 1e-9)), "Theorem 4 (eps form) violated"
    # adversarial: residual along W's top right-singular vector, basis orthogonal to it -> equality
    _, _, vt = np.linalg.svd(W)
    v1 = vt[0]
    d, k = V.shape
    Q, R = np.linalg.qr(np.concatenate([v1[:, None], rng.standard_normal((d, k))], axis=1))
    Vt = Q[:, 1:k + 1]
    z = rng.standard_normal(k)
    x = Vt @ z + 0.05 * np.linalg.norm(z) * v1
    o = orc.forward(W, Vt, x[None, :], 0.2)
    assert o["gate"][0] == orc.FAST
    e = np.linalg.norm(o["y"][0] - W @ x)
    bound = orc.spectral_norm(W) * o["rho"][0] * np.linalg.norm(x)
    assert abs(e / bound - 1.0) <= 1e-6, f"Theorem 4 not tight on the adversarial token: {e / bound}"


def _hadamard8():
    h = np.array([[1]])
    for _ in range(3):
        h = np.block([[h, h], [h, -h]])
    return h


def _exact(Wi, Vr, x, eps):
    """Exact rational GSI for one token, with V given by rational entries (list of columns)."""
    d = len(x)
    k = len(Vr)
    g = [sum(Vr[j][i] * x[i] for i in range(d)) for j in range(k)]
    r = [x[i] - sum(Vr[j][i] * g[j] for j in range(k)) for i in range(d)]
    nr2 = sum(v * v for v in r)
    nx2 = sum(v * v for v in x)
    fast = nr2 < eps * eps * nx2
    if fast:
        vg = [sum(Vr[j][i] * g[j] for j in range(k)) for i in range(d)]
        y = [sum(Wi[o][i] * vg[i] for i in range(d)) for o in range(len(Wi))]
    else:
        y = [sum(Wi[o][i] * x[i] for i in range(d)) for o in range(len(Wi))]
    return nr2, nx2, fast, y


def pin_brute_force_d8(orc):
    """V = first k Hadamard columns / sqrt(8): V V^T = H_k H_k^T / 8 is rational, so nr2, gate
    and y are exact rationals (g itself is not, but only V g enters)."""
    rng = np.random.default_rng(8)
    H = _hadamard8()
    perm = rng.permutation(8)
    H = H[:, perm]                                    # column order not symmetric in general
    Wi = rng.integers(-4, 5, size=(5, 8))
    eps = Fraction(3, 10)
    for k in range(0, 9):
        # scaled columns: V_j = H_j / sqrt(8); exact work uses U_j = H_j / 8 paired with H_j so
        # that sum_j V_j V_j^T = sum_j H_j H_j^T / 8
        Vf = H[:, :k] / math.sqrt(8.0)
        for t in range(12):
            xi = rng.integers(-6, 7, size=8)
            if not xi.any():
                xi[0] = 1
            xq = [Fraction(int(v)) for v in xi]
            Hc = [[Fraction(int(H[i, j])) for i in range(8)] for j in range(k)]
            gH = [sum(Hc[j][i] * xq[i] for i in range(8)) for j in range(k)]
            vg = [sum(Hc[j][i] * gH[j] for j in range(k)) / 8 for i in range(8)]
            r = [xq[i] - vg[i] for i in range(8)]
            nr2 = sum(v * v for v in r)
            nx2 = sum(v * v for v in xq)
            if nr2 == eps * eps * nx2:
                continue  # exact ties are pinned separately
            fast = nr2 < eps * eps * nx2
            src = vg if fast else xq
            y = [sum(int(Wi[o, i]) * src[i] for i in range(8)) for o in range(5)]
            out = orc.forward(Wi.astype(np.float64), Vf, xi.astype(np.float64)[None, :], float(eps))
            assert abs(out["nr2"][0] - float(nr2)) <= 1e-12 * float(nx2), f"nr2 k={k}"
            assert abs(out["nx2"][0] - float(nx2)) <= 1e-12 * float(nx2)
            assert bool(out["gate"][0] == orc.FAST) == fast, f"gate k={k}"
            go = orc.gate_only(Vf, xi.astype(np.float64)[None, :], float(eps))
            assert bool(go["gate"][0] == orc.FAST) == fast, f"gate_only k={k}"
            assert abs(go["nr2"][0] - float(nr2)) <= 1e-12 * float(nx2), f"gate_only nr2 k={k}"
            assert np.max(np.abs(out["y"][0] - np.array([float(v) for v in y]))) <= 1e-11 * (1 + max(abs(float(v)) for v in y))
            # residual is the least-squares distance to span(V) for an orthonormal basis
            if k > 0:
                c = np.linalg.lstsq(Vf, xi.astype(np.float64), rcond=None)[0]
                assert abs(np.sum((xi - Vf @ c) ** 2) - float(nr2)) <= 1e-10 * float(nx2)
        if k == 8:
            out = orc.forward(Wi.astype(np.float64), Vf, rng.integers(-6, 7, size=(4, 8)).astype(np.float64) + 0.5, 0.01)
            assert np.all(out["gate"] == orc.FAST), "k = d must make every token fast"
        if k == 0:
            out = orc.forward(Wi.astype(np.float64), Vf, rng.integers(-6, 7, size=(4, 8)).astype(np.float64) + 0.5, 0.99)
            assert np.all(out["gate"] == orc.SLOW), "k = 0 must make every token slow"


def pin_non_orthonormal(orc):
    """A stored basis that is not orthonormal (as after bf16 rounding): the residual is formed
    explicitly as x - V (V^T x); the Pythagorean shortcut |x|^2 - |g|^2 is a different number."""
    Vq = [[Fraction(1), Fraction(1, 2), Fraction(0), Fraction(0)],
          [Fraction(1, 2), Fraction(1), Fraction(1, 4), Fraction(0)]]          # columns, d = 4, k = 2
    Wq = [[Fraction(1), Fraction(2), Fraction(0), Fraction(-1)],
          [Fraction(0), Fraction(1), Fraction(3), Fraction(1)]]
    xq = [Fraction(3), Fraction(-1), Fraction(2), Fraction(5)]
    for eps in (Fraction(9, 10), Fraction(99, 100)):
        nr2, nx2, fast, y = _exact(Wq, Vq, xq, eps)
        V = np.array([[float(Vq[j][i]) for j in range(2)] for i in range(4)])
        W = np.array([[float(v) for v in row] for row in Wq])
        x = np.array([[float(v) for v in xq]])
        out = orc.forward(W, V, x, float(eps), M=W @ V)
        assert abs(out["nr2"][0] - float(nr2)) <= 1e-13 * float(nx2), "residual not formed explicitly"
        short = float(nx2) - float(np.sum(out["g"][0] ** 2))
        assert abs(short - float(nr2)) > 1e-2 * float(nx2), "case does not separate the shortcut"
        assert bool(out["gate"][0] == orc.FAST) == fast
        assert np.max(np.abs(out["y"][0] - np.array([float(v) for v in y]))) <= 1e-12 * 10


def pin_ties_and_degenerate(orc):
    """V = [e_1, e_2], eps = 1/2, integer x with nr2 = nx2/4 exactly -> slow (rho = eps is slow)."""
    d, k = 8, 2
    V = np.eye(d)[:, :k]
    W = np.arange(1, 3 * d + 1, dtype=np.float64).reshape(3, d) / 7.0
    tie = np.array([3, 0, 1, 1, 1, 0, 0, 0], dtype=np.float64)       # nx2 = 12, nr2 = 3
    more = np.array([3, 0, 1, 1, 1, 1, 0, 0], dtype=np.float64)      # nr2 = 4 > 13/4
    less = np.array([3, 0, 1, 1, 0, 0, 0, 0], dtype=np.float64)      # nr2 = 2 < 11/4
    X = np.stack([tie, more, less])
    out = orc.forward(W, V, X, 0.5)
    assert out["nr2"][0] == 3.0 and out["nx2"][0] == 12.0
    assert list(out["gate"]) == [orc.SLOW, orc.SLOW, orc.FAST], f"tie rule: {out['gate']}"
    assert list(orc.gate_only(V, X, 0.5)["gate"]) == [orc.SLOW, orc.SLOW, orc.FAST], "tie rule (gate_only)"
    z = np.zeros((1, d))
    o = orc.forward(W, V, z, 0.5)
    assert o["gate"][0] == orc.SLOW and np.all(o["y"] == 0.0) and np.isnan(o["rho"][0]), "x = 0"
    for bad in (np.nan, np.inf):
        xb = tie.copy()
        xb[5] = bad
        o = orc.forward(W, V, xb[None, :], 0.5)
        assert o["gate"][0] == orc.SLOW, f"{bad} must go slow"
        assert not np.all(np.isfinite(o["y"][0])), f"{bad} must propagate into y"


def pin_per_token(orc):
    rng, W, V, C = _case(9)
    X = _mixed_tokens(rng, V, C, n=10)
    full = orc.forward(W, V, X, 0.3)
    for t in range(X.shape[0]):
        one = orc.forward(W, V, X[t:t + 1], 0.3)
        assert one["gate"][0] == full["gate"][t]
        # BLAS may block a T-row product differently from a one-row product: rounding only
        assert np.max(np.abs(one["y"][0] - full["y"][t])) <= 1e-14 * np.max(np.abs(full["y"][t]))


def pin_static_projection(orc):
    rng, W, V, C = _case(10)
    X = _mixed_tokens(rng, V, C, n=12)
    out = orc.static_projection(W, V, X)
    coef = np.linalg.lstsq(V, X.T, rcond=None)[0]
    ref = (W @ (V @ coef)).T
    assert np.max(np.abs(out["y"] - ref)) <= 1e-11 * np.max(np.abs(ref)), "static projection != W P x"
    # a non-orthonormal stored basis: y = M (V^T x) is what the fast path returns, not W P x
    Vs = V * 1.01
    o2 = orc.static_projection(W, Vs, X)
    assert np.max(np.abs(o2["y"] - (X @ Vs) @ (W @ Vs).T)) <= 1e-12 * np.max(np.abs(o2["y"]))
    fwd = orc.forward(W, V, X, 1.5)
    assert np.all(fwd["gate"] == orc.FAST)
    assert np.max(np.abs(fwd["y"] - out["y"])) <= 1e-12 * np.max(np.abs(ref))


def pin_dense(orc):
    rng = np.random.default_rng(12)
    Wi = rng.integers(-9, 10, size=(7, 16))
    Xi = rng.integers(-9, 10, size=(5, 16))
    exact = Xi @ Wi.T                                       # integer arithmetic, exact
    got = orc.dense(Wi.astype(np.float64), Xi.astype(np.float64))
    assert np.array_equal(got, exact.astype(np.float64)), "dense map is not W x"


ALL_PINS = [pin_decomposition, pin_in_span, pin_orthogonal, pin_eps_zero, pin_eps_above_one,
            pin_spectral_norm, pin_theorem4, pin_brute_force_d8, pin_non_orthonormal,
            pin_ties_and_degenerate, pin_per_token, pin_static_projection, pin_dense]


def failing_pins(orc):
    """Names of the pins that reject `orc` (used by the mutation tests)."""
    bad = []
    for p in ALL_PINS:
        try:
            p(orc)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            bad.append(p.__name__)
    return bad
