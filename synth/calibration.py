"""Seeded synthetic calibration activations for the depth-cascade calibration of GSI's bases.

Input generation only (no subspace iteration, no orthonormalisation of results, no gate): it
draws a chain of planted bases and activation matrices around them.

Recipe (one chain = consecutive layers of one site):
* Planted bases. P_0 = Q of the QR of a seeded d x k Gaussian (diag(R) > 0); P_{l+1} =
  P_l cos(theta) + U_l sin(theta) with U_l orthonormal and orthogonal to P_l, so every principal
  angle between consecutive planted bases equals theta. theta = 25 degrees gives cosine 0.906,
  the "mean cosine above 0.90 between consecutive layers" of the summary's depth coherence
  (gist.science summary of arXiv 2605.03109, §2.3).
* Activations of layer l: A_l = Z diag(s) P_l^T + sigma E with Z (n x k) and E (n x d) standard
  normal and s decreasing linearly from s_max to s_min: n calibration tokens whose energy lies
  mostly in span(P_l), plus isotropic noise. Stored as float32.
* A cold start Omega (d x k standard normal, float32) for the first layer, stored by rows.

Seeds: numpy PCG64 with SeedSequence(entropy=7000 + chain id, spawn_key=(layer, stream)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from .generate import orthonormal_columns

_S_BASIS, _S_ROT, _S_Z, _S_E, _S_OMEGA = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class CalibrationChain:
    cid: int
    n_layers: int
    n: int            # calibration tokens per layer
    d: int
    k: int
    theta_deg: float = 25.0
    s_max: float = 8.0
    s_min: float = 4.0
    sigma: float = 0.5


# the GPT-J-shaped calibration workload: the 4096-wide input of each of the 28 blocks, k = 256,
# one calibration pass of 2048 tokens
GPTJ_CALIBRATION = CalibrationChain(cid=1, n_layers=28, n=2048, d=4096, k=256)


def _rng(c: CalibrationChain, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=7000 + c.cid, spawn_key=tuple(key))))


def planted_bases(c: CalibrationChain, n_layers: int | None = None) -> list:
    """Planted bases P_0..P_{L-1} (float64, d x k each)."""
    L = c.n_layers if n_layers is None else n_layers
    th = math.radians(c.theta_deg)
    out = [orthonormal_columns(_rng(c, 0, _S_BASIS), c.d, c.k)]
    for l in range(1, L):
        p = out[-1]
        q = orthonormal_columns(_rng(c, l, _S_ROT), c.d, 2 * c.k, lead=p)
        out.append(p * math.cos(th) + q[:, c.k:2 * c.k] * math.sin(th))
    return out


def activations(c: CalibrationChain, layer: int, basis: np.ndarray) -> torch.Tensor:
    """A_l (n x d, float32 CPU tensor) around the planted basis of that layer."""
    s = np.linspace(c.s_max, c.s_min, c.k)
    z = _rng(c, layer, _S_Z).standard_normal((c.n, c.k))
    e = _rng(c, layer, _S_E).standard_normal((c.n, c.d), dtype=np.float32)
    a = (z * s) @ basis.T
    a = a.astype(np.float32) + np.float32(c.sigma) * e
    return torch.from_numpy(np.ascontiguousarray(a))


def cold_start(c: CalibrationChain) -> torch.Tensor:
    """Omega by rows (k x d, float32): the Gaussian start of the first layer."""
    g = _rng(c, 0, _S_OMEGA).standard_normal((c.k, c.d), dtype=np.float32)
    return torch.from_numpy(np.ascontiguousarray(g))
