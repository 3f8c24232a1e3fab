"""Seeded synthetic inputs for GSI: weights W, orthonormal bases V_k, and tokens x.

Shared by the tests, the benchmark and the oracle's timing leg. This module holds none of the
method's arithmetic (no projection onto V_k, no residual, no ratio, no gate, no GEMV): it only
draws random numbers, orthonormalises them with a library QR, and combines them so that each
token's residual ratio equals a planned value by construction.

Construction (one site = one (block, site) pair of a config):

* Basis. Q = QR of a seeded d x (k + m) Gaussian, columns sign-fixed so diag(R) > 0.
  V_k = Q[:, :k] (this is exactly the Q of the QR of the first k Gaussian columns) and
  C = Q[:, k:k+m] is an orthonormal block orthogonal to V_k, m = min(d - k, m_complement).
  Depth-coherent configs rotate block l's basis into block l+1's by a fixed angle theta:
  V_{l+1} = V_l cos(theta) + U sin(theta), U orthonormal and orthogonal to V_l, so every
  principal angle between consecutive bases equals theta (the summary's §2.3 reports mean
  cosine > 0.90 between consecutive layers; theta = 25 deg gives 0.906).
* Token. x = V_k z + s * C w with z ~ N(0, I_k), w ~ N(0, I_m). Because [V_k | C] has
  orthonormal columns, in exact arithmetic the residual of x against V_k is s * C w and the
  ratio is rho = s |w| / sqrt(|z|^2 + s^2 |w|^2); s is solved from a planned rho*.
  Fast tokens get rho* ~ U(eps/2, eps - PLAN_MARGIN), slow ones rho* ~ U(eps + PLAN_MARGIN,
  min(2 eps, 0.95)); PLAN_MARGIN = 5e-3 keeps the *realised* ratio on the stored (rounded)
  operands more than 1e-3 away from eps, which the tests check with the oracle.
* Storage. Everything is generated in float64 (W in float32) and rounded to the config's dtype
  with round-to-nearest-even (torch CPU casts).

Seeds: numpy PCG64 with SeedSequence(entropy=1000 + config id, spawn_key=(block, site, stream)).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from functools import lru_cache

import numpy as np
import torch

from .configs import Config, get

PLAN_MARGIN = 5e-3
RHO_CAP = 0.95

# stream ids inside a site's seed tree
_S_W, _S_BASIS, _S_TOKENS, _S_PLAN, _S_ROT = 0, 1, 2, 3, 4

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _rng(cid: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=1000 + cid, spawn_key=tuple(key))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def store(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float array to the storage dtype (round to nearest even), as a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(TORCH_DTYPE[dtype]).contiguous()


def orthonormal_columns(rng: np.random.Generator, d: int, n: int, lead: np.ndarray | None = None) -> np.ndarray:
    """Q (d x n) of a QR with diag(R) > 0. With `lead` (d x j, orthonormal), QR of [lead | G]."""
    g = rng.standard_normal((d, n if lead is None else n - lead.shape[1]))
    a = g if lead is None else np.concatenate([lead, g], axis=1)
    q, r = np.linalg.qr(a)
    sgn = np.sign(np.diag(r))
    sgn[sgn == 0] = 1.0
    return q * sgn


def _m(cfg: Config, d: int) -> int:
    return min(d - cfg.k, cfg.m_complement)


def _fresh_basis(cid: int, block: int, site: int):
    cfg = get(cid)
    d, k = cfg.sites[site].d, cfg.k
    m = _m(cfg, d)
    q = orthonormal_columns(_rng(cid, block, site, _S_BASIS), d, k + m)
    return q[:, :k].copy(), q[:, k:k + m].copy()


@lru_cache(maxsize=None)
def _chain_basis(cid: int, block: int, site: int):
    """Depth-coherent chain (cached: block l needs block l-1)."""
    cfg = get(cid)
    if block == 0:
        return _fresh_basis(cid, block, site)
    k = cfg.k
    d = cfg.sites[site].d
    m = _m(cfg, d)
    v_prev, _ = _chain_basis(cid, block - 1, site)
    th = math.radians(cfg.depth_rotation_deg)
    q = orthonormal_columns(_rng(cid, block, site, _S_ROT), d, 2 * k, lead=v_prev)
    u = q[:, k:2 * k]
    v = v_prev * math.cos(th) + u * math.sin(th)
    q2 = orthonormal_columns(_rng(cid, block, site, _S_BASIS), d, k + m, lead=v)
    return v, q2[:, k:k + m].copy()


def site_basis(cfg: Config, block: int, site: int):
    """(V_k, C) in float64: d x k orthonormal basis and d x m orthonormal complement block."""
    if cfg.depth_rotation_deg is None:
        return _fresh_basis(cfg.cid, block, site)
    return _chain_basis(cfg.cid, block, site)


def site_weight(cfg: Config, block: int, site: int) -> torch.Tensor:
    """W (d_out x d) in the config's dtype, entries N(0, w_std^2) (w_std = 1/sqrt(d) if unset).

    Drawn in row chunks of 512 with their own seeds so the result does not depend on threads.
    """
    shp = cfg.sites[site]
    std = cfg.w_std if cfg.w_std is not None else 1.0 / math.sqrt(shp.d)
    out = torch.empty((shp.d_out, shp.d), dtype=TORCH_DTYPE[cfg.dtype])
    rows = 512
    chunks = [(i, min(shp.d_out, i + rows)) for i in range(0, shp.d_out, rows)]

    def work(ci):
        a, b = chunks[ci]
        g = _rng(cfg.cid, block, site, _S_W, ci).standard_normal((b - a, shp.d), dtype=np.float32)
        g *= np.float32(std)
        out[a:b] = torch.from_numpy(g).to(out.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(len(chunks))))
    return out


def planned_ratios(cfg: Config, block: int, site: int, n_steps: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Planned residual ratios rho* (float64) and planned slow mask, shape (steps, t_step)."""
    steps = cfg.n_steps if n_steps is None else n_steps
    rng = _rng(cfg.cid, block, site, _S_PLAN)
    eps = cfg.eps
    t = cfg.t_step
    pl = cfg.slow
    slow = np.zeros((steps, t), dtype=bool)
    if pl.kind == "fixed":
        n = steps * t
        pos = rng.choice(n, size=pl.count, replace=False)
        slow.reshape(-1)[pos] = True
    elif pl.kind == "binomial":
        for st in range(steps):
            c = rng.binomial(t, pl.p)
            slow[st, rng.permutation(t)[:c]] = True
    elif pl.kind == "lognormal":
        pass
    else:  # pragma: no cover
        raise ValueError(pl.kind)

    if pl.kind == "lognormal":
        rho = np.empty((steps, t))
        flat = rho.reshape(-1)
        for i in range(flat.size):
            while True:
                r = eps * math.exp(rng.standard_normal() - pl.shift)
                if abs(r - eps) >= PLAN_MARGIN and r <= RHO_CAP:
                    break
            flat[i] = r
        slow = rho > eps
        return rho, slow
    lo_f, hi_f = 0.5 * eps, eps - PLAN_MARGIN
    lo_s, hi_s = eps + PLAN_MARGIN, min(2.0 * eps, RHO_CAP)
    u = rng.random((steps, t))
    rho = np.where(slow, lo_s + u * (hi_s - lo_s), lo_f + u * (hi_f - lo_f))
    return rho, slow


def site_tokens(cfg: Config, block: int, site: int, n_steps: int | None = None, basis=None):
    """Tokens for one site: (X stored [steps*t_step, d], planned slow mask [steps*t_step], rho*).

    `basis` = (V_k, C) from site_basis(cfg, block, site), when the caller already holds it."""
    v, c = site_basis(cfg, block, site) if basis is None else basis
    rho, slow = planned_ratios(cfg, block, site, n_steps)
    n = rho.size
    rng = _rng(cfg.cid, block, site, _S_TOKENS)
    z = rng.standard_normal((n, cfg.k))
    w = rng.standard_normal((n, c.shape[1]))
    r = rho.reshape(-1)
    s = r * np.linalg.norm(z, axis=1) / (np.linalg.norm(w, axis=1) * np.sqrt(1.0 - r * r))
    x = z @ v.T + (s[:, None] * w) @ c.T
    return store(x, cfg.dtype), slow.reshape(-1), r


@dataclass
class SiteInputs:
    block: int
    site: int
    d: int
    d_out: int
    V: torch.Tensor          # [d, k] stored dtype
    X: torch.Tensor          # [n_tokens, d] stored dtype
    planned_slow: np.ndarray  # [n_tokens] bool
    planned_rho: np.ndarray   # [n_tokens] float64

    def weight(self, cfg: Config) -> torch.Tensor:
        return site_weight(cfg, self.block, self.site)


def site_inputs(cfg: Config, block: int, site: int, n_steps: int | None = None) -> SiteInputs:
    shp = cfg.sites[site]
    v, _ = site_basis(cfg, block, site)
    x, slow, rho = site_tokens(cfg, block, site, n_steps)
    return SiteInputs(block, site, shp.d, shp.d_out, store(v, cfg.dtype), x, slow, rho)


def token_steps(cfg: Config) -> int:
    """Steps actually generated per site (pool size when the config cycles a pool)."""
    return cfg.token_pool_steps if cfg.token_pool_steps is not None else cfg.n_steps


def config_inputs(cfg: Config, blocks=None, n_steps: int | None = None, threads: int | None = None):
    """SiteInputs for every (block, site) of `blocks` (default: all), in decode order.

    Sites are generated concurrently, each worker with a single BLAS thread; results do not depend
    on the number of workers (every site has its own seeds). Depth-coherent chains are generated
    block by block within a site, so they stay serial per site.
    """
    from threadpoolctl import threadpool_limits

    blocks = list(range(cfg.n_blocks)) if blocks is None else list(blocks)
    keys = [(b, s) for b in blocks for s in range(len(cfg.sites))]
    if cfg.depth_rotation_deg is not None:
        # warm the per-site chains in parallel over sites, serially over blocks
        def chain(s):
            for b in range(max(blocks) + 1):
                site_basis(cfg, b, s)
        with threadpool_limits(limits=1), ThreadPoolExecutor(min(len(cfg.sites), threads or _threads())) as ex:
            list(ex.map(chain, range(len(cfg.sites))))
    with threadpool_limits(limits=1), ThreadPoolExecutor(threads or _threads()) as ex:
        return list(ex.map(lambda bs: site_inputs(cfg, bs[0], bs[1], n_steps), keys))
