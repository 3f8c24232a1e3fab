"""Seeded synthetic model for the batch-1 decode step: a GPT-J-shaped stack of parallel blocks
(LayerNorm, QKV / out / fc_in / fc_out linear maps, plain attention, GELU) whose activations stay
near planted subspaces, so that the GSI gates see both fast and slow tokens.

Input generation only: this module draws random numbers, orthonormalises them with a library QR
and builds weights from random factors whose column spaces are chosen; it never forms a
projection, residual, ratio or gate of a token, and never runs the block.

Construction (d model width, r = k - 8 planted dimensions, B = an orthonormal basis of
span(S, 1) with S a random orthonormal d x r block and 1 the all-ones direction):
  * token embeddings x0 = S z + s C w with C orthonormal and orthogonal to B; s is solved so
    that the off-subspace part has a planned ratio rho* (fast tokens U(0.02, 0.08), slow ones
    U(0.13, 0.30), slow with probability 0.15). A LayerNorm with unit gain and zero shift keeps
    its output in span(B) plus the centred noise;
  * QKV site: W_q, W_k Gaussian; W_v = T_v R_v B^T + N_v (I - B B^T) with R_v and N_v Gaussian and
    T_v block-diagonal by head (head h's rows hold an orthonormal dh x m block, m = (k - 8) / heads),
    so v of a token in span(B) lies in span(T_v). Basis of the QKV and fc_in sites: B plus
    k - r - 1 random orthonormal columns;
  * out site: its input is, head by head, a softmax-weighted mean of cached values; a mixture
    taken per head stays in span(T_v) because T_v does not couple heads. The prefilled cache
    values are T_v c + small noise and the keys Gaussian. Basis: T_v plus random columns;
  * fc_in site: W_fc_in = 0.1 (T_f R_f B^T + N_f (I - B B^T)) (T_f orthonormal 4d x (r+1)), so its
    outputs are small (about 0.05) and GELU is close to z / 2 on them. fc_out basis: T_f plus
    random columns;
  * out and fc_out write into span(S): W_out = S A_out, W_fc_out = S A_fc, so the residual stream
    stays in span(S) plus the embedding's noise.
All of it is drawn in float64 (CPU) or float32 (a GPU device) with torch generators seeded per
(block, stream) from the workload's seed, then rounded to the storage dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class StepConfig:
    cid: int
    name: str
    dtype: str
    n_blocks: int
    d: int
    n_heads: int
    k: int
    eps: float
    L0: int         # prefilled cache positions
    n_tokens: int   # decode steps (one token each)
    slow_prob: float = 0.15

    @property
    def r(self) -> int:
        return self.k - 8

    @property
    def d_ff(self) -> int:
        return 4 * self.d


STEP_CONFIGS = {
    # GPT-2-124M-shaped widths (d 768, 12 heads), two blocks: the parity workload
    71: StepConfig(71, "gpt2-step-fp16", "f16", 2, 768, 12, 64, 0.10, 24, 6),
    # GPT-J-6B-shaped (d 4096, 16 heads of 256), 28 blocks, a 1024-position prefix: the measured one
    72: StepConfig(72, "gptj-step-bf16", "bf16", 28, 4096, 16, 256, 0.10, 1024, 64),
    # GPT-J-shaped widths, one block: the full-width parity workload
    73: StepConfig(73, "gptj-step-1block-bf16", "bf16", 1, 4096, 16, 256, 0.10, 64, 8),
}


def step_config(cid: int) -> StepConfig:
    return STEP_CONFIGS[cid]


def _gen(cfg: StepConfig, device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    seed = 9000 + cfg.cid
    for v in key:
        seed = seed * 1009 + v
    g.manual_seed(seed % (2 ** 63))
    return g


def _orth(a: torch.Tensor) -> torch.Tensor:
    q, r = torch.linalg.qr(a)
    s = torch.sign(torch.diagonal(r))
    s[s == 0] = 1
    return q * s


def _extend(lead: torch.Tensor, n: int, gen) -> torch.Tensor:
    """lead (orthonormal columns) followed by random orthonormal columns up to n in all."""
    g = torch.randn((lead.shape[0], n - lead.shape[1]), generator=gen, device=lead.device, dtype=lead.dtype)
    return _orth(torch.cat([lead, g], dim=1))


def step_model(cfg: StepConfig, device="cpu") -> dict:
    """The model's weights, bases, LayerNorm parameters, prefilled caches and token embeddings, in
    the storage dtype on `device`. blocks[b] holds "gamma", "beta", "qkv" / "out" / "fc_in" /
    "fc_out" as (W, V) pairs, and "K" / "V" caches of L0 + n_tokens rows (the first L0 filled).
    QKV and fc_in read the same input (the block's LayerNorm output), so they share one basis
    tensor: the two sites can run as one shared-input site (W stacked, one g, one gate)."""
    dev = torch.device(device)
    ft = torch.float64 if dev.type == "cpu" else torch.float32
    st = TORCH_DTYPE[cfg.dtype]
    d, r, k, dff = cfg.d, cfg.r, cfg.k, cfg.d_ff
    g0 = _gen(cfg, dev, 0)
    S = _orth(torch.randn((d, r), generator=g0, device=dev, dtype=ft))
    B = _orth(torch.cat([S, torch.full((d, 1), 1.0 / math.sqrt(d), device=dev, dtype=ft)], dim=1))
    G = torch.randn((d, min(d - r - 1, 256)), generator=g0, device=dev, dtype=ft)
    C = _orth(G - B @ (B.T @ G))
    # embeddings with planned off-subspace ratios
    n = cfg.n_tokens
    z = torch.randn((n, r), generator=g0, device=dev, dtype=ft) * math.sqrt(d / r)
    w = torch.randn((n, C.shape[1]), generator=g0, device=dev, dtype=ft)
    slow = torch.rand(n, generator=g0, device=dev, dtype=ft) < cfg.slow_prob
    lo = torch.where(slow, torch.full_like(z[:, 0], 0.13), torch.full_like(z[:, 0], 0.02))
    hi = torch.where(slow, torch.full_like(z[:, 0], 0.30), torch.full_like(z[:, 0], 0.08))
    rho = lo + (hi - lo) * torch.rand(n, generator=g0, device=dev, dtype=ft)
    s = rho * z.norm(dim=1) / (w.norm(dim=1) * torch.sqrt(1 - rho ** 2))
    x0 = z @ S.T + (s[:, None] * w) @ C.T
    off = lambda N: N - (N @ B) @ B.T  # N (I - B B^T)
    blocks = []
    for b in range(cfg.n_blocks):
        gb = _gen(cfg, dev, 1, b)
        rn = lambda *shape, scale=1.0: torch.randn(shape, generator=gb, device=dev, dtype=ft) * scale
        H, dh = cfg.n_heads, d // cfg.n_heads
        mh = (k - 8) // H
        Tv = torch.zeros((d, H * mh), device=dev, dtype=ft)
        for h in range(H):
            Tv[h * dh:(h + 1) * dh, h * mh:(h + 1) * mh] = _orth(rn(dh, mh))
        rv = H * mh
        Tf = _orth(rn(dff, r + 1))
        Wq = rn(d, d, scale=1 / math.sqrt(d))
        Wk = rn(d, d, scale=1 / math.sqrt(d))
        Wv = Tv @ rn(rv, r + 1, scale=1 / math.sqrt(r + 1)) @ B.T + off(rn(d, d, scale=1 / math.sqrt(d)))
        Wf = 0.1 * (Tf @ rn(r + 1, r + 1, scale=1 / math.sqrt(r + 1)) @ B.T + off(rn(dff, d, scale=1 / math.sqrt(d))))
        Wo = S @ rn(r, d, scale=0.3 / math.sqrt(d))
        Wm = S @ rn(r, dff, scale=1.0 / math.sqrt(dff))
        rs = lambda a: a.to(st).contiguous()  # row-major, in the storage dtype
        Va = rs(_extend(B, k, gb))  # the basis of the block's LayerNorm output, read by QKV and fc_in
        blk = {
            "gamma": torch.ones(d, device=dev, dtype=st), "beta": torch.zeros(d, device=dev, dtype=st),
            "qkv": (rs(torch.cat([Wq, Wk, Wv], dim=0)), Va),
            "out": (rs(Wo), rs(_extend(Tv, k, gb))),
            "fc_in": (rs(Wf), Va),
            "fc_out": (rs(Wm), rs(_extend(Tf, k, gb))),
        }
        K = torch.zeros((cfg.L0 + n, d), device=dev, dtype=st)
        V = torch.zeros((cfg.L0 + n, d), device=dev, dtype=st)
        K[:cfg.L0] = rn(cfg.L0, d).to(st)
        V[:cfg.L0] = (rn(cfg.L0, rv, scale=math.sqrt(d / rv)) @ Tv.T + rn(cfg.L0, d, scale=0.05)).to(st)
        blk["K"], blk["V"] = K, V
        blocks.append(blk)
    return {"blocks": blocks, "x0": x0.to(st).contiguous(), "planned_rho": rho.to(torch.float64).cpu(), "slow": slow.cpu()}
