"""The five synthetic GSI workloads: shapes, dtypes, operating points.

Shapes follow the models the GSI summary page (gist.science, arXiv 2605.03109) names in its
experimental section (§4): GPT-2 124M, GPT-J 6B and OPT 6.7B. The operating points k = 256,
eps in {0.05, 0.10}, and the 99.8% fast fraction for GPT-J come from the same section.

A *site* is one distinct linear-layer input inside a block. q, k and v read the same input, so
they are one site whose weight is the three projections stacked row-wise (d_out = 3 * d_model);
every other map is its own site. This module holds shapes only, no arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Site:
    name: str
    d: int        # input width (columns of W, rows of V_k)
    d_out: int    # output width (rows of W and of M)


@dataclass(frozen=True)
class SlowPlan:
    """How the generator places slow-path tokens.

    kind == "fixed":     exactly `count` slow tokens per (site, step), at seeded positions.
    kind == "lognormal": target ratio rho* = eps * exp(xi - shift), xi ~ N(0, 1); a token is slow
                         iff rho* > eps. `shift` = 1.0364 (the 0.85 normal quantile) makes
                         P(slow) = 0.15.
    kind == "binomial":  slow count per (site, step) ~ Bin(t_step, p), positions from a seeded
                         permutation.
    """
    kind: str
    count: int = 0
    p: float = 0.0
    shift: float = 0.0


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str                 # "f32" | "f16" | "bf16": weights, basis and activations
    n_blocks: int
    sites: tuple
    k: int
    eps: float
    t_step: int                # tokens per call (1 = batch-1 decode)
    n_steps: int               # calls per site (decode length for batch-1)
    slow: SlowPlan
    w_std: float | None        # None: 1/sqrt(d)
    depth_rotation_deg: float | None = None   # block l+1 basis rotated from block l's
    token_pool_steps: int | None = None       # steps generated and then cycled (memory bound)
    notes: str = ""
    m_complement: int = 256    # width of the orthonormal complement the residual noise lives in

    @property
    def n_sites(self) -> int:
        return self.n_blocks * len(self.sites)

    @property
    def n_tokens(self) -> int:
        return self.t_step * self.n_steps

    def site_list(self):
        """Sites in decode order: block-major, then the order of `sites` inside a block."""
        return [(b, s, self.sites[s]) for b in range(self.n_blocks) for s in range(len(self.sites))]


GPT2_SITES = (Site("qkv", 768, 2304), Site("out", 768, 768), Site("fc", 768, 3072), Site("proj", 3072, 768))
GPTJ_SITES = (Site("qkv", 4096, 12288), Site("out", 4096, 4096), Site("fc_in", 4096, 16384),
              Site("fc_out", 16384, 4096))
# GPT-J's attention and MLP read the same block input (parallel residual), so q/k/v and fc_in can
# share one basis, one g and one gate: a single site with the four projections stacked
GPTJ_SHARED_SITES = (Site("qkv_fc_in", 4096, 28672), Site("out", 4096, 4096), Site("fc_out", 16384, 4096))
OPT_SITES = (Site("qkv", 4096, 12288), Site("out", 4096, 4096), Site("fc1", 4096, 16384),
             Site("fc2", 16384, 4096))

CONFIGS = {
    1: Config(1, "single-linear-fp32", "f32", 1, (Site("linear", 768, 768),), k=64, eps=0.10,
              t_step=64, n_steps=1, slow=SlowPlan("fixed", count=6), w_std=None,
              notes="one 768x768 layer; 58 of 64 tokens fast (~90%)"),
    2: Config(2, "gpt2-124m-stack-fp16", "f16", 12, GPT2_SITES, k=256, eps=0.10,
              t_step=1, n_steps=256, slow=SlowPlan("fixed", count=13), w_std=0.02,
              depth_rotation_deg=25.0, notes="13 of 256 tokens slow per site (~95% fast)"),
    3: Config(3, "gptj-6b-stack-bf16", "bf16", 28, GPTJ_SITES, k=256, eps=0.10,
              t_step=1, n_steps=512, slow=SlowPlan("fixed", count=1), w_std=0.02,
              notes="1 of 512 tokens slow per site (99.8% fast)"),
    4: Config(4, "opt-6.7b-stack-bf16", "bf16", 32, OPT_SITES, k=256, eps=0.05,
              t_step=1, n_steps=512, slow=SlowPlan("lognormal", shift=1.0364), w_std=0.02,
              notes="log-normal residual ratios, ~15% slow at random positions"),
    5: Config(5, "gptj-6b-batched-bf16", "bf16", 28, GPTJ_SITES, k=512, eps=0.10,
              t_step=64, n_steps=200, slow=SlowPlan("binomial", p=0.2), w_std=0.02,
              token_pool_steps=20, notes="T=64 per step, Bin(64, 0.2) slow tokens per (site, step)"),
    6: Config(6, "gptj-6b-shared-input-bf16", "bf16", 28, GPTJ_SHARED_SITES, k=256, eps=0.10,
              t_step=1, n_steps=512, slow=SlowPlan("fixed", count=1), w_std=0.02,
              notes="GPT-J-shaped stack with q/k/v and fc_in as one shared-input site (3 sites per block)"),
}


def get(cid: int) -> Config:
    return CONFIGS[cid]


SWEEP_RANKS = (64, 128, 256, 512)
# slow tokens per site out of 512: fast fractions 1, 0.998 (the GPT-J operating point), 0.949,
# 0.85, 0.5 and 0
SWEEP_SLOW_COUNTS = (0, 1, 26, 77, 256, 512)


def sweep_config(k: int) -> Config:
    """The GPT-J-shaped stack at rank k and eps = 0.10, for the operating-point sweep (registered
    under its own id, so every rank has its own bases and tokens). The slow plan is replaced per
    sweep point with dataclasses.replace(cfg, slow=SlowPlan("fixed", count=n))."""
    cid = 600 + k
    if cid not in CONFIGS:
        CONFIGS[cid] = Config(cid, f"gptj-6b-sweep-k{k}-bf16", "bf16", 28, GPTJ_SITES, k=k, eps=0.10,
                              t_step=1, n_steps=512, slow=SlowPlan("fixed", count=1), w_std=0.02,
                              notes="operating-point sweep: rank k, fixed slow count per site")
    return CONFIGS[cid]
