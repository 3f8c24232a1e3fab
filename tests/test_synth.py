"""The seeded generator produces the planned structure, checked with the oracle on stored values.

The realised residual ratio of every token (explicit residual on the rounded W/V/x, fp64 oracle)
must sit on the planned side of eps and at least 1e-3 away from it, so gate bits are unique.
"""
import math

import numpy as np
import torch
import pytest

import synth
from oracle import gsi_oracle as orc


def _margin_check(cfg, block, site, n_steps=None):
    si = synth.site_inputs(cfg, block, site, n_steps)
    out = orc.gate_only(si.V, si.X, cfg.eps)
    rho = out["rho"]
    assert np.all(np.abs(rho - cfg.eps) > 1e-3), f"margin violated: min {np.min(np.abs(rho - cfg.eps))}"
    assert np.array_equal(out["gate"].astype(bool), si.planned_slow), "realised gate differs from the plan"
    # fp64 ratio agrees with the fp32 decision
    assert np.array_equal(rho >= cfg.eps, si.planned_slow)
    return si, out


def test_config1_shape_and_fast_fraction():
    cfg = synth.get(1)
    si, out = _margin_check(cfg, 0, 0)
    assert si.X.shape == (64, 768) and si.V.shape == (768, 64)
    assert int(out["gate"].sum()) == 6                  # 58 of 64 fast
    W = synth.site_weight(cfg, 0, 0)
    assert W.shape == (768, 768) and W.dtype.is_floating_point
    assert abs(float(W.double().std()) * math.sqrt(768) - 1.0) < 0.01


def test_config1_basis_orthonormal_and_qr():
    cfg = synth.get(1)
    v, c = synth.site_basis(cfg, 0, 0)
    assert np.allclose(v.T @ v, np.eye(64), atol=1e-13)
    assert np.allclose(v.T @ c, 0.0, atol=1e-13)
    # V_k is exactly the Q of the QR of the first k Gaussian columns (sign-fixed)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=1001, spawn_key=(0, 0, 1))))
    g = rng.standard_normal((768, 64 + c.shape[1]))[:, :64]
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))
    assert np.allclose(q, v, atol=1e-12)


def test_config2_margins_and_depth_coherence():
    cfg = synth.get(2)
    for site in range(4):
        for block in (0, 5, 11):
            si, out = _margin_check(cfg, block, site)
            assert int(out["gate"].sum()) == 13
    # consecutive bases: every principal angle is 25 degrees (cosine 0.906 > 0.90)
    for site in range(4):
        for block in range(1, 12):
            v0, _ = synth.site_basis(cfg, block - 1, site)
            v1, _ = synth.site_basis(cfg, block, site)
            cos = np.linalg.svd(v0.T @ v1, compute_uv=False)
            assert np.allclose(cos, math.cos(math.radians(25.0)), atol=1e-12)
            assert np.allclose(v1.T @ v1, np.eye(cfg.k), atol=1e-12)


@pytest.mark.parametrize("cid,blocks", [(3, (0, 27)), (4, (0, 31))])
def test_large_configs_margins_sampled(cid, blocks):
    cfg = synth.get(cid)
    n_slow = 0
    n = 0
    for block in blocks:
        for site in range(4):
            si, out = _margin_check(cfg, block, site, n_steps=cfg.n_steps if cid == 3 else 128)
            n_slow += int(out["gate"].sum())
            n += out["gate"].size
            assert si.X.dtype == synth.generate.TORCH_DTYPE["bf16"]
    if cid == 3:
        assert n_slow == len(blocks) * 4          # exactly one slow token per site
    else:
        assert 0.10 < n_slow / n < 0.20            # about 15% slow


def test_config5_binomial_plan():
    cfg = synth.get(5)
    rho, slow = synth.planned_ratios(cfg, 0, 0, n_steps=200)
    frac = slow.mean()
    assert 0.17 < frac < 0.23
    assert (slow.sum(axis=1) >= 16).mean() > 0.05      # the MFMA slow branch is exercised
    assert np.all(np.abs(rho - cfg.eps) >= synth.PLAN_MARGIN - 1e-15)
    si, out = _margin_check(cfg, 0, 3, n_steps=2)
    assert si.X.shape == (128, 16384)


def test_seeds_reproducible():
    cfg = synth.get(2)
    a = synth.site_inputs(cfg, 3, 1)
    b = synth.site_inputs(cfg, 3, 1)
    assert a.X.equal(b.X) and a.V.equal(b.V)
    w1 = synth.site_weight(cfg, 3, 1)
    w2 = synth.site_weight(cfg, 3, 1)
    assert w1.equal(w2)
    c = synth.site_inputs(cfg, 3, 2)
    assert not a.X[:, :8].equal(c.X[:, :8])


@pytest.mark.parametrize("k", [64, 128, 256, 512])
def test_sweep_points_margins(k):
    """Operating-point sweep inputs (GPT-J-shaped sites at rank k): at every slow count, the
    realised gates equal the plan, with the 1e-3 margin, so the fast fraction is the one planned."""
    import dataclasses
    from synth.configs import SWEEP_SLOW_COUNTS, SlowPlan, sweep_config
    from synth.generate import site_basis, site_tokens
    cfg = sweep_config(k)
    for site in range(4):
        basis = site_basis(cfg, 0, site)
        V = synth.store(basis[0], cfg.dtype)
        for n_slow in SWEEP_SLOW_COUNTS:
            c = dataclasses.replace(cfg, slow=SlowPlan("fixed", count=n_slow))
            X, planned, _ = site_tokens(c, 0, site, basis=basis)
            out = orc.gate_only(V, X, cfg.eps)
            assert np.all(np.abs(out["rho"] - cfg.eps) > 1e-3), (k, site, n_slow)
            assert np.array_equal(out["gate"].astype(bool), planned)
            assert int(out["gate"].sum()) == n_slow


def test_config6_shared_input_margins():
    """The shared-input variant (q/k/v and fc_in stacked into one 4096 -> 28672 site)."""
    cfg = synth.get(6)
    assert [s.d_out for s in cfg.sites] == [28672, 4096, 4096]
    for site in range(3):
        si, out = _margin_check(cfg, 0, site)
        assert int(out["gate"].sum()) == 1


def test_step_model_gates_and_margins():
    """The decode-step model (two GPT-2-width blocks): through the oracle's own chain every site's
    ratio stays more than 1e-2 from eps, the QKV and fc_in ratios follow the planned ones, and both
    gates occur; the model's tensors are row-major in the storage dtype."""
    from oracle import gsi_oracle as orc
    from oracle import gsi_step as ostep
    from synth.step import step_config, step_model

    cfg = step_config(71)
    m = step_model(cfg)
    for hb in m["blocks"]:
        for n in ("qkv", "out", "fc_in", "fc_out"):
            W, V = hb[n]
            assert W.is_contiguous() and V.is_contiguous() and W.dtype == V.dtype == torch.float16
    gates, rhos = [], []
    for t in range(cfg.n_tokens):
        x = orc.as_f64(m["x0"][t])
        for b, hb in enumerate(m["blocks"]):
            r = ostep.decode_block(x, hb, orc.as_f64(hb["K"]), orc.as_f64(hb["V"]), cfg.L0 + t, cfg.eps, cfg.n_heads)
            assert np.all(np.abs(r["rho"] - cfg.eps) > 1e-2), (t, b, r["rho"])
            assert abs(r["rho"][0] - float(m["planned_rho"][t])) < 5e-3 and abs(r["rho"][2] - r["rho"][0]) < 5e-3
            gates.append(r["gates"])
            x = r["x_next"]
    gates = np.array(gates)
    assert 0 < gates.sum() < gates.size
