"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Gate bits of every (token, site) are compared with the fp64 oracle (which needs only V and x);
y is compared on sampled sites (all of their tokens) where the oracle also needs W.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gsi_oracle as orc
from tests.gpu_util import TOL, Built, check_site, compare_site, decode, rel_l2, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_rank_linear_amd as g
    assert g.gsi_device_check() == 0
    return g


def _run_stack(cid, sample_sites, n_steps=None, T_step=1):
    cfg = synth.get(cid)
    say(f"case: config {cid} full stack ({cfg.n_blocks} blocks x {len(cfg.sites)} sites), T_step={T_step}")
    built = Built(cfg, n_steps=n_steps, keep_w_for=sample_sites)
    Y, gates, rho, _ = decode(built, cfg.eps, T_step=T_step)
    Ys = built.split_outputs(Y)
    n_slow = 0
    worst = 0.0
    for i, (b, s, si) in enumerate(built.sites):
        e = check_site(built, i, Ys[i], gates[:, i], cfg.eps, with_y=(b, s) in sample_sites)
        if e is not None:
            worst = max(worst, e)
    n_slow = int(gates.sum().item())
    say(f"  gates exact on {gates.numel()} (token, site) pairs, {n_slow} slow; worst sampled y rel L2 {worst:.2e}")
    return gates, worst


def test_config3_gptj_stack_batch1(g):
    cfg = synth.get(3)
    sample = {(0, 0), (0, 1), (0, 2), (0, 3), (cfg.n_blocks - 1, 0), (cfg.n_blocks - 1, 3)}
    gates, worst = _run_stack(3, sample)
    assert gates.shape == (cfg.n_tokens, cfg.n_sites)
    assert int(gates.sum()) == cfg.n_sites  # one slow token per site (99.8% fast)
    assert worst <= TOL["bf16"]


def test_config4_opt_stack_batch1(g):
    cfg = synth.get(4)
    sample = {(0, 0), (0, 2), (cfg.n_blocks - 1, 1), (cfg.n_blocks - 1, 3)}
    gates, worst = _run_stack(4, sample)
    frac = gates.float().mean().item()
    assert 0.10 < frac < 0.20, frac
    assert worst <= TOL["bf16"]


def test_config5_gptj_batched_T64(g):
    """The T = 64 workload exactly as the benchmark runs it: all 20 generated steps of the pool
    (1280 tokens per site), every gate bit of every (token, site), y of every token on three
    sites, one of each shape class (QKV, fc_out, fc_in) from the first and last blocks."""
    cfg = synth.get(5)
    sample = {(0, 0), (0, 3), (cfg.n_blocks - 1, 2)}
    gates, worst = _run_stack(5, sample, n_steps=cfg.token_pool_steps, T_step=cfg.t_step)
    assert gates.shape == (cfg.token_pool_steps * cfg.t_step, cfg.n_sites)
    frac = gates.float().mean().item()
    assert 0.1 < frac < 0.3, frac
    assert worst <= TOL["bf16"]


def _planned_tokens(rng, V, C, eps, n, slow_frac):
    """Tokens with planned residual ratios (by construction from an orthonormal [V | C])."""
    k, m = V.shape[1], C.shape[1]
    slow = rng.random(n) < slow_frac
    rho = np.where(slow, rng.uniform(eps + 5e-3, min(2 * eps, 0.95), n), rng.uniform(eps / 2, eps - 5e-3, n))
    z = rng.standard_normal((n, k))
    w = rng.standard_normal((n, m))
    s = rho * np.linalg.norm(z, axis=1) / (np.linalg.norm(w, axis=1) * np.sqrt(1 - rho ** 2))
    return z @ V.T + (s[:, None] * w) @ C.T


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(100, 40, 8), (257, 64, 32), (1000, 520, 64), (3, 24, 8), (700, 1032, 256)])
def test_ragged_shapes(g, dtype, shape):
    """Output rows not a multiple of the block split, d not a multiple of the lane tiles, k from 8
    up, T = 1, 5, 17, 37 (persistent and batched paths, tails everywhere)."""
    d_out, d, k = shape
    rng = np.random.default_rng(d_out * 7 + d + k)
    Q, R = np.linalg.qr(rng.standard_normal((d, min(d, k + 64))))
    Q = Q * np.sign(np.diag(R))
    V64, C64 = Q[:, :k], Q[:, k:]
    W = torch.from_numpy(rng.standard_normal((d_out, d)) * 0.05).to(dtype)
    V = torch.from_numpy(V64).to(dtype)
    eps = 0.2
    say(f"case: ragged {shape} {dtype}")
    L = g.create_layer(W.cuda(), V.cuda())
    for T in (1, 5, 17, 37):
        X = torch.from_numpy(_planned_tokens(rng, V64, C64, eps, T, 0.3)).to(dtype)
        ref_gate = orc.gate_only(V, X, eps)
        keep = np.abs(ref_gate["rho"] - eps) > 1e-3   # rounding can move a token to the line
        x = X.cuda().contiguous()
        y = torch.zeros((T, d_out), dtype=dtype, device="cuda")
        gate = torch.full((T,), 9, dtype=torch.uint8, device="cuda")
        ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, d_out, d, k, T))
        g.gsi_forward(L, x, eps, y, gate, None, ws)
        torch.cuda.synchronize()
        assert g.gsi_workspace_status(ws) == 0
        assert keep.mean() >= 0.9, f"T={T}: only {keep.sum()} of {T} tokens clear of the gate line"
        ref = orc.forward(W, V, X, eps)
        tol = TOL["f32"] if dtype == torch.float32 else TOL["bf16"]
        # gates and y compared where the gate is unique (tokens with a clear margin)
        compare_site(to_np(y), gate.cpu().numpy(), ref, tol, where=f"ragged {shape} T={T}", keep=keep)


def test_zero_tokens_is_a_no_op(g):
    cfg = synth.get(1)
    si = synth.site_inputs(cfg, 0, 0)
    L = g.create_layer(synth.site_weight(cfg, 0, 0).cuda(), si.V.cuda())
    x = torch.zeros((0, 768), device="cuda")
    y = torch.full((1, 768), 7.0, device="cuda")
    gate = torch.full((1,), 9, dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, 768, 768, 64, 1))
    rc = g.lib.gsi_forward(L.handle, x.data_ptr() or 16, 0, 0.1, y.data_ptr(), gate.data_ptr(), None,
                           ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.all(y == 7.0) and int(gate.item()) == 9


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(12300, 1024, 256), (6150, 1024, 256), (1000, 2048, 256), (3000, 1024, 512),
                                   (300, 4096, 512), (4096, 16384, 256), (200, 2560, 256)])
def test_precompute_tile_paths(g, dtype, shape, split):
    """The precompute M = W V on the matrix-core tile paths: with a create workspace, 128 x 256
    tiles split over K (2 to 16 chunks, ragged last row tiles, K chunks of 512 to 2048 columns)
    and V^T V - I split over K; without one, the 64-, 32- and 16-row tiles of the single-pass
    kernel (chosen by d_out), two 256-column tiles (k = 512) and the one-pass V^T V - I kernel.
    V^T V - I is checked through rho of single tokens (persistent path) against the oracle's
    residual norms."""
    d_out, d, k = shape
    rng = np.random.default_rng(d_out + 3 * d + k)
    Q, R = np.linalg.qr(rng.standard_normal((d, k + 32)))
    Q = Q * np.sign(np.diag(R))
    V64, C64 = Q[:, :k], Q[:, k:]
    W = torch.from_numpy(rng.standard_normal((d_out, d)) * 0.03).to(dtype)
    V = torch.from_numpy(V64).to(dtype)
    say(f"case: precompute tiles {shape} {dtype} split={split}")
    L = g.create_layer(W.cuda(), V.cuda(), split=split)
    torch.cuda.synchronize()
    M = to_np(g.layer_image(L))
    ref = orc.precompute_image(W, V)
    # one rounding to the 16-bit type on top of float32 accumulation
    assert rel_l2(M, ref) <= 4e-3, rel_l2(M, ref)
    # (V (V^T V - I))^T, the batched path's second projection, from aux's documented layout
    # against its definition on the stored V. V^T V - I is formed in float32, and its entries are
    # small (~4e-4 for bf16-rounded bases, ~2e-5 for fp16 ones), so the float32 sum error of V^T V
    # (~1e-7 sqrt(d)) weighs more for fp16: measured in a CPU emulation, 1.7e-3 - 3.3e-3 (bf16)
    # and up to 6e-2 (fp16, d = 16384) relative; a wrong row, column or operand part is O(1).
    es = 2
    a256 = lambda n: (n + 255) // 256 * 256
    off = a256(a256(k * d * es) + a256(k * k * 4) + 256 * 80)
    aux = L._keep[2]
    vdt = to_np(aux[off:off + k * d * es].view(dtype).view(k, d))
    V_st = orc.as_f64(V)
    ref_vdt = (V_st.T @ V_st - np.eye(k)) @ V_st.T
    assert rel_l2(vdt, ref_vdt) <= (1e-2 if dtype == torch.bfloat16 else 0.15), rel_l2(vdt, ref_vdt)
    eps = 0.2
    X = torch.from_numpy(_planned_tokens(rng, V64, C64, eps, 3, 0.5)).to(dtype)
    x = X.cuda().contiguous()
    y = torch.zeros((3, d_out), dtype=dtype, device="cuda")
    gate = torch.full((3,), 9, dtype=torch.uint8, device="cuda")
    rho = torch.zeros(3, dtype=torch.float32, device="cuda")
    ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, d_out, d, k, 3))
    g.gsi_forward(L, x, eps, y, gate, rho, ws)
    torch.cuda.synchronize()
    assert g.gsi_workspace_status(ws) == 0
    ref_rho = np.sqrt(orc.residual_norms(V, X) / orc.squared_norms(X))
    np.testing.assert_allclose(rho.cpu().numpy(), ref_rho, rtol=1e-4, atol=1e-6)
    ref_g = orc.gate_only(V, X, eps)
    keep = np.abs(ref_g["rho"] - eps) > 1e-3
    assert keep.mean() >= 0.9, f"only {keep.sum()} of 3 tokens clear of the gate line"
    assert np.array_equal(gate.cpu().numpy()[keep], ref_g["gate"][keep])


def test_config6_shared_input_block(g):
    """Shared-input sites: one GPT-J-shaped block whose q/k/v and fc_in form one 4096 -> 28672
    site (one basis, one g, one gate), then out and fc_out; 64 batch-1 tokens, 1 slow per site."""
    import dataclasses
    cfg = dataclasses.replace(synth.get(6), n_blocks=1, n_steps=64)
    say("case: config 6 shared-input block (3 sites, QKV+fc_in 4096->28672), 64 tokens")
    built = Built(cfg, blocks=[0], keep_w_for="all")
    Y, gates, _, _ = decode(built, cfg.eps)
    Ys = built.split_outputs(Y)
    worst = 0.0
    for i in range(len(built.sites)):
        worst = max(worst, check_site(built, i, Ys[i], gates[:, i], cfg.eps, with_y=True))
    say(f"  gates exact, worst y rel L2 {worst:.2e}")
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("eps", [0.0, 1.5])
def test_batched_all_slow_and_all_fast(g, dtype, eps):
    """T = 64 through the batched path with every token slow (eps = 0: the slow product on all
    four 16-row tiles, an empty fast list) or every token fast (eps = 1.5: the fast product on
    four tiles, an empty slow list), against the oracle."""
    d_out, d, k, T = 1000, 2048, 256, 64
    rng = np.random.default_rng(71)
    Q, R = np.linalg.qr(rng.standard_normal((d, k + 64)))
    Q = Q * np.sign(np.diag(R))
    W = torch.from_numpy(rng.standard_normal((d_out, d)) * 0.03).to(dtype)
    V = torch.from_numpy(Q[:, :k]).to(dtype)
    X = torch.from_numpy(_planned_tokens(rng, Q[:, :k], Q[:, k:], 0.1, T, 0.3)).to(dtype)
    say(f"case: batched T=64, eps={eps}, {dtype}")
    L = g.create_layer(W.cuda(), V.cuda())
    y = torch.zeros((T, d_out), dtype=dtype, device="cuda")
    gate = torch.full((T,), 9, dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, d_out, d, k, T))
    g.gsi_forward(L, X.cuda().contiguous(), eps, y, gate, None, ws)
    torch.cuda.synchronize()
    assert g.gsi_workspace_status(ws) == 0
    gb = gate.cpu().numpy()
    assert np.all(gb == (1 if eps == 0.0 else 0))
    ref = orc.forward(W, V, X, eps)
    err, worst = compare_site(to_np(y), gb, ref, TOL["bf16"], where=f"batched eps={eps}")
    say(f"  y rel L2 {err:.2e}, worst token {worst:.2e}")


@pytest.mark.parametrize("shape", [(64, 65536, 512), (262144, 64, 64)])
def test_maximum_sizes(g, shape):
    """The widest input the ABI accepts (d = 65536, at the largest rank 512: V rows and the input
    row far beyond an LDS region and the register window) and the most output rows (d_out =
    262144: 1024 rows of y per decode block, most of M read from HBM), bf16, per-token (T = 1, 3)
    and batched (T = 17) paths, against the oracle."""
    d_out, d, k = shape
    rng = np.random.default_rng(d_out + d + k)
    Q, R = np.linalg.qr(rng.standard_normal((d, min(d, k + 64))))
    Q = Q * np.sign(np.diag(R))
    V64, C64 = Q[:, :k], Q[:, k:]
    W = torch.from_numpy((rng.standard_normal((d_out, d)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(V64).to(torch.bfloat16)
    eps = 0.2
    say(f"case: maximum sizes {shape}")
    L = g.create_layer(W.cuda(), V.cuda())
    for T in (1, 3, 17):
        X = torch.from_numpy(_planned_tokens(rng, V64, C64, eps, T, 0.4)).to(torch.bfloat16)
        ref = orc.forward(W, V, X, eps)
        keep = np.abs(orc.gate_only(V, X, eps)["rho"] - eps) > 1e-3
        assert keep.mean() >= 0.9, f"T={T}: only {keep.sum()} of {T} tokens clear of the gate line"
        y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
        gate = torch.full((T,), 9, dtype=torch.uint8, device="cuda")
        ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, d_out, d, k, T))
        g.gsi_forward(L, X.cuda().contiguous(), eps, y, gate, None, ws)
        torch.cuda.synchronize()
        assert g.gsi_workspace_status(ws) == 0
        err, worst = compare_site(to_np(y), gate.cpu().numpy(), ref, TOL["bf16"], where=f"max {shape} T={T}",
                                  keep=keep)
        say(f"  T={T}: y rel L2 {err:.2e}, worst token {worst:.2e}")


@pytest.mark.parametrize("cid,blocks,n_tok,T_step", [(2, 2, 30, 2), (2, 2, 30, 15), (3, 1, 30, 15), (3, 1, 32, 16)])
def test_stack_small_steps(g, cid, blocks, n_tok, T_step):
    """Stacks decoded T_step tokens at a time: T_step 2 and 15 (the per-token kernel, sites in
    order within each step) and 16 (the batched path), on GPT-2-shaped fp16 and GPT-J-shaped bf16
    blocks; every gate bit and y of every token of every site against the oracle."""
    import dataclasses
    cfg = dataclasses.replace(synth.get(cid), n_blocks=blocks, n_steps=n_tok)
    say(f"case: config {cid}, {blocks} block(s), {n_tok} tokens, T_step={T_step}")
    built = Built(cfg, keep_w_for="all")
    Y, gates, _, _ = decode(built, cfg.eps, T_step=T_step)
    Ys = built.split_outputs(Y)
    worst = 0.0
    for i in range(len(built.sites)):
        worst = max(worst, check_site(built, i, Ys[i], gates[:, i], cfg.eps, with_y=True))
    say(f"  gates exact, worst site y rel L2 {worst:.2e}")
