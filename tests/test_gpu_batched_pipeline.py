"""GPU parity of the two-kernel batched path (16-bit weights, T >= 16) where its pipelining and
splits have edges: shapes whose K chunks are not multiples of 32 columns, several 64-token chunks
of one layer (each chunk's projection runs in the launch of the previous chunk's products),
stacks whose sites change mode from one site to the next (a dense site has no projection), and a
stack of mixed ranks (every site's buffers carved for the largest k). Gates bit for bit, y within
2e-2 relative L2 against the fp64 oracle [GSI §2.1-§2.2]."""
import numpy as np
import pytest
import torch

import synth
from oracle import gsi_oracle as orc
from tests.gpu_util import TOL, compare_site, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_rank_linear_amd as g
    assert g.gsi_device_check() == 0
    return g


def _planned_tokens(rng, V, C, eps, n, slow_frac):
    """Tokens with planned residual ratios, built from an orthonormal [V | C]."""
    k, m = V.shape[1], C.shape[1]
    slow = rng.random(n) < slow_frac
    rho = np.where(slow, rng.uniform(eps + 5e-3, min(2 * eps, 0.95), n), rng.uniform(eps / 2, eps - 5e-3, n))
    z = rng.standard_normal((n, k))
    w = rng.standard_normal((n, m))
    s = rho * np.linalg.norm(z, axis=1) / (np.linalg.norm(w, axis=1) * np.sqrt(1 - rho ** 2))
    return z @ V.T + (s[:, None] * w) @ C.T


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(192, 800, 32), (64, 1056, 64), (640, 96, 32), (128, 4128, 256), (1024, 640, 512)])
def test_two_kernel_ragged_shapes(g, dtype, shape):
    """d a multiple of 32 but not of 256 (K chunks of 8-column multiples, partial sub-chunks),
    d_out from one row tile up, k from 32 to 512; T = 16, 64 and 150 (chunks of 64, 64, 22)."""
    d_out, d, k = shape
    rng = np.random.default_rng(d_out * 13 + d * 3 + k)
    Q, R = np.linalg.qr(rng.standard_normal((d, min(d, k + 64))))
    Q = Q * np.sign(np.diag(R))
    V64, C64 = Q[:, :k], Q[:, k:]
    W = torch.from_numpy(rng.standard_normal((d_out, d)) * 0.05).to(dtype)
    V = torch.from_numpy(V64).to(dtype)
    eps = 0.2
    say(f"case: two-kernel ragged {shape} {dtype}")
    L = g.create_layer(W.cuda(), V.cuda())
    for T in (16, 64, 150):
        X = torch.from_numpy(_planned_tokens(rng, V64, C64, eps, T, 0.3)).to(dtype)
        ref = orc.forward(W, V, X, eps)
        keep = np.abs(ref["rho"] - eps) > 1e-3  # rounding can move a token to the line
        assert keep.mean() >= 0.9, f"T={T}: only {keep.sum()} of {T} tokens clear of the gate line"
        y = torch.zeros((T, d_out), dtype=dtype, device="cuda")
        gate = torch.full((T,), 9, dtype=torch.uint8, device="cuda")
        ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, d_out, d, k, T))
        g.gsi_forward(L, X.cuda().contiguous(), eps, y, gate, None, ws)
        torch.cuda.synchronize()
        assert g.gsi_workspace_status(ws) == 0
        n_slow = int(ref["gate"][keep].sum())
        err, worst = compare_site(to_np(y), gate.cpu().numpy(), ref, TOL["bf16"], where=f"{shape} T={T}", keep=keep)
        say(f"  T={T}: {n_slow} slow, y rel L2 {err:.2e}, worst token {worst:.2e}")


def _stack_run(g, sites, layers, modes, n, T_step, eps, dtype):
    stack = g.gsi_stack_create_modes(layers, modes)
    X = torch.cat([X for X, _, _ in sites], dim=1).contiguous().cuda()
    Y = torch.zeros((n, sum(W.shape[0] for _, W, _ in sites)), dtype=dtype, device="cuda")
    gates = torch.full((n, len(sites)), 7, dtype=torch.uint8, device="cuda")
    rho = torch.zeros((n, len(sites)), dtype=torch.float32, device="cuda")
    ws = g.new_workspace(g.gsi_stack_workspace_bytes(stack, T_step))
    g.gsi_stack_decode(stack, X, n // T_step, T_step, eps, Y, gates, rho, ws)
    torch.cuda.synchronize()
    assert g.gsi_workspace_status(ws) == 0
    out, o = [], 0
    for _, W, _ in sites:
        out.append(to_np(Y[:, o:o + W.shape[0]]))
        o += W.shape[0]
    stack.destroy()
    return out, gates.cpu().numpy()


@pytest.mark.parametrize("T_step", [64, 80])
def test_mixed_modes_pipelined(g, T_step):
    """Gated, static and dense sites in every order of neighbours (GPT-2-shaped blocks 0 and 1,
    fp16), two steps: the pipeline crosses sites, steps and (T_step = 80) 64-token chunks; a
    dense site's products run with no projection beside them."""
    cfg = synth.get(2)
    n = 2 * T_step
    say(f"case: mixed modes, batched stack, T_step={T_step}")
    modes = [0, 1, 2, 0, 2, 2, 1, 1]
    sites, layers, keep = [], [], []
    for s, m in enumerate(modes):
        si = synth.site_inputs(cfg, s // 4, s % 4, n_steps=n)
        W = synth.site_weight(cfg, s // 4, s % 4)
        Wd = W.cuda()
        keep.append(Wd)
        # dense sites 2 and 4 are dense layers; dense site 5 is a gated layer run in the dense mode
        L = g.create_dense_layer(Wd) if m == 2 and s != 5 else g.create_layer(Wd, si.V.cuda())
        layers.append(L)
        sites.append((si.X, W, si))
    ys, gates = _stack_run(g, sites, layers, modes, n, T_step, cfg.eps, torch.float16)
    for s, ((X, W, si), m) in enumerate(zip(sites, modes)):
        if m == 0:
            ref = orc.forward(W, si.V, X, cfg.eps)
        elif m == 1:
            ref = dict(orc.static_projection(W, si.V, X), gate=np.zeros(n, dtype=np.uint8))
        else:
            ref = {"y": orc.dense(W, X), "gate": np.ones(n, dtype=np.uint8)}
        err, _ = compare_site(ys[s], gates[:, s], ref, TOL["f16"], where=f"site {s} mode {m}")
        say(f"  site {s} mode {m}: y rel L2 {err:.2e}")


def test_mixed_ranks_pipelined(g):
    """GPT-2-shaped block 0 (fp16) with the bases of sites 1 and 3 cut to their first 64 columns
    (k = 64 beside k = 256) and their tokens planned against the cut basis (the next 128 columns
    as the complement), T_step = 64, two steps; gates are compared where the oracle's ratio is
    clear of the line (the stored basis is only nearly orthonormal)."""
    cfg = synth.get(2)
    n = 128
    rng = np.random.default_rng(2064)
    say("case: mixed ranks 256/64, batched stack, T_step=64")
    sites, layers, keep_dev, kept = [], [], [], []
    for s in range(4):
        si = synth.site_inputs(cfg, 0, s, n_steps=n)
        W = synth.site_weight(cfg, 0, s)
        if s % 2 == 0:
            V, X = si.V, si.X
        else:
            V = si.V[:, :64].contiguous()
            Vf = si.V.double().numpy()
            X = torch.from_numpy(_planned_tokens(rng, Vf[:, :64], Vf[:, 64:192], cfg.eps, n, 0.3)).to(torch.float16)
        Wd, Vd = W.cuda(), V.cuda()
        keep_dev += [Wd, Vd]
        layers.append(g.create_layer(Wd, Vd))
        sites.append((X, W, V))
    ys, gates = _stack_run(g, sites, layers, [0, 0, 0, 0], n, 64, cfg.eps, torch.float16)
    for s, (X, W, V) in enumerate(sites):
        ref = orc.forward(W, V, X, cfg.eps)
        keep = np.abs(ref["rho"] - cfg.eps) > 1e-3
        assert keep.mean() >= 0.9, f"site {s}: only {keep.sum()} of {n} tokens clear of the gate line"
        kept.append(int(keep.sum()))
        n_slow = int(ref["gate"][keep].sum())
        err, _ = compare_site(ys[s], gates[:, s], ref, TOL["f16"], where=f"site {s} k={V.shape[1]}", keep=keep)
        say(f"  site {s} k={V.shape[1]}: {n_slow} slow, y rel L2 {err:.2e}")
