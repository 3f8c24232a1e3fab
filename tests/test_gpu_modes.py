"""GPU parity of the site modes against the fp64 oracle: static projection (gateless y = M g),
dense sites (y = W x) and a stack that gates only its MLP maps, through the batch-1 kernel
(T_step 1 and 5) and the batched path (T_step 64); a dense layer through gsi_forward."""
import numpy as np
import pytest
import torch

import synth
from oracle import gsi_oracle as orc
from tests.gpu_util import TOL, compare_site, rel_l2, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_rank_linear_amd as g
    assert g.gsi_device_check() == 0
    return g


def _sites(cfg, block, n_tok):
    out = []
    for s in range(len(cfg.sites)):
        si = synth.site_inputs(cfg, block, s, n_steps=n_tok)
        out.append((si, synth.site_weight(cfg, block, s)))
    return out


def _decode(g, stack, sites, T_step, eps, dtype):
    n = sites[0][0].X.shape[0]
    X = torch.cat([si.X for si, _ in sites], dim=1).contiguous().cuda()
    Y = torch.zeros((n, sum(si.d_out for si, _ in sites)), dtype=dtype, device="cuda")
    gates = torch.full((n, len(sites)), 7, dtype=torch.uint8, device="cuda")
    rho = torch.zeros((n, len(sites)), dtype=torch.float32, device="cuda")
    ws = g.new_workspace(g.gsi_stack_workspace_bytes(stack, T_step))
    g.gsi_stack_decode(stack, X, n // T_step, T_step, eps, Y, gates, rho, ws)
    torch.cuda.synchronize()
    assert g.gsi_workspace_status(ws) == 0
    ys, o = [], 0
    for si, _ in sites:
        ys.append(to_np(Y[:, o:o + si.d_out]))
        o += si.d_out
    return ys, gates.cpu().numpy(), rho.cpu().numpy()


@pytest.mark.parametrize("T_step", [1, 5, 64])
def test_mlp_only_stack(g, T_step):
    """One GPT-J-shaped block whose attention maps (QKV, out) are dense layers and whose MLP maps
    (fc_in, fc_out) are gated [GSI §2: the MLP-only predecessor]; 64 tokens."""
    cfg = synth.get(3)
    n = 64 - 64 % T_step
    say(f"case: MLP-only GPT-J-shaped block, T_step={T_step}")
    sites = _sites(cfg, 0, n)
    layers, keep = [], []
    for s, (si, W) in enumerate(sites):
        Wd = W.cuda()
        keep.append(Wd)
        layers.append(g.create_dense_layer(Wd) if s < 2 else g.create_layer(Wd, si.V.cuda()))
    stack = g.gsi_stack_create(layers)
    ys, gates, rho = _decode(g, stack, sites, T_step, cfg.eps, torch.bfloat16)
    for s, (si, W) in enumerate(sites):
        if s < 2:
            assert np.all(gates[:, s] == 1) and np.all(np.isnan(rho[:, s])), f"dense site {s}"
            ref = {"y": orc.dense(W, si.X), "gate": np.ones(n, dtype=np.uint8)}
        else:
            ref = orc.forward(W, si.V, si.X, cfg.eps)
        err, worst = compare_site(ys[s], gates[:, s], ref, TOL["bf16"], where=f"MLP-only site {s}")
        say(f"  site {s}: y rel L2 {err:.2e}, worst token {worst:.2e}")
    stack.destroy()


@pytest.mark.parametrize("T_step", [1, 64])
def test_static_projection_stack(g, T_step):
    """A GPT-2-shaped block (fp16) with every site in static-projection mode: y = M g for every
    token, gate 0, rho NaN, including the tokens the gate would send to the slow path
    [GSI §2.2 static projection; §4 negative control]."""
    cfg = synth.get(2)
    n = 64
    say(f"case: static projection, GPT-2-shaped block, T_step={T_step}")
    sites = _sites(cfg, 0, n)
    layers, keep = [], []
    for si, W in sites:
        Wd = W.cuda()
        keep.append(Wd)
        layers.append(g.create_layer(Wd, si.V.cuda()))
    stack = g.gsi_stack_create_modes(layers, [g.GSI_SITE_STATIC] * len(layers))
    ys, gates, rho = _decode(g, stack, sites, T_step, cfg.eps, torch.float16)
    n_gated_slow = 0
    for s, (si, W) in enumerate(sites):
        assert np.all(gates[:, s] == 0) and np.all(np.isnan(rho[:, s]))
        ref = orc.static_projection(W, si.V, si.X)
        n_gated_slow += int(orc.gate_only(si.V, si.X, cfg.eps)["gate"].sum())
        err, worst = compare_site(ys[s], gates[:, s], dict(ref, gate=np.zeros(n, dtype=np.uint8)), TOL["f16"],
                                  where=f"static site {s}")
        say(f"  site {s}: y rel L2 {err:.2e}, worst token {worst:.2e}")
    assert n_gated_slow > 0, "the inputs include tokens the gate would send to the slow path"
    stack.destroy()


@pytest.mark.parametrize("T", [1, 7, 40])
def test_dense_layer_forward(g, T):
    """gsi_forward on a dense layer: y = W x for every token, gate 1 (per-token kernel for T < 16,
    batched path from 16)."""
    rng = np.random.default_rng(31 + T)
    d_out, d = 1500, 1032
    W = torch.from_numpy(rng.standard_normal((d_out, d)) * 0.03).to(torch.bfloat16)
    X = torch.from_numpy(rng.standard_normal((T, d))).to(torch.bfloat16)
    say(f"case: dense layer forward T={T}")
    L = g.create_dense_layer(W.cuda())
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    gate = torch.full((T,), 9, dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(g.gsi_workspace_bytes(L.dtype, d_out, d, 0, T))
    g.gsi_forward(L, X.cuda().contiguous(), 0.1, y, gate, None, ws)
    torch.cuda.synchronize()
    assert g.gsi_workspace_status(ws) == 0
    ref = {"y": orc.dense(W, X), "gate": np.ones(T, dtype=np.uint8)}
    compare_site(to_np(y), gate.cpu().numpy(), ref, TOL["bf16"], where=f"dense T={T}")


def test_mixed_modes_follow_each_other(g):
    """Gated, static and dense sites in one stack, every order of neighbours, 16 tokens; a site's
    result does not depend on its neighbours' modes."""
    cfg = synth.get(2)
    n = 16
    say("case: mixed modes, GPT-2-shaped blocks 0 and 1")
    sites = _sites(cfg, 0, n) + _sites(cfg, 1, n)
    modes = [0, 1, 2, 0, 2, 2, 1, 1]
    layers, keep = [], []
    for s, ((si, W), m) in enumerate(zip(sites, modes)):
        Wd = W.cuda()
        keep.append(Wd)
        # dense sites 2 and 4 are dense layers; dense site 5 is a gated layer run in the dense mode
        layers.append(g.create_dense_layer(Wd) if m == 2 and s != 5 else g.create_layer(Wd, si.V.cuda()))
    stack = g.gsi_stack_create_modes(layers, modes)
    ys, gates, _ = _decode(g, stack, sites, 1, cfg.eps, torch.float16)
    for s, ((si, W), m) in enumerate(zip(sites, modes)):
        if m == 0:
            ref = orc.forward(W, si.V, si.X, cfg.eps)
        elif m == 1:
            ref = dict(orc.static_projection(W, si.V, si.X), gate=np.zeros(n, dtype=np.uint8))
        else:
            ref = {"y": orc.dense(W, si.X), "gate": np.ones(n, dtype=np.uint8)}
        compare_site(ys[s], gates[:, s], ref, TOL["f16"], where=f"site {s} mode {m}")
    stack.destroy()


def test_modes_rejected(g):
    """A dense layer cannot run gated or static; unknown modes are refused."""
    cfg = synth.get(1)
    si = synth.site_inputs(cfg, 0, 0)
    W = synth.site_weight(cfg, 0, 0).cuda()
    Ld = g.create_dense_layer(W)
    Lg = g.create_layer(W, si.V.cuda())
    for modes, layers in (([0], [Ld]), ([1], [Ld]), ([3], [Lg]), ([-1], [Lg])):
        with pytest.raises(g.GsiError, match="GSI_ERR_SHAPE"):
            g.gsi_stack_create_modes(layers, modes)
