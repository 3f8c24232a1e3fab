"""GPU parity of the decode-step block (gsi_block_step): GSI sites embedded in an unchanged plain
attention [GSI §3 item 4, §5], GPT-J-shaped parallel blocks on the synthetic step model.

Each call is checked op by op against the fp64 oracle applied to the GPU's own stored inputs of
that op (teacher forcing): LayerNorm, the four sites (gates bit for bit where the oracle's ratio
is more than 1e-3 from eps, y within 2e-2), the cache row written, attention, GELU and the
residual add (within 8e-3, one rounding to the 16-bit type). A chain run from the embeddings is
then compared with the oracle's own chain."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import gsi_oracle as orc
from oracle import gsi_step as ostep
from synth.step import step_config, step_model
from tests.gpu_util import TOL, compare_site, rel_l2, say, to_np

pytestmark = pytest.mark.gpu

OP_TOL = 8e-3
SITES_A = ("qkv", "fc_in")
SITES_B = ("out", "fc_out")


@pytest.fixture(scope="module")
def g():
    import gated_rank_linear_amd as g
    assert g.gsi_device_check() == 0
    return g


class Model:
    """The synthetic step model on the GPU: per block two stacks, LayerNorm parameters, caches.
    shared: stack A is one shared-input site (QKV and fc_in rows stacked on their common basis)."""

    def __init__(self, g, cfg, shared=False):
        self.cfg = cfg
        self.shared = shared
        self.host = step_model(cfg)
        self.blocks = []
        self.keep = []
        for hb in self.host["blocks"]:
            dev = {n: (hb[n][0].cuda(), hb[n][1].cuda()) for n in SITES_A + SITES_B}
            layers = {n: g.create_layer(*dev[n]) for n in dev}
            if shared:
                assert hb["qkv"][1] is hb["fc_in"][1]  # one basis for the block's LayerNorm output
                Wc = torch.cat([dev["qkv"][0], dev["fc_in"][0]], dim=0).contiguous()
                layers["qkv_fc_in"] = g.create_layer(Wc, dev["qkv"][1])
                A = g.gsi_stack_create([layers["qkv_fc_in"]])
            else:
                A = g.gsi_stack_create([layers[n] for n in SITES_A])
            B = g.gsi_stack_create([layers[n] for n in SITES_B])
            blk = {"A": A, "B": B, "gamma": hb["gamma"].cuda(), "beta": hb["beta"].cuda(),
                   "K": hb["K"].cuda(), "V": hb["V"].cuda(), "layers": layers, "dev": dev}
            self.blocks.append(blk)
        torch.cuda.synchronize()
        d, dff = cfg.d, cfg.d_ff
        dt = self.host["x0"].dtype
        self.xa = torch.zeros(2 * d, dtype=dt, device="cuda")
        self.ya = torch.zeros(3 * d + dff, dtype=dt, device="cuda")
        self.xb = torch.zeros(d + dff, dtype=dt, device="cuda")
        self.yb = torch.zeros(2 * d, dtype=dt, device="cuda")
        self.gates = torch.zeros(4, dtype=torch.uint8, device="cuda")
        self.rho = torch.zeros(4, dtype=torch.float32, device="cuda")
        b0 = self.blocks[0]
        self.ws = g.new_workspace(g.gsi_block_step_workspace_bytes(b0["A"], b0["B"], cfg.n_heads))

    def step(self, g, b, x, pos):
        blk = self.blocks[b]
        g.gsi_block_step(blk["A"], blk["B"], blk["gamma"], blk["beta"], x, blk["K"], blk["V"], pos,
                         self.cfg.n_heads, self.cfg.eps, self.xa, self.ya, self.xb, self.yb, self.gates, self.rho,
                         self.ws)

    def destroy(self):
        for blk in self.blocks:
            blk["A"].destroy()
            blk["B"].destroy()


def _site_check(W, V, x_in, y_got, gate_got, eps, dt, where, tally):
    """One site call: gate bit for bit and y within tolerance where the oracle's ratio is clear of
    the line; within 1e-3 of it either gate is valid and y is compared with that gate's path."""
    ref = orc.forward(W, V, x_in[None], eps)
    clear = bool(abs(ref["rho"][0] - eps) > 1e-3)
    tally.append(clear)
    if not clear:
        ref = orc.forward(W, V, x_in[None], 0.0 if gate_got else 1.5)  # that path for this token
    compare_site(y_got[None], np.array([gate_got]), ref, TOL["bf16"], where=where)
    return int(ref["gate"][0])


def _teacher_forced(g, model, n_tokens):
    cfg = model.cfg
    d, dff, H = cfg.d, cfg.d_ff, cfg.n_heads
    tally, n_slow = [], 0
    for t in range(n_tokens):
        x = model.host["x0"][t].cuda().clone()
        pos = cfg.L0 + t
        for b in range(cfg.n_blocks):
            hb = model.host["blocks"][b]
            blk = model.blocks[b]
            x_before = to_np(x)
            model.step(g, b, x, pos)
            torch.cuda.synchronize()
            assert g.gsi_workspace_status(model.ws) == 0
            xa, ya, xb, yb = (to_np(v) for v in (model.xa, model.ya, model.xb, model.yb))
            gates = model.gates.cpu().numpy()
            where = f"token {t} block {b}"
            if model.shared:  # one gate and one ratio, reported for QKV and fc_in alike
                rho = model.rho.cpu().numpy()
                assert gates[0] == gates[1] and rho[0] == rho[1], f"{where}: {gates} {rho}"
            # LayerNorm of the stored x, written twice
            assert np.array_equal(xa[:d], xa[d:]), where
            e = rel_l2(xa[:d], ostep.layer_norm(x_before, hb["gamma"], hb["beta"]))
            assert e <= OP_TOL, f"{where}: LayerNorm rel L2 {e:.2e}"
            # stack A on the GPU's a
            n_slow += _site_check(*hb["qkv"], xa[:d], ya[:3 * d], gates[0], cfg.eps, model.xa.dtype, f"{where} qkv", tally)
            n_slow += _site_check(*hb["fc_in"], xa[:d], ya[3 * d:], gates[1], cfg.eps, model.xa.dtype, f"{where} fc_in", tally)
            # the new k and v joined the caches bit for bit
            Kc, Vc = to_np(blk["K"][:pos + 1]), to_np(blk["V"][:pos + 1])
            assert np.array_equal(Kc[pos], ya[d:2 * d]) and np.array_equal(Vc[pos], ya[2 * d:3 * d]), where
            e = rel_l2(xb[:d], ostep.attention_decode(ya[:d], Kc, Vc, H))
            assert e <= OP_TOL, f"{where}: attention rel L2 {e:.2e}"
            e = rel_l2(xb[d:], ostep.gelu_tanh(ya[3 * d:]))
            assert e <= OP_TOL, f"{where}: GELU rel L2 {e:.2e}"
            # stack B on the GPU's o and u
            n_slow += _site_check(*hb["out"], xb[:d], yb[:d], gates[2], cfg.eps, model.xa.dtype, f"{where} out", tally)
            n_slow += _site_check(*hb["fc_out"], xb[d:], yb[d:], gates[3], cfg.eps, model.xa.dtype, f"{where} fc_out", tally)
            e = rel_l2(to_np(x), x_before + yb[:d] + yb[d:])
            assert e <= OP_TOL, f"{where}: residual rel L2 {e:.2e}"
    assert np.mean(tally) >= 0.9, f"only {sum(tally)} of {len(tally)} site calls clear of the gate line"
    return len(tally), n_slow


def test_step_blocks_teacher_forced(g):
    """GPT-2-shaped widths (d 768, 12 heads of 64, fp16), two blocks, six tokens after a 24-position
    prefix (two attention chunks per head)."""
    cfg = step_config(71)
    say(f"case: {cfg.name}, teacher-forced per op")
    model = Model(g, cfg)
    n, n_slow = _teacher_forced(g, model, cfg.n_tokens)
    say(f"  {n} site calls, {n_slow} slow")
    assert 0 < n_slow < n
    model.destroy()


def test_step_full_width_teacher_forced(g):
    """GPT-J-shaped widths (d 4096, 16 heads of 256, d_ff 16384, bf16), one block, eight tokens (two
    planned slow) after a 64-position prefix."""
    cfg = step_config(73)
    say(f"case: {cfg.name}, teacher-forced per op")
    model = Model(g, cfg)
    n, n_slow = _teacher_forced(g, model, cfg.n_tokens)
    say(f"  {n} site calls, {n_slow} slow")
    assert 0 < n_slow < n
    model.destroy()


def test_step_shared_input_teacher_forced(g):
    """Stack A as one shared-input site (QKV and fc_in stacked, d 4096 -> 28672, one basis, one g,
    one gate) at GPT-J-shaped widths: the same per-op checks, each map against its own site in the
    oracle (the same basis and input give the same ratio), and one gate reported for both maps."""
    cfg = step_config(73)
    say(f"case: {cfg.name}, stack A as one shared-input site, teacher-forced per op")
    model = Model(g, cfg, shared=True)
    n, n_slow = _teacher_forced(g, model, cfg.n_tokens)
    say(f"  {n} site calls, {n_slow} slow")
    assert 0 < n_slow < n
    model.destroy()


def test_step_shared_input_chain(g):
    """Two GPT-2-shaped blocks with a shared-input stack A, six tokens chained through
    gsi_decode_step: the final rows against the oracle's float64 chain (within 3e-2) and against the
    two-site stack A's rows (within 3e-2: the same maps, different work splits)."""
    cfg = step_config(71)
    say(f"case: {cfg.name}, shared-input stack A, chained")
    ms, mt = Model(g, cfg, shared=True), Model(g, cfg)
    nb = cfg.n_blocks
    Kh = [orc.as_f64(hb["K"]) for hb in ms.host["blocks"]]
    Vh = [orc.as_f64(hb["V"]) for hb in ms.host["blocks"]]
    gates_all = torch.zeros((cfg.n_tokens, nb * 4), dtype=torch.uint8, device="cuda")
    for t in range(cfg.n_tokens):
        pos = cfg.L0 + t
        xs = ms.host["x0"][t].cuda().clone()
        xt = xs.clone()
        xo = orc.as_f64(ms.host["x0"][t])
        for m, x, gv in ((ms, xs, gates_all[t]), (mt, xt, None)):
            bl = m.blocks
            g.gsi_decode_step([k["A"] for k in bl], [k["B"] for k in bl], [k["gamma"] for k in bl],
                              [k["beta"] for k in bl], [k["K"] for k in bl], [k["V"] for k in bl], pos,
                              cfg.n_heads, cfg.eps, x, m.xa, m.ya, m.xb, m.yb,
                              gv if gv is not None else torch.zeros(nb * 4, dtype=torch.uint8, device="cuda"),
                              None, m.ws)
        torch.cuda.synchronize()
        for b in range(nb):
            r = ostep.decode_block(xo, ms.host["blocks"][b], Kh[b], Vh[b], pos, cfg.eps, cfg.n_heads)
            xo = r["x_next"]
        gv = gates_all[t].cpu().numpy().reshape(nb, 4)
        assert np.array_equal(gv[:, 0], gv[:, 1]), f"token {t}: {gv}"
        e = rel_l2(to_np(xs), xo)
        assert e <= 3e-2, f"token {t}: final row rel L2 {e:.2e} against the oracle"
        e = rel_l2(to_np(xs), to_np(xt))
        assert e <= 3e-2, f"token {t}: final row rel L2 {e:.2e} against the two-site stack A"
    assert g.gsi_workspace_status(ms.ws) == 0
    ms.destroy()
    mt.destroy()


def test_step_long_cache(g):
    """A 2000-position prefix (43 attention chunks per head at 12 heads), two tokens."""
    cfg = dataclasses.replace(step_config(71), L0=2000, n_tokens=2, n_blocks=1)
    say(f"case: {cfg.name} with a 2000-position prefix")
    model = Model(g, cfg)
    _teacher_forced(g, model, cfg.n_tokens)
    model.destroy()


def test_step_chain_matches_oracle_chain(g):
    """Two blocks, six tokens from the embeddings, each block's output feeding the next: the GPU's
    final rows and gates against the oracle's own float64 chain (gates compared where the oracle's
    ratio is more than 1e-2 from eps; the rows within 3e-2, the chain's roundings compound)."""
    cfg = step_config(71)
    say(f"case: {cfg.name}, chained")
    model = Model(g, cfg)
    d = cfg.d
    Kh = [orc.as_f64(hb["K"]) for hb in model.host["blocks"]]
    Vh = [orc.as_f64(hb["V"]) for hb in model.host["blocks"]]
    worst = 0.0
    for t in range(cfg.n_tokens):
        x = model.host["x0"][t].cuda().clone()
        xo = orc.as_f64(model.host["x0"][t])
        pos = cfg.L0 + t
        for b in range(cfg.n_blocks):
            model.step(g, b, x, pos)
            torch.cuda.synchronize()
            r = ostep.decode_block(xo, model.host["blocks"][b], Kh[b], Vh[b], pos, cfg.eps, cfg.n_heads)
            gates = model.gates.cpu().numpy()[[0, 2, 1, 3]]  # GPU order QKV, fc_in, out, fc_out
            clear = np.abs(r["rho"] - cfg.eps) > 1e-2
            assert np.array_equal(gates[clear], r["gates"][clear]), f"token {t} block {b}: gates {gates} vs {r['gates']}"
            xo = r["x_next"]
        e = rel_l2(to_np(x), xo)
        worst = max(worst, e)
        assert e <= 3e-2, f"token {t}: final row rel L2 {e:.2e}"
    say(f"  worst final-row rel L2 {worst:.2e}")
    model.destroy()


def test_block_step_rejects_bad_shapes(g):
    """Stacks in the wrong order, a head count that does not divide d, a head width outside
    {64, 128, 256}: GSI_ERR_SHAPE before anything is enqueued."""
    cfg = step_config(71)
    model = Model(g, cfg)
    blk = model.blocks[0]
    x = model.host["x0"][0].cuda().clone()
    for A, B, H in ((blk["B"], blk["A"], 12), (blk["A"], blk["B"], 7), (blk["A"], blk["B"], 24)):
        with pytest.raises(g.GsiError, match="GSI_ERR_SHAPE"):
            g.gsi_block_step(A, B, blk["gamma"], blk["beta"], x, blk["K"], blk["V"], cfg.L0, H, cfg.eps, model.xa,
                             model.ya, model.xb, model.yb, model.gates, model.rho, model.ws)
    with pytest.raises(g.GsiError, match="GSI_ERR_EPS"):
        g.gsi_block_step(blk["A"], blk["B"], blk["gamma"], blk["beta"], x, blk["K"], blk["V"], cfg.L0, 12, -1.0,
                         model.xa, model.ya, model.xb, model.yb, model.gates, model.rho, model.ws)
    model.destroy()


def test_decode_step_equals_block_calls(g):
    """gsi_decode_step over both blocks gives, bit for bit, the rows, gates and cache rows of the same
    blocks called one by one through gsi_block_step (six tokens)."""
    cfg = step_config(71)
    say(f"case: {cfg.name}, whole-step call against block calls")
    m1, m2 = Model(g, cfg), Model(g, cfg)
    nb = cfg.n_blocks
    gates_all = torch.zeros((cfg.n_tokens, nb * 4), dtype=torch.uint8, device="cuda")
    rho_all = torch.zeros((cfg.n_tokens, nb * 4), dtype=torch.float32, device="cuda")
    for t in range(cfg.n_tokens):
        pos = cfg.L0 + t
        x1 = m1.host["x0"][t].cuda().clone()
        x2 = x1.clone()
        g1 = []
        for b in range(nb):
            m1.step(g, b, x1, pos)
            g1.append(m1.gates.clone())
        bl = m2.blocks
        g.gsi_decode_step([k["A"] for k in bl], [k["B"] for k in bl], [k["gamma"] for k in bl],
                          [k["beta"] for k in bl], [k["K"] for k in bl], [k["V"] for k in bl], pos, cfg.n_heads,
                          cfg.eps, x2, m2.xa, m2.ya, m2.xb, m2.yb, gates_all[t], rho_all[t], m2.ws)
        torch.cuda.synchronize()
        assert torch.equal(x1, x2), f"token {t}: rows differ"
        assert torch.equal(torch.cat(g1), gates_all[t]), f"token {t}: gates differ"
        for b in range(nb):
            assert torch.equal(m1.blocks[b]["K"][pos], m2.blocks[b]["K"][pos])
            assert torch.equal(m1.blocks[b]["V"][pos], m2.blocks[b]["V"][pos])
    assert g.gsi_workspace_status(m2.ws) == 0
    m1.destroy()
    m2.destroy()


def test_decode_step_graph_replays_equal_eager(g):
    """One gsi_decode_step_devpos call captured in a HIP graph and replayed token after token (the
    position advanced on the device) gives, bit for bit, the rows, gates and cache rows of eager
    gsi_decode_step calls at the same positions; the first token runs the device-position call
    eagerly. Eager work and a synchronisation separate the replays."""
    cfg = step_config(71)
    say(f"case: {cfg.name}, captured step replayed against eager steps")
    m1, m2 = Model(g, cfg), Model(g, cfg)
    nb, n = cfg.n_blocks, cfg.n_tokens
    b1, b2 = m1.blocks, m2.blocks
    lists = lambda bl: ([k["A"] for k in bl], [k["B"] for k in bl], [k["gamma"] for k in bl],
                        [k["beta"] for k in bl], [k["K"] for k in bl], [k["V"] for k in bl])
    pos_dev = torch.tensor([cfg.L0], dtype=torch.int32, device="cuda")
    xg = torch.zeros_like(m2.host["x0"][0], device="cuda")
    gates_g = torch.zeros(nb * 4, dtype=torch.uint8, device="cuda")
    rho_g = torch.zeros(nb * 4, dtype=torch.float32, device="cuda")
    gates_e = torch.zeros(nb * 4, dtype=torch.uint8, device="cuda")
    rho_e = torch.zeros(nb * 4, dtype=torch.float32, device="cuda")
    step2 = lambda: g.gsi_decode_step_devpos(*lists(b2), pos_dev, cfg.n_heads, cfg.eps, xg, m2.xa, m2.ya, m2.xb,
                                             m2.yb, gates_g, rho_g, m2.ws)
    graph = None
    for t in range(n):
        pos = cfg.L0 + t
        x1 = m1.host["x0"][t].cuda().clone()
        g.gsi_decode_step(*lists(b1), pos, cfg.n_heads, cfg.eps, x1, m1.xa, m1.ya, m1.xb, m1.yb, gates_e, rho_e,
                          m1.ws)
        xg.copy_(m2.host["x0"][t].cuda())
        if t == 0:
            step2()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step2()
        else:
            graph.replay()
        torch.cuda.synchronize()
        assert int(pos_dev.item()) == pos + 1, f"token {t}: position not advanced"
        assert torch.equal(x1, xg), f"token {t}: rows differ"
        assert torch.equal(gates_e, gates_g), f"token {t}: gates differ"
        assert torch.equal(rho_e, rho_g), f"token {t}: ratios differ"
        for b in range(nb):
            assert torch.equal(b1[b]["K"][pos], b2[b]["K"][pos]), f"token {t} block {b}: key row"
            assert torch.equal(b1[b]["V"][pos], b2[b]["V"][pos]), f"token {t} block {b}: value row"
    assert g.gsi_workspace_status(m2.ws) == 0
    del graph
    m1.destroy()
    m2.destroy()
