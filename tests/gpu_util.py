"""Helpers for the GPU parity tests: upload synthetic sites, run libgsi, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import gsi_oracle as orc

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}   # relative L2 of y per (site, call)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


class Built:
    """A config's sites on the GPU plus the host copies the oracle needs."""

    def __init__(self, cfg, n_steps=None, blocks=None, keep_w_for=()):
        import gated_rank_linear_amd as g
        self.cfg = cfg
        self.blocks = list(range(cfg.n_blocks)) if blocks is None else list(blocks)
        self.sites = []     # (block, site, SiteInputs)
        self.layers = []
        self.W_host = {}
        self._dev = []
        for b in self.blocks:
            for s in range(len(cfg.sites)):
                si = synth.site_inputs(cfg, b, s, n_steps)
                W = synth.site_weight(cfg, b, s)
                if keep_w_for == "all" or (b, s) in keep_w_for:
                    self.W_host[(b, s)] = W
                Wd = W.cuda()
                Vd = si.V.cuda()
                L = g.create_layer(Wd, Vd)
                self._dev.append((Wd, Vd))
                self.sites.append((b, s, si))
                self.layers.append(L)
                del W
        torch.cuda.synchronize()
        self.n_tokens = self.sites[0][2].X.shape[0]
        self.x_ld = sum(si.d for _, _, si in self.sites)
        self.y_ld = sum(si.d_out for _, _, si in self.sites)
        self.dtype = self.sites[0][2].X.dtype

    def stacked_inputs(self) -> torch.Tensor:
        X = torch.cat([si.X for _, _, si in self.sites], dim=1).contiguous()
        return X.cuda()

    def split_outputs(self, Y: torch.Tensor):
        out, o = [], 0
        for _, _, si in self.sites:
            out.append(Y[:, o:o + si.d_out])
            o += si.d_out
        return out


def decode(built: Built, eps: float, T_step: int = 1, n_steps=None):
    import gated_rank_linear_amd as g
    st = g.gsi_stack_create(built.layers)
    n = built.n_tokens
    steps = n // T_step if n_steps is None else n_steps
    X = built.stacked_inputs()
    Y = torch.zeros((n, built.y_ld), dtype=built.dtype, device="cuda")
    gates = torch.full((n, len(built.layers)), 7, dtype=torch.uint8, device="cuda")
    rho = torch.zeros((n, len(built.layers)), dtype=torch.float32, device="cuda")
    ws = g.new_workspace(g.gsi_stack_workspace_bytes(st, T_step))
    g.gsi_stack_decode(st, X, steps, T_step, eps, Y, gates, rho, ws)
    torch.cuda.synchronize()
    assert g.gsi_workspace_status(ws) == 0, "in-kernel wait timed out"
    return Y, gates, rho, st


def compare_site(y_got, gate_got, ref: dict, tol: float, where: str = "", keep=None):
    """Parity of one site's outputs with the oracle's `ref` (a forward() result): gate bits exact,
    and y within `tol` relative L2 three ways: over the whole site, for every token on its own,
    and over the slow tokens alone (so that a wrong slow path cannot hide among the fast tokens).
    `keep` (bool per token) restricts the comparison to tokens whose gate is unique. Returns
    (site error, worst token error)."""
    gate_got = np.asarray(gate_got).astype(np.uint8)
    ref_gate = np.asarray(ref["gate"]).astype(np.uint8)
    y = np.asarray(y_got, dtype=np.float64)
    Y = np.asarray(ref["y"], dtype=np.float64)
    if keep is not None:
        keep = np.asarray(keep, dtype=bool)
        gate_got, ref_gate, y, Y = gate_got[keep], ref_gate[keep], y[keep], Y[keep]
    mism = np.nonzero(gate_got != ref_gate)[0]
    assert mism.size == 0, f"{where}: gate bits differ at tokens {mism[:10]}"
    err = rel_l2(y, Y)
    assert err <= tol, f"{where}: y rel L2 {err:.3e} > {tol}"
    den = np.linalg.norm(Y, axis=1)
    per = np.linalg.norm(y - Y, axis=1) / np.where(den > 0, den, 1.0)
    worst = float(per.max()) if per.size else 0.0
    if per.size:
        t = int(np.argmax(per))
        assert worst <= tol, f"{where}: token {t} (gate {ref_gate[t]}) y rel L2 {worst:.3e} > {tol}"
    slow = ref_gate == 1
    if slow.any():
        es = rel_l2(y[slow], Y[slow])
        assert es <= tol, f"{where}: slow tokens' y rel L2 {es:.3e} > {tol}"
    return err, worst


def check_site(built: Built, idx: int, Y_site: torch.Tensor, gate_col: torch.Tensor, eps: float, with_y: bool):
    b, s, si = built.sites[idx]
    ref_gate = orc.gate_only(si.V, si.X, eps)
    got_gate = gate_col.cpu().numpy().astype(np.uint8)
    rho = ref_gate["rho"]
    assert np.all(np.abs(rho - eps) > 1e-3), f"site {(b, s)}: generator margin violated"
    mism = np.nonzero(got_gate != ref_gate["gate"])[0]
    assert mism.size == 0, f"site {(b, s)}: gate bits differ at tokens {mism[:10]} rho={rho[mism[:10]]}"
    if not with_y:
        return None
    W = built.W_host[(b, s)]
    ref = orc.forward(W, si.V, si.X, eps)
    err, _ = compare_site(to_np(Y_site), got_gate, ref, TOL[built.cfg.dtype], where=f"site {(b, s)}")
    return err
