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
    err = rel_l2(to_np(Y_site), ref["y"])
    tol = TOL[built.cfg.dtype]
    assert err <= tol, f"site {(b, s)}: y rel L2 {err:.3e} > {tol}"
    return err
