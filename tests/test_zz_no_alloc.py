"""gsi_stack_decode_noalloc (the batch-1 stack decode with its exchange state in a file-scope
device array) against gsi_stack_decode with a caller workspace: two calls in a row through the C
ABI, the second with a smaller input, on GPT-2-shaped fp16 sites (all three site modes) and a
GPT-J-shaped bf16 block; gate bits and y must be identical (same kernel, same data)."""
import ctypes

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


def _stack(g, cfg, blocks, n_tok, modes=None):
    sites, layers, keep = [], [], []
    for b in blocks:
        for s in range(len(cfg.sites)):
            si = synth.site_inputs(cfg, b, s, n_steps=n_tok)
            W = synth.site_weight(cfg, b, s)
            Wd = W.cuda()
            keep.append(Wd)
            layers.append(g.create_layer(Wd, si.V.cuda()))
            sites.append((si, W))
    st = g.gsi_stack_create(layers) if modes is None else g.gsi_stack_create_modes(layers, modes)
    torch.cuda.synchronize()
    return st, sites, keep


def _run(g, st, X, n_tok, T_step, eps, y_ld, n_sites, dtype, noalloc):
    Y = torch.full((n_tok, y_ld), 3.0, dtype=dtype, device="cuda")
    gates = torch.full((n_tok, n_sites), 7, dtype=torch.uint8, device="cuda")
    rho = torch.zeros((n_tok, n_sites), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = g.lib.gsi_stack_decode_noalloc(ctypes.c_void_p(st.handle), ctypes.c_void_p(X.data_ptr()),
                                            n_tok // T_step, T_step, ctypes.c_float(eps),
                                            ctypes.c_void_p(Y.data_ptr()), ctypes.c_void_p(gates.data_ptr()),
                                            ctypes.c_void_p(rho.data_ptr()), ctypes.c_void_p(stream))
        assert rc == 0, g.lib.gsi_status_string(rc)
    else:
        ws = g.new_workspace(g.gsi_stack_workspace_bytes(st, T_step))
        g.gsi_stack_decode(st, X, n_tok // T_step, T_step, eps, Y, gates, rho, ws)
        torch.cuda.synchronize()
        assert g.gsi_workspace_status(ws) == 0
    torch.cuda.synchronize()
    return Y, gates, rho


@pytest.mark.parametrize("cid,blocks,modes,T_step", [
    (2, [0, 1], None, 1),
    (2, [0, 1], [0, 1, 2, 0, 1, 0, 2, 0], 3),
    (3, [0], None, 1),
])
def test_noalloc_matches_workspace_entry_point(g, cid, blocks, modes, T_step):
    cfg = synth.get(cid)
    dtype = torch.float16 if cfg.dtype == "f16" else torch.bfloat16
    n_tok = 48
    say(f"case: no-allocation decode, config {cid}, blocks {blocks}, modes {modes}, T_step {T_step}")
    st, sites, keep = _stack(g, cfg, blocks, n_tok, modes)
    X = torch.cat([si.X for si, _ in sites], dim=1).contiguous().cuda()
    y_ld = sum(si.d_out for si, _ in sites)
    for n in (n_tok, 18):   # two calls in a row, the second smaller
        n -= n % T_step
        Xn = X[:n].contiguous()
        Yr, Gr, Rr = _run(g, st, Xn, n, T_step, cfg.eps, y_ld, len(sites), dtype, noalloc=False)
        Yn, Gn, Rn = _run(g, st, Xn, n, T_step, cfg.eps, y_ld, len(sites), dtype, noalloc=True)
        assert torch.equal(Gn, Gr), f"n={n}: gate bits differ"
        assert torch.equal(Yn, Yr), f"n={n}: y differs"
        assert torch.equal(torch.nan_to_num(Rn, nan=-1.0), torch.nan_to_num(Rr, nan=-1.0)), f"n={n}: rho differs"
        # and both against the oracle on the first site
        si, W = sites[0]
        m = 0 if modes is None else modes[0]
        ref = orc.forward(W, si.V, si.X[:n], cfg.eps) if m == 0 else None
        if ref is not None:
            compare_site(to_np(Yn[:, :si.d_out]), Gn[:, 0].cpu().numpy(), ref, TOL[cfg.dtype], where=f"n={n}")
    st.destroy()


def test_noalloc_rejects_what_it_cannot_hold(g):
    """T_step >= 16 needs the batched path's scratch, which the fixed array does not hold."""
    cfg = synth.get(1)
    si = synth.site_inputs(cfg, 0, 0)
    W = synth.site_weight(cfg, 0, 0).cuda()
    L = g.create_layer(W, si.V.cuda())
    st = g.gsi_stack_create([L])
    p = ctypes.c_void_p(si.X.cuda().data_ptr())
    rc = g.lib.gsi_stack_decode_noalloc(ctypes.c_void_p(st.handle), p, 1, 16, ctypes.c_float(0.1), p, p, None, None)
    assert rc == -5   # GSI_ERR_WORKSPACE
    rc = g.lib.gsi_stack_decode_noalloc(ctypes.c_void_p(st.handle), p, 1, 1, ctypes.c_float(-1.0), p, p, None, None)
    assert rc == -4
    st.destroy()
