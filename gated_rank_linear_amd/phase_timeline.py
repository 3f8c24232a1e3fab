"""Per-phase timeline of the batch-1 decode kernel (a profiling tool, not part of the library's
interface).

Loads the phase-stamp build of libgsi (`python -m gated_rank_linear_amd.build --phase-stamps`
makes _lib/libgsi_phases.so; libgsi itself carries no stamps), decodes 64 tokens through a
4-block GPT-J-shaped stack (QKV 4096->12288, out 4096->4096, fc_in 4096->16384, fc_out
16384->4096, bf16, every token fast) at k = 64 and k = 256, and prints, for the 16 site steps of
token 32, the median over three sampled blocks (0, 100, 200; their sync wave) of each phase's
wall-clock duration. Each stamp costs about 70 ns, so a stamped site is longer than an unstamped
one by roughly 0.6 us.

    python -m gated_rank_linear_amd.phase_timeline
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PHASE_LIB = os.path.join(HERE, "_lib", "libgsi_phases.so")
PHASES = ["A", "A->post", "post->E1", "E1->B", "B", "B->ypost", "ypost->E2", "E2->gate", "gate->ret"]


def main() -> None:
    if not os.path.exists(PHASE_LIB):
        raise SystemExit("build the phase-stamp library first: python -m gated_rank_linear_amd.build --phase-stamps")
    if os.environ.get("GSI_LIB") != PHASE_LIB:
        # the binding loads its library when the package is first imported (as `-m` does before
        # this runs): run again as a child process with the stamp build selected
        import subprocess
        env = dict(os.environ, GSI_LIB=PHASE_LIB)
        raise SystemExit(subprocess.run([sys.executable, os.path.abspath(__file__)], env=env).returncode)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import gated_rank_linear_amd as g
    from synth.configs import SlowPlan, sweep_config
    from synth.generate import site_basis, site_tokens, store

    assert os.path.samefile(g.LIB_PATH, PHASE_LIB), g.LIB_PATH
    lib = ctypes.CDLL(PHASE_LIB)
    for k in (64, 256):
        cfg = dataclasses.replace(sweep_config(k), n_steps=64, slow=SlowPlan("fixed", count=0))
        nb = 4
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1)
        bases = [site_basis(cfg, 0, s) for s in range(4)]
        layers, keep = [], []
        for _ in range(nb):
            for s, st in enumerate(cfg.sites):
                W = (torch.randn((st.d_out, st.d), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
                V = store(bases[s][0], "bf16").cuda()
                layers.append(g.create_layer(W, V))
                keep.append((W, V))
        stack = g.gsi_stack_create(layers)
        blk = torch.cat([site_tokens(cfg, 0, s, basis=bases[s])[0] for s in range(4)], dim=1)
        X = blk.repeat(1, nb).contiguous().cuda()
        Y = torch.zeros((64, sum(st.d_out for st in cfg.sites) * nb), dtype=torch.bfloat16, device="cuda")
        gates = torch.zeros((64, 16), dtype=torch.uint8, device="cuda")
        ws = g.new_workspace(g.gsi_stack_workspace_bytes(stack, 1))
        for _ in range(2):
            g.gsi_stack_decode(stack, X, 64, 1, cfg.eps, Y, gates, None, ws)
            torch.cuda.synchronize()
        if g.gsi_workspace_status(ws) != 0:
            raise SystemExit("decode kernel reported a wait timeout")
        buf = (ctypes.c_ulonglong * (3 * 16 * 11))()
        if lib.gsi_phase_stamps(buf) != 0:
            raise SystemExit("gsi_phase_stamps failed")
        a = np.frombuffer(buf, dtype=np.uint64).reshape(3, 16, 11).astype(np.float64) * 0.01  # us (100 MHz)
        print(f"k={k}: per-site phase durations (us), median over the 3 sampled blocks", flush=True)
        for s in range(16):
            d = np.diff(a[:, s, :10], axis=1)   # stamps 0..9 in order
            entry = a[:, s, 0] - a[:, s, 10]      # step entry (plan row, pointers) to phase A
            total = a[:, s, 9] - a[:, s, 10]
            gap = (a[:, s + 1, 10] - a[:, s, 9]) if s < 15 else np.full(3, np.nan)
            med = np.median(d, axis=0)
            print(f"  site {s:2d} ({cfg.sites[s % 4].name:6s}) entry={np.median(entry):5.2f} "
                  + " ".join(f"{n}={v:5.2f}" for n, v in zip(PHASES, med))
                  + f" | total {np.median(total):5.2f} next {np.nanmedian(gap) if s < 15 else 0:5.2f}", flush=True)
        stack.destroy()
        del layers, keep, X, Y, ws
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
