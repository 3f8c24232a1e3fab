"""Benchmark: batch-1 GSI decode on the GPT-J-6B-shaped linear stack (one MI355X).

Workload (default): 28 blocks x 4 linear sites (QKV 4096->12288, out 4096->4096,
fc_in 4096->16384, fc_out 16384->4096), bf16, k = 256, eps = 0.10, synthetic weights and tokens
with ~99.8% of tokens on the fast path. One step = one token through all 112 sites (the whole
hot path: projection, residual norm, gate, M g or W x), batch 1, sites strictly in order.

Prints one JSON line (rank 0, N = 1). `value` is tokens/s with every input already resident in
HBM; the timed region is `--steps` tokens after `--warmup` tokens. The roofline object prices
the decode kernel against the 8 TB/s HBM peak using the algorithmic bytes of the realised gates
(per token and site: V_k, plus M, plus W when the gate is slow), measured with HIP events on the
kernel's stream. The CPU baseline times the fp64 oracle on a bounded sample (see --cpu-seconds).
The line also carries the create-time precompute (M = W V_k, V_k^T V_k - I and, for 16-bit layers,
(V_k (V_k^T V_k - I))^T) at k = 256 and at k = 512 as matrix-core TFLOP/s, and the bandwidth of an
in-repo streaming-read kernel. Unless --no-extras is given, it also carries the same layers run
in the other site modes (`site_modes`: every site a static projection, MLP-only gating, every
site dense) and the extra workloads (`extra_workloads`: shared-input sites, T = 64 batched, the
decode step, the GPT-2- and OPT-shaped stacks, the operating-point sweep at k = 256, the
depth-cascade calibration).

`--config 5` instead times the T = 64 workload (k = 512, ~20% slow tokens per step) through the
batched path and prints its own line (tokens/s and algorithmic GB/s).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "batch-1 GSI decode tokens/s + achieved HBM GB/s vs peak, GPT-J-6B-shaped stack"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512, help="tokens decoded in the timed region")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--config", type=int, default=3, help="synthetic workload id (3 = GPT-J-shaped, the headline)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall time of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reps", type=int, default=3, help="timed repetitions (the median is reported)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (reference kernel for HBM counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="operating-point sweep on the GPT-J-shaped stack: rank k x fast fraction, "
                         "against a dense batch-1 GEMV chain (prints its own line)")
    ap.add_argument("--sweep-ranks", default="64,128,256,512")
    ap.add_argument("--calibration", action="store_true",
                    help="depth-cascade calibration of the bases on the GPT-J-shaped chain (prints its own line)")
    ap.add_argument("--cal-cold", type=int, default=8, help="subspace-iteration steps of a cold start")
    ap.add_argument("--cal-warm", type=int, default=2, help="steps of a cascade (warm) start")
    ap.add_argument("--step", action="store_true",
                    help="batch-1 decode step of the GPT-J-shaped model: the GSI sites around an unchanged "
                         "plain attention, against the same step with every site dense (prints its own line)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload (not its site modes, nor the shared-input, T = 64 "
                         "and decode-step workloads)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: libgsi has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Per-GPU work is one decode stream; see the design notes for how the path would shard.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_rank_linear_amd as g
    import synth
    from synth.generate import config_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if g.gsi_device_check() != 0:
        raise SystemExit("not a gfx950 device")
    if args.sweep:
        print(json.dumps(sweep(args, g, torch, np)), flush=True)
        return
    if args.calibration:
        print(json.dumps(calibration(args, g, torch, np)), flush=True)
        return
    if args.step:
        print(json.dumps(decode_step(args, g, torch, np)), flush=True)
        return
    cfg = synth.get(args.config)
    if cfg.t_step != 1:
        out = batched(args, cfg, g, torch, np)
    else:
        out = batch1(args, cfg, g, torch, np)
    if args.config == 3 and not args.no_extras:
        out["extra_workloads"] = extra_workloads(args, g, torch, np)
    print(json.dumps(out), flush=True)


def extra_workloads(args, g, torch, np) -> dict:
    """More workloads timed in the same run: the shared-input GPT-J-shaped stack (batch 1, q/k/v
    and fc_in as one site), the GPT-2-shaped (fp16) and OPT-shaped (bf16, ~14% slow tokens)
    stacks at batch 1, the T = 64 batched workload (k = 512, ~20% slow tokens per step) and
    the decode step (the GSI sites of a GPT-J-shaped model around an unchanged plain attention,
    against the same step with dense sites), each with its own bytes and roofline fraction; the
    operating-point sweep at k = 256 (tokens/s against the fast fraction, next to the vendor dense
    chain); and the depth-cascade calibration of the bases (GPU time against cold starts on the
    same kernels, without its oracle leg)."""
    import argparse
    import gc

    import synth
    res = {}
    a6 = argparse.Namespace(**vars(args))
    a6.steps, a6.warmup, a6.reps, a6.no_cpu_baseline = 512, 32, 3, True
    o6 = batch1(a6, synth.get(6), g, torch, np, light=True)
    res["gptj_shared_input_batch1"] = {k: o6[k] for k in ("value", "unit", "ms_per_step", "roofline", "fast_fraction")}
    res["gptj_shared_input_batch1"]["workload"] = o6["config"]["workload"]
    gc.collect()
    torch.cuda.empty_cache()
    a5 = argparse.Namespace(**vars(args))
    a5.steps, a5.warmup, a5.reps = 40, 10, 1
    o5 = batched(a5, synth.get(5), g, torch, np)
    res["gptj_batched_t64"] = {k: o5[k] for k in ("value", "unit", "ms_per_step", "roofline", "slow_fraction",
                                                    "sites_with_slow_tokens")}
    res["gptj_batched_t64"]["workload"] = o5["config"]["workload"]
    gc.collect()
    torch.cuda.empty_cache()
    a7 = argparse.Namespace(**vars(args))
    a7.steps, a7.warmup, a7.no_cpu_baseline = 48, 8, True
    o7 = decode_step(a7, g, torch, np)
    res["gptj_decode_step"] = {k: o7[k] for k in ("value", "unit", "ms_per_step", "roofline", "fast_fraction",
                                                   "dense_step", "speedup_vs_dense", "two_site_stack_a", "graph")}
    res["gptj_decode_step"]["workload"] = o7["config"]["workload"]
    gc.collect()
    torch.cuda.empty_cache()
    for cid, key in ((2, "gpt2_stack_fp16_batch1"), (4, "opt_stack_bf16_batch1")):
        a2 = argparse.Namespace(**vars(args))
        a2.steps, a2.warmup, a2.reps, a2.no_cpu_baseline = 512, 32, 1, True
        o2 = batch1(a2, synth.get(cid), g, torch, np, light=True)
        res[key] = {k: o2[k] for k in ("value", "unit", "ms_per_step", "roofline", "fast_fraction")}
        res[key]["workload"] = o2["config"]["workload"]
        gc.collect()
        torch.cuda.empty_cache()
    a9 = argparse.Namespace(**vars(args))
    a9.sweep_ranks = "256"
    o9 = sweep(a9, g, torch, np)
    res["gptj_sweep_k256"] = {"unit": "tokens/s", "dense": o9["dense"], "rows": o9["rows"],
                              "workload": o9["config"]["workload"] + ", k=256, planned slow counts per 512 tokens"}
    gc.collect()
    torch.cuda.empty_cache()
    a8 = argparse.Namespace(**vars(args))
    a8.no_cpu_baseline = True
    o8 = calibration(a8, g, torch, np)
    res["gptj_calibration"] = {k: o8[k] for k in ("cascade_s", "cold_every_layer_s", "cascade_saving_vs_cold",
                                                   "svd_every_layer_s", "time_ratio_cascade_to_svd", "step_ms",
                                                   "max_sine_vs_planted")}
    res["gptj_calibration"]["unit"] = "s"
    res["gptj_calibration"]["workload"] = o8["config"]["workload"]
    gc.collect()
    torch.cuda.empty_cache()
    return res


def batch1(args, cfg, g, torch, np, light: bool = False) -> dict:
    """The batch-1 stack decode of a workload with T_step = 1 (the headline when cfg is the
    GPT-J-shaped stack). light: only the decode and its bytes (no CPU baseline, no rank-512
    precompute, no stream-read kernel)."""
    import synth
    from synth.generate import config_inputs

    es = 2 if cfg.dtype != "f32" else 4

    # ---------------- inputs: generate on the host, upload, precompute M on the GPU ----------------
    t0 = time.time()
    sites = config_inputs(cfg)
    log(f"[bench] generated bases and tokens for {len(sites)} sites in {time.time() - t0:.1f}s")
    layers, keep, bufs = [], [], []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    for si in sites:
        W = synth.site_weight(cfg, si.block, si.site).cuda()
        V = si.V.cuda()
        # M and aux are allocated before the timed region: it holds the precompute kernels only
        nb = g.gsi_layer_aux_bytes(g.dtype_code(W.dtype), si.d_out, si.d, cfg.k)
        bufs.append((torch.empty((si.d_out, cfg.k), dtype=W.dtype, device=W.device),
                     torch.empty(nb, dtype=torch.uint8, device=W.device)))
        keep.append((W, V))
    # M = W V, V^T V, and for 16-bit layers (V (V^T V - I))^T (the batched gate's second projection)
    pre_flop = sum(2.0 * si.d_out * si.d * cfg.k + 2.0 * cfg.k * cfg.k * si.d * (1 if cfg.dtype == "f32" else 2)
                   for si in sites)
    # one create workspace for all layers (the creates run one after another on the stream)
    wc = max(g.gsi_layer_create_workspace_bytes(g.dtype_code(W.dtype), si.d_out, si.d, cfg.k)
             for si, (W, _) in zip(sites, keep))
    ws_create = torch.empty(wc, dtype=torch.uint8, device="cuda") if wc else None
    # one untimed pass first: the runtime loads each kernel's code on its first launch
    for (W, V), (M, aux) in zip(keep, bufs):
        g.gsi_layer_create(W, V, M, aux, ws_create).destroy()
    # every layer's precompute enqueued back to back, as a model load would run it
    torch.cuda.synchronize()
    ev0.record()
    for (W, V), (M, aux) in zip(keep, bufs):
        layers.append(g.gsi_layer_create(W, V, M, aux, ws_create))
    ev1.record()
    torch.cuda.synchronize()
    pre_ms = ev0.elapsed_time(ev1)
    del bufs
    log(f"[bench] uploaded weights and ran the M = W V precompute in {time.time() - t0:.1f}s "
        f"(precompute kernels {pre_ms:.1f} ms)")
    del ws_create
    pre512 = precompute_rank512(g, torch, cfg, sites, keep) if cfg.dtype != "f32" and cfg.k == 256 and not light else None
    stack = g.gsi_stack_create(layers)
    n_sites = len(layers)
    X = torch.cat([si.X for si in sites], dim=1).contiguous().cuda()
    n_tok = X.shape[0]
    y_ld = sum(si.d_out for si in sites)
    Y = torch.zeros((n_tok, y_ld), dtype=X.dtype, device="cuda")
    gates = torch.zeros((n_tok, n_sites), dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(g.gsi_stack_workspace_bytes(stack, 1))
    stream = torch.cuda.current_stream()

    def run(tokens: int):
        done = 0
        while done < tokens:
            n = min(n_tok, tokens - done)
            g.gsi_stack_decode(stack, X, n, 1, cfg.eps, Y, gates, None, ws, stream)
            done += n

    run(args.warmup)
    torch.cuda.synchronize()
    if g.gsi_workspace_status(ws) != 0:
        raise SystemExit("decode kernel reported a wait timeout")

    times = []
    for _ in range(max(1, args.reps)):
        torch.cuda.synchronize()
        ev0.record(stream)
        t_wall = time.perf_counter()
        run(args.steps)
        ev1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        times.append((ev0.elapsed_time(ev1) / 1e3, t_wall))
    if g.gsi_workspace_status(ws) != 0:
        raise SystemExit("decode kernel reported a wait timeout")
    stream_gbps = stream_read_gbps(torch) if not light else None
    if args.copy_calibration and not light:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2
    times.sort()
    t_gpu, t_wall = times[len(times) // 2]
    n_launch = (args.steps + n_tok - 1) // n_tok

    # ---------------- algorithmic bytes from the realised gates ----------------
    gb = gates.cpu().numpy()
    v_b = np.array([si.d * cfg.k * es for si in sites], dtype=np.float64)
    m_b = np.array([si.d_out * cfg.k * es for si in sites], dtype=np.float64)
    w_b = np.array([si.d_out * si.d * es for si in sites], dtype=np.float64)
    tok_idx = np.arange(args.steps) % n_tok
    slow = gb[tok_idx].astype(np.float64)                       # [steps, sites]
    bytes_total = float(np.sum(v_b + m_b) * args.steps + np.sum(slow * w_b[None, :]))
    fast_frac = 1.0 - float(slow.mean())
    achieved = bytes_total / t_gpu / 1e9
    tok_s = args.steps / t_gpu

    tokens_per_launch = args.steps / n_launch
    traffic, traffic_src = measured_traffic(cfg, tokens_per_launch)

    # ---------------- CPU baseline: the fp64 oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, sites, keep, args.cpu_seconds)

    out = {
        "metric": METRIC if cfg.cid == 3 else f"batch-1 GSI decode tokens/s + achieved HBM GB/s vs peak, {cfg.name}",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_gpu * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[cfg.dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_blocks} blocks x {len(cfg.sites)} sites "
                               + ", ".join(f"{s.name} {s.d}->{s.d_out}" for s in cfg.sites)
                               + f", k={cfg.k}, eps={cfg.eps}, batch 1, {n_tok} distinct tokens",
                   "batch": 1, "k": cfg.k, "eps": cfg.eps, "sites": n_sites},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": decode_kernel_name(cfg), "launches": n_launch,
                     "bytes_per_launch": bytes_total / n_launch, "launch_ms": round(t_gpu * 1e3 / n_launch, 4)},
        "cpu_baseline": cpu,
        "fast_fraction": round(fast_frac, 5),
        "wall_ms_per_step": round(t_wall * 1e3 / args.steps, 5),
        "stream_read_gbps": round(stream_gbps, 1) if stream_gbps else None,
        "frac_of_stream_read": round(achieved / stream_gbps, 4) if stream_gbps else None,
        "precompute": {"ms": round(pre_ms, 2), "tflop": round(pre_flop / 1e12, 4),
                       "tflops": round(pre_flop / (pre_ms / 1e3) / 1e12, 2) if pre_ms > 0 else None,
                       "mfma_bf16_peak_tflops": BF16_MFMA_PEAK_TFLOPS},
        "precompute_k512": pre512,
    }
    if cfg.cid == 3 and not light and not args.no_extras:
        out["site_modes"] = site_modes(args, cfg, g, torch, np, layers, sites, X, n_tok, stream)
    # release the stack's device table while the runtime is up
    stack.destroy()
    torch.cuda.synchronize()
    return out


def site_modes(args, cfg, g, torch, np, layers, sites, X, n_tok, stream) -> dict:
    """The headline stack's layers run in the other site modes [GSI §2 intro, §2.2, §4]: every
    site a static projection (y = M g, no residual norm, no gate), MLP-only gating (the attention
    maps q/k/v and out dense, y = W x; the MLP maps gated) and every site dense (y = W x, the same
    kernel). Each is timed like the headline (warm-up, then --steps tokens, HIP events on the
    stream). Algorithmic bytes by mode per token and site: static V_k + M, dense W, gated V_k + M,
    plus W when the token is slow."""
    es = 2 if cfg.dtype != "f32" else 4
    v_b = np.array([si.d * cfg.k * es for si in sites], dtype=np.float64)
    m_b = np.array([si.d_out * cfg.k * es for si in sites], dtype=np.float64)
    w_b = np.array([si.d_out * si.d * es for si in sites], dtype=np.float64)
    attention = np.array([cfg.sites[si.site].name in ("qkv", "out") for si in sites])
    plans = {
        "static_projection": [g.GSI_SITE_STATIC] * len(layers),
        "mlp_only_gating": [g.GSI_SITE_DENSE if a else g.GSI_SITE_GATED for a in attention],
        "all_dense": [g.GSI_SITE_DENSE] * len(layers),
    }
    y_ld = sum(si.d_out for si in sites)
    res = {}
    for name, modes in plans.items():
        st = g.gsi_stack_create_modes(layers, modes)
        Y = torch.zeros((n_tok, y_ld), dtype=X.dtype, device="cuda")
        gates = torch.zeros((n_tok, len(layers)), dtype=torch.uint8, device="cuda")
        ws = g.new_workspace(g.gsi_stack_workspace_bytes(st, 1))

        def run(tokens):
            done = 0
            while done < tokens:
                n = min(n_tok, tokens - done)
                g.gsi_stack_decode(st, X, n, 1, cfg.eps, Y, gates, None, ws, stream)
                done += n

        run(args.warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(args.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        if g.gsi_workspace_status(ws) != 0:
            raise SystemExit(f"decode kernel reported a wait timeout ({name})")
        t = e0.elapsed_time(e1) / 1e3
        mode = np.array(modes)
        slow = gates.cpu().numpy()[np.arange(args.steps) % n_tok].astype(np.float64)
        per_tok = np.where(mode == g.GSI_SITE_DENSE, w_b, v_b + m_b)
        gated = mode == g.GSI_SITE_GATED
        total = float(per_tok.sum() * args.steps + np.sum(slow[:, gated] * w_b[None, gated]))
        achieved = total / t / 1e9
        res[name] = {"value": round(args.steps / t, 2), "unit": "tokens/s",
                     "ms_per_step": round(t * 1e3 / args.steps, 5),
                     "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                                  "bytes_per_step": total / args.steps},
                     "sites": {"gated": int(gated.sum()), "static": int((mode == g.GSI_SITE_STATIC).sum()),
                               "dense": int((mode == g.GSI_SITE_DENSE).sum())}}
        if gated.any():
            res[name]["fast_fraction_gated_sites"] = round(1.0 - float(slow[:, gated].mean()), 5)
        st.destroy()
        del Y, gates, ws
        torch.cuda.synchronize()
    dense = res["all_dense"]["value"]
    for name in ("static_projection", "mlp_only_gating"):
        res[name]["speedup_vs_all_dense"] = round(res[name]["value"] / dense, 3)
    return res


def batched(args, cfg, g, torch, np):
    """A T-token-per-step workload (the GPT-J-shaped stack at T = 64, k = 512): every site runs
    the batched path (projection, device-side gate and compaction, M g for the fast tokens and W x
    for the slow ones on the matrix cores) once per step. Inputs: a pool of generated steps,
    cycled (the workload's own recipe); --steps counts steps of T tokens. Bytes per (step, site)
    from the realised gates: V_k, plus M if any token is fast, plus W if any token is slow."""
    from synth.generate import config_inputs, token_steps

    es = 2 if cfg.dtype != "f32" else 4
    pool = token_steps(cfg)
    t0 = time.time()
    sites = []
    for b0 in range(0, cfg.n_blocks, 4):
        sites += config_inputs(cfg, blocks=range(b0, min(cfg.n_blocks, b0 + 4)), n_steps=pool)
        log(f"[bench] generated blocks {b0}..{min(cfg.n_blocks, b0 + 4) - 1} ({time.time() - t0:.0f}s)")
    log(f"[bench] generated bases and {pool} steps of {cfg.t_step} tokens for {len(sites)} sites in {time.time() - t0:.1f}s")
    layers, keep = [], []
    for si in sites:
        W = synth_weight(cfg, si)
        L = g.create_layer(W, si.V.cuda())
        layers.append(L)
        keep.append(W)
    torch.cuda.synchronize()
    stack = g.gsi_stack_create(layers)
    n_sites = len(layers)
    X = torch.cat([si.X for si in sites], dim=1).contiguous().cuda()
    n_tok = X.shape[0]
    y_ld = sum(si.d_out for si in sites)
    Y = torch.zeros((n_tok, y_ld), dtype=X.dtype, device="cuda")
    gates = torch.zeros((n_tok, n_sites), dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(g.gsi_stack_workspace_bytes(stack, cfg.t_step))
    stream = torch.cuda.current_stream()
    slow_steps = []

    def run(steps: int, record: bool):
        done = 0
        while done < steps:
            n = min(pool, steps - done)
            g.gsi_stack_decode(stack, X, n, cfg.t_step, cfg.eps, Y, gates, None, ws, stream)
            if record:
                slow_steps.append(gates[: n * cfg.t_step].view(n, cfg.t_step, n_sites).clone())
            done += n

    run(args.warmup, False)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(max(1, args.reps)):
        slow_steps.clear()
        torch.cuda.synchronize()
        ev0.record(stream)
        run(args.steps, True)
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / 1e3)
    if g.gsi_workspace_status(ws) != 0:
        raise SystemExit("batched path reported a wait timeout")
    if args.copy_calibration:  # reference kernel for the HBM counters: a 1 GiB device copy
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2
    times.sort()
    t_gpu = times[len(times) // 2]
    gs = torch.cat(slow_steps).cpu().numpy().astype(bool)          # [steps, T, sites]
    any_slow = gs.any(axis=1)
    any_fast = (~gs).any(axis=1)
    v_b = np.array([si.d * cfg.k * es for si in sites], dtype=np.float64)
    m_b = np.array([si.d_out * cfg.k * es for si in sites], dtype=np.float64)
    w_b = np.array([si.d_out * si.d * es for si in sites], dtype=np.float64)
    bytes_total = float(np.sum(v_b[None, :] + any_fast * m_b[None, :] + any_slow * w_b[None, :]))
    tok_s = args.steps * cfg.t_step / t_gpu
    achieved = bytes_total / t_gpu / 1e9
    out = {
        "metric": "GSI batched decode tokens/s + achieved HBM GB/s vs peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_gpu * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_blocks} blocks x {len(cfg.sites)} sites, k={cfg.k}, eps={cfg.eps}, "
                               f"T={cfg.t_step} per step, pool of {pool} steps cycled", "batch": cfg.t_step, "k": cfg.k,
                   "eps": cfg.eps, "sites": n_sites},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "batched path, all kernels of a step", "bytes_per_step": bytes_total / args.steps},
        "slow_fraction": round(float(gs.mean()), 4),
        "sites_with_slow_tokens": round(float(any_slow.mean()), 4),
        "cpu_baseline": None,
    }
    tr, tr_src = measured_traffic_batched(cfg)
    out["roofline"]["traffic"], out["roofline"]["traffic_source"] = tr, tr_src
    stack.destroy()
    torch.cuda.synchronize()
    return out


def sweep(args, g, torch, np):
    """Operating-point sweep on the GPT-J-shaped stack (28 blocks x QKV / out / fc_in / fc_out,
    bf16, batch 1, eps = 0.10): for each rank k and each planned fast fraction f (fixed slow
    counts out of 512 tokens per site), decode tokens/s through the persistent decode kernel,
    next to a dense batch-1 chain (torch linear, i.e. the vendor BLAS GEMV, y = W x for all 112
    sites in order) on the same weights. Per point the line gives the measured speedup over the
    dense chain and three read-ratio models: the pages' (f M + (1 - f) W against W, the model
    their 3.0x / 10.5x / 15.6x fit), the same with V_k's reads added, and the bytes this kernel
    reads (V_k + M always, since M g is formed before the gate is known, plus W when slow).

    Inputs: block 0's four sites get their own bases and tokens per rank (synth sweep configs);
    blocks 1..27 hold device copies of block 0's V and tokens at their own addresses, and every
    (block, site) has its own seeded Gaussian W drawn on the GPU. Timing is what differs from the
    headline run, not the values, so the copies stream from HBM like distinct data (the 11.3 GB
    of W per token is far above the 256 MB last-level cache)."""
    import dataclasses

    from synth.configs import SWEEP_SLOW_COUNTS, SlowPlan, sweep_config
    from synth.generate import site_basis, site_tokens, store

    ranks = [int(v) for v in args.sweep_ranks.split(",") if v]
    base = sweep_config(ranks[0])
    n_blocks, shapes = base.n_blocks, base.sites
    n_tok = base.n_steps
    bf16 = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6000)
    Ws = []
    for b in range(n_blocks):
        for st in shapes:
            w = torch.randn((st.d_out, st.d), generator=gen, device="cuda")
            Ws.append((w * base.w_std).to(bf16))
            del w
    torch.cuda.synchronize()
    w_bytes = np.array([st.d_out * st.d * 2 for st in shapes] * n_blocks, dtype=np.float64)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()

    # ---- dense baseline: y = W x for every site in order, one token at a time ----
    xs = [torch.randn((1, st.d), generator=gen, device="cuda").to(bf16) for st in shapes]
    F = torch.nn.functional

    def dense(tokens):
        for _ in range(tokens):
            for i, W in enumerate(Ws):
                F.linear(xs[i % len(shapes)], W)

    dense(4)
    torch.cuda.synchronize()
    n_dense = 64
    ev0.record(stream)
    dense(n_dense)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_dense = ev0.elapsed_time(ev1) / 1e3 / n_dense
    dense_tok_s = 1.0 / t_dense
    log(f"[sweep] dense chain: {dense_tok_s:.1f} tokens/s, {w_bytes.sum() / t_dense / 1e9:.0f} GB/s")
    rows = []
    for k in ranks:
        cfg = sweep_config(k)
        t0 = time.time()
        bases = [site_basis(cfg, 0, s) for s in range(len(shapes))]
        Vd = [store(v, cfg.dtype).cuda() for v, _ in bases]
        layers, keep = [], []
        for b in range(n_blocks):
            for s in range(len(shapes)):
                V = Vd[s] if b == 0 else Vd[s].clone()
                layers.append(g.create_layer(Ws[b * len(shapes) + s], V))
                keep.append(V)
        stack = g.gsi_stack_create(layers)
        torch.cuda.synchronize()
        v_bytes = np.array([st.d * k * 2 for st in shapes] * n_blocks, dtype=np.float64)
        m_bytes = np.array([st.d_out * k * 2 for st in shapes] * n_blocks, dtype=np.float64)
        ws = g.new_workspace(g.gsi_stack_workspace_bytes(stack, 1))
        y_ld = sum(st.d_out for st in shapes) * n_blocks
        Y = torch.zeros((n_tok, y_ld), dtype=bf16, device="cuda")
        gates = torch.zeros((n_tok, len(layers)), dtype=torch.uint8, device="cuda")
        log(f"[sweep] k={k}: bases and layers in {time.time() - t0:.1f}s")
        for n_slow in SWEEP_SLOW_COUNTS:
            c = dataclasses.replace(cfg, slow=SlowPlan("fixed", count=n_slow))
            blk = torch.cat([site_tokens(c, 0, s, basis=bases[s])[0] for s in range(len(shapes))], dim=1).cuda()
            X = blk.repeat(1, n_blocks).contiguous()
            del blk
            steps = n_tok if n_slow <= n_tok // 4 else 64
            g.gsi_stack_decode(stack, X, 32, 1, cfg.eps, Y, gates, None, ws, stream)  # warm-up
            times = []
            for _ in range(3):
                ev0.record(stream)
                g.gsi_stack_decode(stack, X, steps, 1, cfg.eps, Y, gates, None, ws, stream)
                ev1.record(stream)
                torch.cuda.synchronize()
                times.append(ev0.elapsed_time(ev1) / 1e3)
            if g.gsi_workspace_status(ws) != 0:
                raise SystemExit("decode kernel reported a wait timeout")
            t = sorted(times)[1] / steps
            slow = gates[:steps].cpu().numpy().astype(np.float64)          # [steps, sites]
            f = 1.0 - float(slow.mean())
            kernel_bytes = float(np.sum(v_bytes + m_bytes) + np.sum(slow.mean(axis=0) * w_bytes))
            pages_bytes = float(np.sum(f * m_bytes + (1.0 - f) * w_bytes))
            vinc_bytes = pages_bytes + float(np.sum(v_bytes))
            rows.append({"k": k, "planned_slow_per_512": n_slow, "fast_fraction": round(f, 5),
                         "tokens_s": round(1.0 / t, 1), "ms_per_token": round(t * 1e3, 4),
                         "kernel_gbps": round(kernel_bytes / t / 1e9, 1),
                         "speedup_vs_dense": round(t_dense / t, 3),
                         "model_pages_read_ratio": round(float(w_bytes.sum()) / pages_bytes, 3),
                         "model_with_vk": round(float(w_bytes.sum()) / vinc_bytes, 3),
                         "model_kernel_bytes": round(float(w_bytes.sum()) / kernel_bytes, 3)})
            log(f"[sweep] {rows[-1]}")
            del X
        del stack, layers, keep, Vd, ws, Y, gates
        torch.cuda.synchronize()
    out = {"metric": "GSI operating-point sweep: batch-1 decode tokens/s vs rank k and fast fraction, "
                     "GPT-J-6B-shaped stack", "unit": "tokens/s", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"gptj-6b-shaped sweep: {n_blocks} blocks x 4 sites, eps=0.1, batch 1, "
                                  f"{n_tok} tokens per site"},
           "dense": {"tokens_s": round(dense_tok_s, 1), "ms_per_token": round(t_dense * 1e3, 4),
                     "gbps": round(float(w_bytes.sum()) / t_dense / 1e9, 1),
                     "what": "torch linear (vendor BLAS) y = W x, 112 sites in order, batch 1"},
           "rows": rows}
    del Ws, xs
    return out


def calibration(args, g, torch, np):
    """Calibration of the bases with the depth cascade [GSI §2.3] on the GPT-J-shaped chain:
    28 layers of 2048 calibration tokens x 4096 (float32), k = 256, planted subspaces 25 degrees
    apart. Three ways, each timed with HIP events on the GPU:
      cascade  layer 0 from a Gaussian start (--cal-cold steps), every later layer from the
               previous layer's basis (--cal-warm steps);
      cold     every layer from the Gaussian start (--cal-cold steps);
      svd      a full SVD of every layer's activation matrix (torch.linalg.svd, the vendor
               solver), timed on a sample of layers and scaled to 28.
    Accuracy: the largest principal sine of each basis against the leading right singular
    vectors of that layer's SVD (the exact subspace) on the sampled layers, and against the
    planted basis on every layer. Bytes and flops per subspace-iteration step: the two float32
    products read A twice (2 n d 4 B) and do 4 n d k flops; the Gram-Schmidt kernel re-reads the
    earlier rows, k^2 d 4 B per projection pass."""
    import math

    from oracle import gsi_calibration as cal
    from synth.calibration import GPTJ_CALIBRATION as c
    from synth.calibration import activations, cold_start, planted_bases

    t0 = time.time()
    P = planted_bases(c)
    As = [activations(c, l, P[l]).cuda() for l in range(c.n_layers)]
    Om = cold_start(c).cuda()
    log(f"[calibration] generated {c.n_layers} layers of {c.n} x {c.d} in {time.time() - t0:.1f}s")
    ws = torch.empty(g.gsi_calibrate_workspace_bytes(c.n, c.d, c.k), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((c.k, c.d), dtype=torch.float32, device="cuda") for _ in range(c.n_layers)]
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()  # warm-up (first launches)
        torch.cuda.synchronize()
        ev0.record(stream)
        fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3

    def cascade():
        for l in range(c.n_layers):
            g.gsi_calibrate(As[l], Om if l == 0 else outs[l - 1], args.cal_cold if l == 0 else args.cal_warm,
                            outs[l], ws)

    def cold():
        for l in range(c.n_layers):
            g.gsi_calibrate(As[l], Om, args.cal_cold, outs[l], ws)

    def one_step():
        g.gsi_calibrate(As[0], Om, 1, outs[0], ws)

    t_step = timed(one_step)
    t_cold = timed(cold)
    sines_cold = [cal.principal_sines(P[l], outs[l].double().cpu().numpy().T)[0] for l in range(c.n_layers)]
    cold_q = {l: outs[l].double().cpu().numpy().T for l in (0, 1, c.n_layers - 1)}
    t_cascade = timed(cascade)
    casc_q = [outs[l].double().cpu().numpy().T for l in range(c.n_layers)]
    sines_casc = [cal.principal_sines(P[l], casc_q[l])[0] for l in range(c.n_layers)]
    sample = [0, 1, c.n_layers - 1]
    svd_t = []
    exact = {}
    for l in sample:
        torch.cuda.synchronize()
        ev0.record(stream)
        _, _, vh = torch.linalg.svd(As[l], full_matrices=False)
        ev1.record(stream)
        torch.cuda.synchronize()
        svd_t.append(ev0.elapsed_time(ev1) / 1e3)
        exact[l] = vh[: c.k].double().cpu().numpy().T
    t_svd = float(np.median(svd_t)) * c.n_layers
    acc = {f"layer_{l}": {"cascade_vs_exact": float(cal.principal_sines(exact[l], casc_q[l])[0]),
                          "cold_vs_exact": float(cal.principal_sines(exact[l], cold_q[l])[0]),
                          "exact_vs_planted": float(cal.principal_sines(P[l], exact[l])[0])} for l in sample}
    step_bytes = 2.0 * c.n * c.d * 4
    step_flop = 4.0 * c.n * c.d * c.k
    cpu = None
    if not args.no_cpu_baseline:
        # the fp64 oracle's cascade on the first layers of the same chain (layer 0 cold, then warm),
        # timed on the host cores and scaled to the 28 layers by steps
        from threadpoolctl import threadpool_info
        n_layers_cpu = 3
        A_host = [As[l].cpu().numpy() for l in range(n_layers_cpu)]
        t0 = time.perf_counter()
        cal.calibrate_cascade(A_host, Om.cpu().numpy().T, args.cal_cold, args.cal_warm)
        el = time.perf_counter() - t0
        steps_cpu = args.cal_cold + (n_layers_cpu - 1) * args.cal_warm
        steps_all = args.cal_cold + (c.n_layers - 1) * args.cal_warm
        threads = max([q.get("num_threads", 1) for q in threadpool_info()] or [1])
        cpu = {"value": round(el / steps_cpu * steps_all, 3), "unit": "s", "cores": int(threads), "kind": "oracle",
               "sample": f"fp64 oracle cascade on layers 0-{n_layers_cpu - 1} ({steps_cpu} steps) in {el:.1f}s, "
                         f"scaled to {steps_all} steps; BLAS threads {threads}"}
    out = {"metric": "GSI basis calibration with the depth cascade: GPU time for all layers, GPT-J-shaped chain",
           "unit": "s", "n_gpus": 1, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"calibration chain: {c.n_layers} layers, {c.n} tokens x d={c.d}, k={c.k}, "
                                  f"planted subspaces {c.theta_deg} degrees apart, cold {args.cal_cold} steps, "
                                  f"warm {args.cal_warm} steps"},
           "cascade_s": round(t_cascade, 4), "cold_every_layer_s": round(t_cold, 4),
           # the like-for-like saving: the same kernels and step, warm starts against cold ones
           "cascade_saving_vs_cold": round(1.0 - t_cascade / t_cold, 4),
           # context only: the vendor SVD computes the exact subspace with another algorithm, so
           # this ratio is not the cascade's saving
           "svd_every_layer_s": round(t_svd, 4), "svd_sampled_layers_s": [round(v, 4) for v in svd_t],
           "time_ratio_cascade_to_svd": round(t_cascade / t_svd, 4),
           "step_ms": round(t_step * 1e3, 3),
           "step_products": {"bytes": step_bytes, "flop": step_flop},
           "accuracy": acc,
           "max_sine_vs_planted": {"cascade": round(float(max(sines_casc)), 5), "cold": round(float(max(sines_cold)), 5)},
           "cpu_baseline": cpu}
    del As, outs, ws
    return out


def decode_step(args, g, torch, np):
    """Batch-1 decode step of a GPT-J-shaped model (28 parallel blocks, d 4096, 16 heads of 256,
    d_ff 16384, k 256, eps 0.10, bf16) on the synthetic step model: per block gsi_block_step
    (LayerNorm, stack A, plain attention over a key/value cache that starts with a 1024-position
    prefix, GELU, the [out, fc_out] stack, residual add), token after token, each block's output
    feeding the next. Stack A is one shared-input site: QKV and fc_in read the same LayerNorm
    output, so their rows are stacked on one basis (one g, one gate for both). The same step with
    the sites in the dense site mode (y = W x, the same kernels otherwise) is the reference. The
    line also gives both for stack A as two sites [QKV, fc_in] ("two_site_stack_a"). Tokens/s over --steps tokens
    (default 48) after --warmup (default 8), one gsi_decode_step call per token followed by a
    synchronisation (decoding is autoregressive: a token's input exists only once the previous
    token is done), HIP events on the stream the library enqueues on; "queued" gives the rate with
    the synthetic tokens enqueued back to back, "graph" the rate of one captured step
    (gsi_decode_step_devpos) replayed per token.
    Algorithmic bytes per token: per site V_k + M (+ W when slow), W for the dense step, plus the
    attention's key and value rows (2 (pos + 1) d 2 bytes per block)."""
    import dataclasses

    from oracle import gsi_oracle as orc
    from oracle import gsi_step as ostep
    from synth.step import step_config, step_model

    n_warm = min(args.warmup, 8) if args.warmup != 64 else 8
    n_time = min(args.steps, 48) if args.steps != 512 else 48
    cfg = dataclasses.replace(step_config(72), n_tokens=n_warm + n_time)
    t0 = time.time()
    model = step_model(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"[step] generated {cfg.n_blocks} blocks on the GPU in {time.time() - t0:.1f}s")
    names_a, names_b = ("qkv", "fc_in"), ("out", "fc_out")
    blocks = []
    for hb in model["blocks"]:
        layers = {n: g.create_layer(hb[n][0], hb[n][1]) for n in names_a + names_b}
        # QKV and fc_in share the LayerNorm output's basis: one site with their rows stacked
        wc = torch.cat([hb["qkv"][0], hb["fc_in"][0]], dim=0).contiguous()
        layers["qkv_fc_in"] = g.create_layer(wc, hb["qkv"][1])
        blocks.append({"layers": layers, "hb": hb, "wc": wc,
                       "A": g.gsi_stack_create([layers["qkv_fc_in"]]),
                       "B": g.gsi_stack_create([layers[n] for n in names_b]),
                       "Ad": g.gsi_stack_create_modes([layers["qkv_fc_in"]], [g.GSI_SITE_DENSE]),
                       "Bd": g.gsi_stack_create_modes([layers[n] for n in names_b], [g.GSI_SITE_DENSE] * 2),
                       "A2": g.gsi_stack_create([layers[n] for n in names_a]),
                       "A2d": g.gsi_stack_create_modes([layers[n] for n in names_a], [g.GSI_SITE_DENSE] * 2)})
    torch.cuda.synchronize()
    log(f"[step] layers and stacks in {time.time() - t0:.1f}s")
    d, dff, H = cfg.d, cfg.d_ff, cfg.n_heads
    dt = torch.bfloat16
    xa = torch.zeros(2 * d, dtype=dt, device="cuda")
    ya = torch.zeros(3 * d + dff, dtype=dt, device="cuda")
    xb = torch.zeros(d + dff, dtype=dt, device="cuda")
    yb = torch.zeros(2 * d, dtype=dt, device="cuda")
    n_tok = cfg.n_tokens
    gates = torch.zeros((n_tok, cfg.n_blocks, 4), dtype=torch.uint8, device="cuda")
    ws = g.new_workspace(max(g.gsi_block_step_workspace_bytes(blocks[0][a], blocks[0]["B"], H) for a in ("A", "A2")))
    K0 = [hb["K"].clone() for hb in model["blocks"]]  # the prefix, restored before each pass
    V0 = [hb["V"].clone() for hb in model["blocks"]]
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gam = [hb["gamma"] for hb in model["blocks"]]
    bet = [hb["beta"] for hb in model["blocks"]]
    Ks = [hb["K"] for hb in model["blocks"]]
    Vs = [hb["V"] for hb in model["blocks"]]
    gates = gates.view(n_tok, cfg.n_blocks * 4)

    def run(dense, sync_each=True, two_site=False):
        for b, hb in enumerate(model["blocks"]):
            hb["K"].copy_(K0[b])
            hb["V"].copy_(V0[b])
        xs = model["x0"].clone()
        sa, sb = ("Ad", "Bd") if dense else ("A", "B")
        if two_site:
            sa = "A2d" if dense else "A2"
        A = [blk[sa] for blk in blocks]
        B = [blk[sb] for blk in blocks]
        h0 = 0.0
        for t in range(n_tok):
            if t == n_warm:
                ev0.record(stream)
                h0 = time.perf_counter()
            # one call per token: the library enqueues the blocks' 4 n_blocks + 1 launches
            g.gsi_decode_step(A, B, gam, bet, Ks, Vs, cfg.L0 + t, H, cfg.eps, xs[t], xa, ya, xb, yb, gates[t], None, ws)
            if sync_each:  # autoregressive: the next token's input exists only after this token
                torch.cuda.synchronize()
        host = (time.perf_counter() - h0) / n_time
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / n_time, xs, host

    def run_graph(dense):
        # one step captured in a HIP graph with the position in device memory, replayed per token
        # (each replay followed by a synchronisation, as in run); token 0 runs the call eagerly
        for b, hb in enumerate(model["blocks"]):
            hb["K"].copy_(K0[b])
            hb["V"].copy_(V0[b])
        xs = model["x0"].clone()
        A = [blk["Ad" if dense else "A"] for blk in blocks]
        B = [blk["Bd" if dense else "B"] for blk in blocks]
        pos_dev = torch.tensor([cfg.L0], dtype=torch.int32, device="cuda")
        xg = torch.empty_like(xs[0])
        gg = torch.zeros(cfg.n_blocks * 4, dtype=torch.uint8, device="cuda")
        call = lambda: g.gsi_decode_step_devpos(A, B, gam, bet, Ks, Vs, pos_dev, H, cfg.eps, xg, xa, ya, xb, yb, gg,
                                                None, ws)
        xg.copy_(xs[0])
        call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        w = max(n_warm, 1)
        for t in range(1, n_tok):
            if t == w:
                ev0.record(stream)
            xg.copy_(xs[t])
            graph.replay()
            torch.cuda.synchronize()
        ev1.record(stream)
        torch.cuda.synchronize()
        assert int(pos_dev.item()) == cfg.L0 + n_tok
        del graph
        return ev0.elapsed_time(ev1) / 1e3 / (n_tok - w)

    t2_gsi, _, _ = run(False, two_site=True)
    gt2 = gates[n_warm:].view(n_time, cfg.n_blocks, 4).cpu().numpy().astype(np.int64)
    t2_dense, _, _ = run(True, two_site=True)
    t_gsi, xs, host_gsi = run(False)
    t_gsi_q, _, _ = run(False, sync_each=False)
    gt = gates[n_warm:].view(n_time, cfg.n_blocks, 4).cpu().numpy().astype(np.int64)  # [QKV, fc_in, out, fc_out]
    t_dense, _, host_dense = run(True)
    t_dense_q, _, _ = run(True, sync_each=False)
    t_gsi_g = run_graph(False)
    t_dense_g = run_graph(True)
    assert g.gsi_workspace_status(ws) == 0
    # algorithmic bytes of the timed tokens: per site V_k + M (+ W when slow), W for dense sites;
    # the shared-input site reads V_k once for QKV and fc_in
    k = cfg.k

    def step_bytes(sites, gts):
        gsi_b, dense_b = 0.0, 0.0
        for t in range(n_time):
            pos = cfg.L0 + n_warm + t
            att = 2.0 * (pos + 1) * d * 2 * cfg.n_blocks
            for col, (do, di) in sites:
                slow = gts[t, :, col].sum()
                gsi_b += cfg.n_blocks * (di * k + do * k) * 2.0 + slow * do * di * 2.0
                dense_b += cfg.n_blocks * do * di * 2.0
            gsi_b += att
            dense_b += att
        return gsi_b / n_time, dense_b / n_time

    gsi_b, dense_b = step_bytes([(0, (3 * d + dff, d)), (2, (d, d)), (3, (d, dff))], gt)
    gsi2_b, dense2_b = step_bytes([(0, (3 * d, d)), (1, (dff, d)), (2, (d, d)), (3, (d, dff))], gt2)
    order = ("qkv", "fc_in", "out", "fc_out")
    fast = 1.0 - gt[:, :, [0, 2, 3]].mean()
    # CPU baseline: the oracle's step on block 0 for as many tokens as about --cpu-seconds allow
    cpu = None
    if not args.no_cpu_baseline:
        import threadpoolctl
        hb = model["blocks"][0]
        blk64 = {"gamma": orc.as_f64(hb["gamma"].cpu()), "beta": orc.as_f64(hb["beta"].cpu())}
        for n in order:
            W64, V64 = orc.as_f64(hb[n][0].cpu()), orc.as_f64(hb[n][1].cpu())
            blk64[n] = (W64, V64, orc.precompute_image(W64, V64))
        K64, V64c = orc.as_f64(K0[0].cpu()), orc.as_f64(V0[0].cpu())
        x64 = orc.as_f64(model["x0"].cpu())
        t1 = time.perf_counter()
        n_cpu = 0
        while time.perf_counter() - t1 < args.cpu_seconds:
            t = n_cpu % n_tok  # the step's tokens in turn, each at its own position
            ostep.decode_block(x64[t], blk64, K64, V64c, cfg.L0 + t, cfg.eps, H)
            n_cpu += 1
        el = time.perf_counter() - t1
        threads = max([q.get("num_threads", 1) for q in threadpoolctl.threadpool_info()] or [1])
        cpu = {"value": round(n_cpu / (el * cfg.n_blocks), 4), "unit": "tokens/s", "cores": int(threads),
               "kind": "oracle", "sample": f"fp64 oracle step, block 0 x {n_cpu} tokens in {el:.1f}s, scaled "
                                           f"x{cfg.n_blocks} blocks; M precomputed; BLAS threads {threads}"}
    out = {"metric": "batch-1 decode step tokens/s, GSI sites around an unchanged plain attention, GPT-J-shaped",
           "value": round(1.0 / t_gsi, 2), "unit": "tokens/s", "n_gpus": 1, "steps": n_time, "warmup": n_warm,
           "ms_per_step": round(t_gsi * 1e3, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{cfg.name}: {cfg.n_blocks} parallel blocks, d {d}, {H} heads, d_ff {dff}, "
                                  f"k {k}, eps {cfg.eps}, cache prefix {cfg.L0}, batch 1"},
           "roofline": {"bound": "hbm", "achieved": round(gsi_b / t_gsi / 1e9, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(gsi_b / t_gsi / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                        "kernel": "all launches of a step", "bytes_per_step": round(gsi_b)},
           "fast_fraction": round(float(fast), 5),
           "dense_step": {"value": round(1.0 / t_dense, 2), "ms_per_step": round(t_dense * 1e3, 4),
                          "achieved_gbps": round(dense_b / t_dense / 1e9, 1), "bytes_per_step": round(dense_b)},
           "speedup_vs_dense": round(t_dense / t_gsi, 3),
           # the same step from a captured graph (gsi_decode_step_devpos), one replay per token
           "graph": {"value": round(1.0 / t_gsi_g, 2), "ms_per_step": round(t_gsi_g * 1e3, 4),
                     "achieved_gbps": round(gsi_b / t_gsi_g / 1e9, 1), "dense_value": round(1.0 / t_dense_g, 2),
                     "speedup_vs_dense": round(t_dense_g / t_gsi_g, 3)},
           "two_site_stack_a": {"value": round(1.0 / t2_gsi, 2), "ms_per_step": round(t2_gsi * 1e3, 4),
                                "achieved_gbps": round(gsi2_b / t2_gsi / 1e9, 1),
                                "dense_value": round(1.0 / t2_dense, 2), "speedup_vs_dense": round(t2_dense / t2_gsi, 3),
                                "fast_fraction": round(float(1.0 - gt2.mean()), 5)},
           # the given tokens enqueued without waiting between them (not autoregressive)
           "queued": {"value": round(1.0 / t_gsi_q, 2), "ms_per_step": round(t_gsi_q * 1e3, 4),
                      "dense_value": round(1.0 / t_dense_q, 2)},
           "cpu_baseline": cpu}
    for blk in blocks:
        for key in ("A", "B", "Ad", "Bd", "A2", "A2d"):
            blk[key].destroy()
    torch.cuda.synchronize()
    return out


def synth_weight(cfg, si):
    import synth
    return synth.site_weight(cfg, si.block, si.site).cuda()


def precompute_rank512(g, torch, cfg, sites, keep):
    """The create-time precompute (V^T, M = W V, V^T V - I, (V (V^T V - I))^T) at rank k = 512 over the same weights:
    the shapes of the T = 64 GPT-J-shaped workload, whose precompute is the one matrix-core bound
    step of the method. V is a seeded Gaussian matrix scaled by 1/sqrt(d) (orthonormality does not
    change the work). Only the kernels are timed."""
    k = 512
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5120)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flop = 0.0
    vs, bufs, made = [], [], []
    for si, (W, _) in zip(sites, keep):
        vs.append((torch.randn((si.d, k), generator=gen, device="cuda") / si.d ** 0.5).to(W.dtype))
        nb = g.gsi_layer_aux_bytes(g.dtype_code(W.dtype), si.d_out, si.d, k)
        bufs.append((torch.empty((si.d_out, k), dtype=W.dtype, device="cuda"),
                     torch.empty(nb, dtype=torch.uint8, device="cuda")))
        flop += 2.0 * si.d_out * si.d * k + 2.0 * k * k * si.d * 2
    wc = max(g.gsi_layer_create_workspace_bytes(g.dtype_code(W.dtype), si.d_out, si.d, k)
             for si, (W, _) in zip(sites, keep))
    ws_create = torch.empty(wc, dtype=torch.uint8, device="cuda") if wc else None
    torch.cuda.synchronize()
    ev0.record()
    for (W, _), V, (M, aux) in zip(keep, vs, bufs):
        made.append(g.gsi_layer_create(W, V, M, aux, ws_create))
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    del made, bufs, vs
    return {"k": k, "ms": round(ms, 2), "tflop": round(flop / 1e12, 4),
            "tflops": round(flop / (ms / 1e3) / 1e12, 2), "mfma_bf16_peak_tflops": BF16_MFMA_PEAK_TFLOPS,
            "frac": round(flop / (ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}


def stream_read_gbps(torch) -> float:
    """Read bandwidth of the in-repo streaming-read kernel (libgsi_bench.so, one pass over 4 GiB
    with 16-byte non-temporal loads) on the same GPU: a practical ceiling to set the decode
    kernel's bandwidth against, beside the 8 TB/s peak. Best of 5 passes, HIP events."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "gated_rank_linear_amd", "_lib", "libgsi_bench.so"))
    lib.gsi_bench_stream_read.restype = ctypes.c_int
    lib.gsi_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    x = torch.ones(1 << 32, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(5):
        ev0.record(stream)
        rc = lib.gsi_bench_stream_read(x.data_ptr(), x.numel() // 16, sink.data_ptr(), stream.cuda_stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        if rc != 0:
            raise SystemExit(f"stream-read kernel failed ({rc})")
        best = max(best, x.numel() / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    del x, sink
    return best


def decode_kernel_name(cfg) -> str:
    """The decode kernel instance the library launches for this stack: element type and input
    window (2 chunks of 16 bytes per data thread when every input row fits in 512 chunks, else 8)."""
    es = 4 if cfg.dtype == "f32" else 2
    need = max((s.d * es // 16 + 255) // 256 for s in cfg.sites)
    t = {"f32": "float", "f16": "gsi::f16_t", "bf16": "gsi::bf16_t"}[cfg.dtype]
    return f"gsi::decode_kernel<{t}, {2 if need <= 2 else 8}>"


def batched_sources_sha256() -> str:
    """sha256 over the sources of the batched path's kernels and its driver."""
    import hashlib

    h = hashlib.sha256()
    for f in ("gsi_dense.hip", "gsi_api.cpp", "gsi_internal.h"):
        h.update(open(os.path.join(ROOT, "gated_rank_linear_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic_batched(cfg):
    """HBM bytes per step of the batched path (all its launches) from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a 1 GiB copy); (None,
    reason) when the sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "batched_path_gptj_t64_bf16.traffic.json")
    if cfg.cid != 5 or not os.path.exists(path):
        return None, "no counter run for this workload"
    rec = json.load(open(path))
    if batched_sources_sha256() != rec.get("sources_sha256"):
        return None, "batched path changed since the committed counter run"
    return rec["traffic_bytes_per_step"], "rocprofv3 FETCH_SIZE + WRITE_SIZE per step of the committed profile run, copy-calibrated"


def decode_sources_sha256() -> str:
    """sha256 over the sources the decode kernel is built from (kernel, work split, shared header)."""
    import hashlib

    h = hashlib.sha256()
    for f in ("gsi_decode.hip", "gsi_plan.h", "gsi_internal.h"):
        h.update(open(os.path.join(ROOT, "gated_rank_linear_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic(cfg, tokens_per_launch: float):
    """HBM bytes of one timed launch from the committed rocprofv3 counter runs (FETCH_SIZE and
    WRITE_SIZE of the profiled launch, each scaled by what the counter reads for a 1 GiB copy),
    per token of the profiled launch times the tokens of the timed launch; (None, reason) when the
    decode kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_gptj_stack_bf16.traffic.json")
    if cfg.cid != 3 or not os.path.exists(path):
        return None, "no counter run for this workload"
    rec = json.load(open(path))
    if decode_sources_sha256() != rec.get("sources_sha256"):
        return None, "decode kernel changed since the committed counter run"
    per_tok = rec["traffic_bytes_per_launch"] / rec["tokens_per_launch"]
    return round(per_tok * tokens_per_launch), (
        f"rocprofv3 FETCH_SIZE + WRITE_SIZE of the committed profile run ({rec['tokens_per_launch']} tokens per "
        f"launch, copy-calibrated), scaled to {tokens_per_launch:g} tokens")


def cpu_baseline(cfg, sites, keep, seconds: float):
    """Time the fp64 oracle (unchanged) on block 0's sites, batch-1 token after token, for about
    `seconds` of wall time, and scale to the whole stack (all blocks have the same shapes). The
    fp64 M precompute is excluded (reported by the oracle as a separate step)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import gsi_oracle as orc

    blk = [(si, w) for si, w in zip(sites, keep) if si.block == 0]
    prep = []
    for si, (W, V) in blk:
        W64 = orc.as_f64(W.cpu())
        V64 = orc.as_f64(si.V)
        prep.append((W64, V64, orc.precompute_image(W64, V64), orc.as_f64(si.X)))
    n_avail = prep[0][3].shape[0]
    t0 = time.perf_counter()
    n = 0
    while True:
        t = n % n_avail
        for W64, V64, M64, X64 in prep:
            orc.forward(W64, V64, X64[t:t + 1], cfg.eps, M=M64)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_token_stack = el / n * cfg.n_blocks
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    try:
        cpu_name = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        cpu_name = "unknown"
    return {"value": round(1.0 / per_token_stack, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle, block 0's {len(prep)} sites x {n} batch-1 tokens in {el:.1f}s, "
                      f"scaled x{cfg.n_blocks} blocks; M precompute excluded; BLAS threads {threads}; {cpu_name}"}


if __name__ == "__main__":
    main()
