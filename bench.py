"""Throughput of the canvas denoise step on one MI355X.

A step is one pass of the whole hot path over one batch: (at the first step of each canvas)
the uniform canvas at t = 1, then dg_denoise_step (30-layer decoder over prefix cache + canvas)
and dg_step_sample (fused LM head -> Step with lock-in) at the schedule's next grid point.
Inputs (weights, caches) are resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--repeats R] [--workload C2] [--sampler euler|eb]
                    [--no-cpu-baseline] [--no-breakdown] [--experts bf16|fp8|mxfp4]

Prints one JSON line.  `value` = canvas tokens refined per second (batch * 256 * steps/s), from the
median of R timed runs of K steps each (each run bracketed by device synchronisations).  After
the timed region one more schedule of steps runs with per-class launch timing: `breakdown` gives
each kernel class's time per step and its achieved rate against the roof that bounds it (HBM
bytes or bf16 MFMA FLOPs, algorithmic: what the method must move or compute).
With `--sampler eb` a step samples with the pages' default sampler (entropy-bounded acceptance,
temperature 0.8 -> 0.4, adaptive stop) instead of the Euler Step with lock-in.  `--experts`
swaps the workload's expert weight format (fp8 e4m3 or MXFP4, weights-only with bf16
activations): a variant of the workload, named in `config.workload`, not the headline figure.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROF_EVERY = 4          # one timed step in PROF_EVERY carries the MoE gate/up timing events
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps first (60 at C2 is ~0.7 s: a GPU that idled between processes "
                         "takes ~0.5 s of load to reach its steady clocks)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of K steps each; ms_per_step is their median")
    ap.add_argument("--workload", default="C2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-class timing after the timed region")
    ap.add_argument("--breakdown", action="store_true", help="(default) per-class timing after the timed region")
    ap.add_argument("--sampler", choices=("euler", "eb"), default="euler")
    ap.add_argument("--experts", choices=("bf16", "fp8", "mxfp4"), default=None,
                    help="expert weight format (default: the workload's); fp8 and mxfp4 are weights-only "
                         "formats with bf16 activations")
    ap.add_argument("--act-fp8", action="store_true",
                    help="W8A8 experts: fp8 weights and per-row e4m3 activation codes on the fp8 MFMA "
                         "(a variant of the workload, not the headline)")
    ap.add_argument("--self-cond", action="store_true",
                    help="give the model a self-conditioning block (hidden width 896) and feed each step's "
                         "signal into the next step (a variant of the workload, not the headline)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the causal encoder instead: context encoding of the workload's prefix in one call, "
                         "then the append-after-encode pass of one canvas (one JSON line of its own)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed region, copy 512 MiB device to device 4 times (a plain copy of known "
                         "size for scaling hardware byte counters)")
    return ap.parse_args()


# HBM bytes of one MoE gate/up launch on this workload, from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE; KiB per dispatch, mean of 90 launches), each scaled by the same counter
# on a 512 MiB device-to-device copy (FETCH_SIZE reads 262155.5 KiB for 524288 KiB read: x1.9999;
# WRITE_SIZE reads 524288 KiB: x1).  Valid only while the kernel sources hash to `sources`.
MOE_TRAFFIC = {"sources": "a788bd3f38ac425f9a1b5abad2545458f03ea03317db0891063df1b4d95bd561",
               "fetch_kib": 527983.5, "write_kib": 3872.0, "bytes_per_launch": 1085227651}
TRAFFIC_SOURCES = ("k_gemm.hip", "gemm_dma.h", "gemm_core.h", "common.h", "internal.h")


def kernel_digest():
    import hashlib
    h = hashlib.sha256()
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "discrete_text_diffusion_amd", "csrc")
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(expert_dtype):
    """Stored bytes per expert weight: fp8 one (plus one bf16 scale per row, not counted), MXFP4 a
    half-byte code plus one scale byte per 32 weights, bf16 two."""
    return {"fp8": 1.0, "mxfp4": 0.5 + 1.0 / 32}.get(expert_dtype, 2.0)


def class_roofs(cfg, uniq, gate_up_bytes):
    """Algorithmic work per step of each timed kernel class and the roof that bounds it at this
    workload: (bound, amount, unit, peak) with amount in bytes (HBM) or FLOPs (bf16 MFMA)."""
    wb = weight_bytes(cfg.expert_dtype)
    ab = 2 if cfg.act_dtype == "bf16" else 4
    B, L, d, nl = cfg.batch, cfg.canvas, cfg.d_model, cfg.n_layers
    R = B * L
    hbm = lambda b: ("hbm", b, "GB/s", HBM_PEAK_GBS)
    mfma = lambda f: ("mfma", f, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS)
    # weights, the SwiGLU rows read, the expert output rows written (activation type)
    down = ((uniq * cfg.expert_hidden + cfg.shared_hidden) * d * wb
            + (R * cfg.top_k * cfg.expert_hidden + R * cfg.shared_hidden) * ab + (R * cfg.top_k + R) * d * ab)
    flops = 0.0
    for l in range(nl):
        keys = (cfg.prefix if cfg.is_global(l) else min(cfg.window, cfg.prefix)) + L
        flops += 4.0 * R * cfg.n_q_heads * cfg.head_dim * keys
    samp_bytes = cfg.vocab * d * ab
    samp_flops = 2.0 * R * cfg.vocab * d
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    # self-conditioning: p_hat_0 . E streams E once more (same bytes and FLOPs as the logits); the
    # feed-forward block's weights are negligible beside it
    sc = {"self_condition": hbm(samp_bytes) if samp_flops / samp_bytes < ridge else mfma(samp_flops)} \
        if getattr(cfg, "sc_hidden", 0) else {}
    return {**sc,
        "moe_gate_up": hbm(nl * gate_up_bytes),
        "moe_down": hbm(nl * down),
        "attention": mfma(flops),
        "sampler": hbm(samp_bytes) if samp_flops / samp_bytes < ridge else mfma(samp_flops),
        "qkv_rope": hbm(nl * (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim * d * ab),
        "o_proj": hbm(nl * cfg.n_q_heads * cfg.head_dim * d * ab),
        "routing": hbm(nl * cfg.n_experts * d * ab),
    }


def cpu_baseline(cfg, W, kv, H_dev):
    """The oracle, untuned, on a bounded sample of the same workload: the first two local/global
    periods of decoder layers (12 layers at the 5:1 pattern, all canvas rows) and the sampler
    statistics for every canvas row over the full vocabulary, scaled to one full step (mean local
    layer x n_local + mean global layer x n_global + sampler)."""
    import numpy as np
    import torch
    from oracle import model as M
    from oracle import step as S
    from oracle.numerics import rounder
    from synth import gen
    from synth.host import layer_np, np64

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    period = cfg.global_every if cfg.global_every > 0 else 1
    sample_layers = list(range(min(cfg.n_layers, 2 * period)))
    rnd = rounder(cfg.act_dtype)
    h0 = gen.resid_input(cfg.replace(resid_input=True)).numpy().astype(np.float64)
    times = {"local": [], "global": []}
    for tag, l in [("global" if cfg.is_global(l) else "local", l) for l in sample_layers]:
        lw = M.layer_arrays(layer_np(W["layers"][l]), cfg.expert_dtype)   # conversion: not timed
        K, V = np64(kv[l][0]), np64(kv[l][1])
        t0 = time.perf_counter()
        M.denoise_layer(cfg, l, h0, lw, K, V, [cfg.prefix] * cfg.batch, rnd)
        times[tag].append(time.perf_counter() - t0)
        del lw, K, V
    E = np64(W["embed"])
    ns = cfg.rows
    H = H_dev[:ns].float().cpu().numpy().astype(np.float64)
    rows = np.arange(ns)
    t0 = time.perf_counter()
    z = S.logits(H, E, cfg.tau)
    S.sample_stats(z, cfg.seed, 1, rows // cfg.canvas, rows % cfg.canvas)
    t_samp = time.perf_counter() - t0
    t_loc = sum(times["local"]) / max(len(times["local"]), 1)
    t_glb = sum(times["global"]) / max(len(times["global"]), 1)
    n_glob = sum(cfg.is_global(l) for l in range(cfg.n_layers))
    n_loc = cfg.n_layers - n_glob
    t_step = n_loc * t_loc + n_glob * t_glb + (cfg.rows / ns) * t_samp
    sample_s = sum(times["local"]) + sum(times["global"]) + t_samp
    return {"value": round(cfg.rows / t_step, 3), "unit": "canvas-token-steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"oracle float64 on host: layers 0-{len(sample_layers) - 1} ({len(times['local'])} local at "
                       f"{t_loc:.2f} s, {len(times['global'])} global at {t_glb:.2f} s) over all {cfg.rows} rows, "
                       f"sampler for {ns} of {cfg.rows} rows ({t_samp:.2f} s); scaled to {n_loc} local + {n_glob} "
                       f"global layers = {t_step:.1f} s per step; {sample_s:.1f} s measured")}


def run_prefill(args):
    """dg_prefill_kv at the workload's widths: encoding a `prefix`-token prompt from an empty cache in
    one call, then appending one `canvas`-token block at that prefix (the K - 1 append passes of
    block-AR generation).  Tokens per second of each, the median of the timed runs, with a per-class
    breakdown of one run each."""
    import numpy as np
    import torch
    from discrete_text_diffusion_amd import dg
    from discrete_text_diffusion_amd.model import Model, values_dmajor
    from synth import configs, gen

    cfg0 = configs.get(args.workload)
    P, L = cfg0.prefix, cfg0.canvas
    cfg = cfg0.replace(batch=1, prefix=P + L)                # cache room for the appended block
    dev = torch.device("cuda:0")
    log(f"[prefill] {cfg.name}: encode {P} tokens, then append {L}")
    W = gen.make_weights(cfg, dev)
    kv = values_dmajor(gen.empty_kv(cfg, dev))
    model = Model(cfg, W, kv, [0])
    ws = model.workspace(1, P, P + L)
    toks = gen.uniform_tokens((1, P + L), cfg.vocab, cfg.seed, "prefill-tokens", dev)
    prompt, block = toks[:, :P].contiguous(), toks[:, P:].contiguous()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps, profile=False):
        out = []
        for _ in range(reps):
            model.set_kv(kv, [0])
            fn(True)
            torch.cuda.synchronize()
            if profile:
                dg.dg_profile_enable(model.ctx, (1 << len(dg.PROF_NAMES)) - 1)
            ev0.record(stream)
            fn(False)
            ev1.record(stream)
            torch.cuda.synchronize()
            dg.dg_profile_enable(model.ctx, 0)
            out.append(ev0.elapsed_time(ev1))
        return out

    def encode(setup):
        if not setup:
            model.prefill_kv(prompt, ws, stream=stream)

    def append(setup):
        if setup:
            model.prefill_kv(prompt, ws, stream=stream)
        else:
            model.prefill_kv(block, ws, stream=stream)

    res = {}
    for name, fn, n in (("encode", encode, P), ("append", append, L)):
        timed(fn, 1)                                            # warm-up
        runs = timed(fn, max(args.repeats, 1))
        ms = float(np.median(runs))
        timed(fn, 1, profile=True)
        bd = {}
        for c, cname in enumerate(dg.PROF_NAMES):
            t, k = dg.dg_profile_read(model.ctx, c)
            if k:
                bd[cname] = {"ms": round(t, 3), "launches": k}
        res[name] = {"tokens": n, "ms": round(ms, 3), "ms_runs": [round(x, 3) for x in runs],
                     "tokens_per_s": round(n / (ms * 1e-3), 1), "breakdown": bd}
        log(f"[prefill] {name}: {n} tokens in {ms:.3f} ms ({n / (ms * 1e-3):.0f} tokens/s)")
    assert dg.dg_query_status(model.ctx, ws) == dg.DG_OK
    out = {"metric": "causal encoder tokens/s (context encoding and append-after-encode, 1 MI355X)",
           "value": res["encode"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
           "dtype": cfg.act_dtype, "data": "synthetic (seeded N(0,0.02) weights, uniform tokens)",
           "config": {"workload": f"{args.workload} widths: prefill {P} + append {L}", "layers": cfg.n_layers,
                      "d_model": cfg.d_model, "experts": cfg.n_experts, "top_k": cfg.top_k},
           "encode": res["encode"], "append": res["append"]}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.prefill:
        return run_prefill(args)
    import numpy as np
    import torch
    from discrete_text_diffusion_amd import dg
    from discrete_text_diffusion_amd.model import Model, values_dmajor
    from synth import configs, gen

    cfg = configs.get(args.workload)
    if args.experts is not None and args.experts != cfg.expert_dtype:
        cfg = cfg.replace(expert_dtype=args.experts, name=f"{cfg.name}-{args.experts}experts")
    if args.act_fp8:
        if cfg.expert_dtype != "fp8":
            print("--act-fp8 needs fp8 expert weights (--experts fp8)", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.replace(act_quant="fp8", name=f"{cfg.name}-w8a8")
    if args.self_cond:
        if args.sampler == "eb":
            print("--self-cond runs with the Euler sampler's step calls", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.replace(sc_hidden=896, name=f"{cfg.name}-selfcond")
    dev = torch.device("cuda:0")
    log(f"[bench] workload {cfg.name}: building inputs on {torch.cuda.get_device_name(0)}")
    t0 = time.time()
    W = gen.make_weights(cfg, dev)
    kv = gen.make_random_kv(cfg, dev)
    model = Model(cfg, W, values_dmajor(kv), [cfg.prefix] * cfg.batch)
    B, L = cfg.batch, cfg.canvas
    ws = model.workspace(B, L, cfg.prefix)
    canvas = torch.empty(B, L, dtype=torch.int32, device=dev)
    lock = torch.empty(B, L, dtype=torch.uint8, device=dev)
    n_locked = torch.empty(B, dtype=torch.int32, device=dev)
    hidden = torch.empty(B * L, cfg.d_model, dtype=torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32,
                         device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s; HBM used {torch.cuda.memory_allocated() / 2**30:.1f} GiB")
    T = cfg.steps
    h = 1.0 / T
    stream = torch.cuda.current_stream()

    prev = torch.zeros(B, L, dtype=torch.int32, device=dev)
    done = torch.zeros(B, dtype=torch.int32, device=dev)
    # self-conditioning signal carried from one step to the next (none at a canvas's first step)
    sc = torch.zeros(B * L, cfg.d_model, dtype=torch.float32, device=dev) if args.self_cond else None

    def step(s):
        k = s % T
        if k == 0:
            dg.dg_init_canvas(canvas, lock, B, L, cfg.vocab, cfg.seed + s // T, stream)
            if args.sampler == "eb":
                done.zero_()
        model.denoise_step(canvas, L, ws, hidden_out=hidden, stream=stream, sc_in=sc if k > 0 else None)
        if args.sampler == "eb":
            p = dg.EbParams(t=1.0 - k * h, tau_start=0.8, tau_end=0.4, gamma=0.1, stop_entropy=0.005,
                            seed=cfg.seed, step=k, has_prev=int(k > 0), final_step=int(k == T - 1), adaptive=1)
            dg.dg_step_entropy_bounded(model.ctx, hidden, canvas, prev, done, None, None, B, L, p, ws, stream)
            return
        p = dg.StepParams(schedule=cfg.schedule, t=1.0 - k * h, h=h, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                          seed=cfg.seed, step=k)
        model.step_sample(hidden, canvas, lock, n_locked, p, ws, stream=stream,
                          sc_out=sc if k + 1 < T else None)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    assert dg.dg_query_status(model.ctx, ws) == dg.DG_OK, "non-finite values during warmup"

    # The MoE gate/up launches are timed live with HIP events in every PROF_EVERY-th timed step: an
    # event between two launches keeps the next kernel from starting under the previous one's
    # tail (~4.5 us per event), so sampling the launches keeps the measurement from slowing the
    # step it measures.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = []
    done_steps = args.warmup
    for r in range(max(args.repeats, 1)):
        torch.cuda.synchronize()
        ev0.record(stream)
        for s in range(args.steps):
            dg.dg_profile_enable(model.ctx, (1 << dg.PROF_MOE_GATE_UP) if s % PROF_EVERY == 0 else 0)
            step(done_steps + s)
        ev1.record(stream)
        torch.cuda.synchronize()
        done_steps += args.steps
        reps.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] timed run {r + 1}/{max(args.repeats, 1)}: {reps[-1]:.4f} ms/step")
    dg.dg_profile_enable(model.ctx, 0)
    ms_step = float(np.median(reps))
    moe_ms, moe_n = dg.dg_profile_read(model.ctx, dg.PROF_MOE_GATE_UP)
    log(f"[bench] median of {len(reps)} timed runs of {args.steps} steps: {ms_step:.3f} ms/step")

    # unique experts of the last layer's routing (same workload in every layer)
    idx = torch.empty(B * L, cfg.top_k, dtype=torch.int32, device=dev)
    dg.dg_test_read_routing(model.ctx, ws, B * L, None, idx, None, stream)
    torch.cuda.synchronize()
    uniq = int(torch.unique(idx).numel())
    wbytes = weight_bytes(cfg.expert_dtype)
    abytes = 2 if cfg.act_dtype == "bf16" else 4
    R = B * L
    # one launch: gate+up weights of the routed experts in use and of the shared expert, the
    # normalised rows read once, the SwiGLU rows written once
    gate_up_bytes = int((uniq * 2 * cfg.expert_hidden + 2 * cfg.shared_hidden) * cfg.d_model * wbytes
                     + R * cfg.d_model * abytes
                     + (R * cfg.top_k * cfg.expert_hidden + R * cfg.shared_hidden) * abytes)
    moe_avg_ms = moe_ms / max(moe_n, 1)
    traffic = (MOE_TRAFFIC["bytes_per_launch"]
               if args.workload == "C2" and cfg.expert_dtype == "bf16" and kernel_digest() == MOE_TRAFFIC["sources"]
               else None)
    achieved = gate_up_bytes / (moe_avg_ms * 1e-3) / 1e9

    if args.calib_copy:
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copies: 4 x {src.numel() * 2} bytes read and written")
        del src, dst

    breakdown = None
    if not args.no_breakdown:
        dg.dg_profile_enable(model.ctx, (1 << len(dg.PROF_NAMES)) - 1)
        for s in range(T):
            step(s)
        torch.cuda.synchronize()
        dg.dg_profile_enable(model.ctx, 0)
        roofs = class_roofs(cfg, uniq, gate_up_bytes)
        breakdown = {}
        for c, name in enumerate(dg.PROF_NAMES):
            ms, n = dg.dg_profile_read(model.ctx, c)
            if not n:
                continue
            e = {"ms_per_step": round(ms / T, 4), "launches_per_step": n // T}
            if name in roofs:
                bound, amount, unit, peak = roofs[name]
                rate = amount / (ms / T * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
                e.update({"bound": bound, "achieved": round(rate, 1), "peak": peak, "unit": unit,
                          "frac": round(rate / peak, 4)})
            breakdown[name] = e
        log(f"[bench] breakdown {json.dumps(breakdown)}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        H = torch.empty_like(hidden)
        dg.dg_init_canvas(canvas, lock, B, L, cfg.vocab, cfg.seed, stream)
        model.denoise_step(canvas, L, ws, hidden_out=H, stream=stream)
        torch.cuda.synchronize()
        cpu = cpu_baseline(cfg, W, kv, H)
        log(f"[bench] cpu baseline {cpu}")

    steps_per_s = 1000.0 / ms_step
    out = {
        "metric": "canvas-token denoise steps/sec (30L, 256 canvas, 1 MI355X) + % of roofline",
        "value": round(steps_per_s * B * L, 1),
        "unit": "canvas-token-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "repeats": len(reps), "ms_per_step_runs": [round(x, 4) for x in reps],
        "steps_per_s": round(steps_per_s, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": (cfg.act_dtype if cfg.expert_dtype in ("f32", "bf16") else f"bf16+{cfg.expert_dtype}w"
                  + ("+fp8a" if getattr(cfg, "act_quant", "") == "fp8" else "")),
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) caches, uniform canvas)",
        "config": {"workload": f"{args.workload}: {cfg.name}", "layers": cfg.n_layers, "batch": B, "canvas": L,
                   "prefix": cfg.prefix, "vocab": cfg.vocab, "d_model": cfg.d_model, "experts": cfg.n_experts,
                   "top_k": cfg.top_k, "schedule_steps": T,
                   "sampler": "entropy-bounded" if args.sampler == "eb" else "euler+lock-in",
                   "self_conditioning": bool(args.self_cond)},
        "roofline": {"kernel": "moe_gate_up (routed + shared experts gate/up + SwiGLU, one launch)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_ms": round(moe_avg_ms, 5), "launches": moe_n,
                     "algorithmic_bytes_per_launch": gate_up_bytes, "unique_experts": uniq},
        "cpu_baseline": cpu,
    }
    if breakdown:
        out["breakdown"] = breakdown
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
