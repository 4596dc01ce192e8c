#!/usr/bin/env python3
"""Throughput of the sparse-MoE block on one MI355X.

A step is one pass of the whole block -- router, bucketing, grouped gate/up
with SiLU*up, grouped down, combine -- over one batch of synthetic tokens,
replayed from a hipGraph captured for that batch size.  The default workload
is one Qwen3-30B-A3B MoE layer (H=2048, E=128, k=8, I=768, bf16 weights) at
decode batch T=64; inputs and weights are resident in HBM before timing.

Prints one JSON line: tokens/s (whole job), ms per step, the roofline of the
dominant kernel (grouped gate/up: HBM-bound) measured with HIP events on the
stream the kernels run on, the whole-block HBM fraction, and the fp64 CPU
oracle timed on this host's cores on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload q64|q8|q48q|q4096]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-block tokens/s at T=64, Qwen3-30B-A3B shape; % of HBM peak BW"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
WORKLOAD_TEXT = {
    "q64": "Qwen3-30B-A3B MoE layer (H=2048, E=128, top-8, I=768), decode T=64, bf16 weights, hipGraph replay",
    "q8": "Qwen3-30B-A3B MoE layer (H=2048, E=128, top-8, I=768), decode T=8, bf16 weights, hipGraph replay",
    "q48q": "Qwen3-30B-A3B MoE layer, decode T=48, 4-bit blockwise weights (64 per fp32 absmax), hipGraph replay",
    "q4096": "Qwen3-30B-A3B MoE layer, prefill T=4096, bf16, Zipf-skewed router bias, hipGraph replay",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_model(H, I, E, k, T, n_act, wfmt):
    """Algorithmic HBM bytes of each kernel and of the block (each weight of an
    active expert read once, activations read once, outputs written once)."""
    if wfmt == "bf16":
        w_gu = 2 * I * H * 2
        w_d = H * I * 2
    else:
        w_gu = 2 * I * H // 2 + 2 * I * (H // 64) * 4
        w_d = H * I // 2 + H * (I // 64) * 4
    N = T * k
    gate_up = n_act * w_gu + T * H * 2 + N * I * 2
    down = n_act * w_d + N * I * 2 + N * H * 4
    block = n_act * (w_gu + w_d) + E * H * 2 + T * H * 2 + T * H * 4
    flops = T * (k * 2 * 3 * H * I + 2 * E * H)
    return dict(gate_up=gate_up, down=down, block=block, flops=flops)


def cpu_baseline(inp, budget_s=10.0):
    """fp64 per-token oracle on this host: repeat the batch until ~budget_s."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    W = O.ExpertWeights(inp)
    ids, _, _ = O.route(inp.x, inp.w_router, inp.k, inp.bias)
    W.preload(np.unique(ids))                  # bf16 -> fp64 conversion, not timed
    n_tok, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        O.forward_per_token(inp, W)
        n_tok += inp.T
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return dict(value=n_tok / el, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"fp64 per-token oracle (router, top-k, SwiGLU experts, combine) over the "
                       f"{inp.T}-token batch repeated {reps}x = {n_tok} tokens in {el:.1f} s; "
                       f"expert weights pre-converted to fp64 (not timed)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="q64", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--stage-steps", type=int, default=50)
    ap.add_argument("--cold-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major", action="store_true",
                    help="keep expert weights row-major instead of the tiled layout")
    ap.add_argument("--sweep", action="store_true", help="also time every decode bucket (stderr + JSON extra)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs (--gpus > 1) are not "
              "supported (sharding is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic as S
    from mixture_experts_decode_router_amd import _lib as L
    from mixture_experts_decode_router_amd.layer import MoELayer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    inp = S.make(args.workload)
    T, H, E, k, I = inp.T, inp.H, inp.E, inp.k, inp.I
    log(f"[bench] workload {args.workload}: T={T} H={H} E={E} k={k} I={I} wfmt={inp.wfmt}")
    lay = MoELayer(inp, t_max=T, tiled=not args.row_major)
    stream = torch.cuda.Stream()
    x_static = lay.upload_x(inp.x)
    out_static = torch.empty(T, H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    buckets = [b for b in S.SWEEP_T if b < T] + [T] if args.sweep and T <= 64 else [T]
    lay.capture(buckets, x_static, out_static, stream)
    log(f"[bench] captured buckets {buckets}")

    # ---------------- timed region: K graph replays, back to back
    for _ in range(args.warmup):
        lay.replay(T, stream)
    torch.cuda.synchronize()
    ev = L.hip_events(2)
    t0 = time.perf_counter()
    L.hip_event_record(ev[0], stream)
    for _ in range(args.steps):
        lay.replay(T, stream)
    L.hip_event_record(ev[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = L.hip_event_elapsed_ms(ev[0], ev[1])
    L.hip_events_destroy(ev)
    ms_per_step = wall * 1e3 / args.steps
    value = T * args.steps / wall
    counts = lay.read_counts(stream=stream)
    n_act = int((counts > 0).sum())
    model = bytes_model(H, I, E, k, T, n_act, inp.wfmt)
    log(f"[bench] {args.steps} replays: wall {ms_per_step * 1e3:.1f} us/step, events "
        f"{gpu_ms * 1e3 / args.steps:.1f} us/step, {value:,.0f} tokens/s, n_active={n_act}")

    # ---------------- per-kernel durations: eager forwards with stage events
    S_ = args.stage_steps
    evs = L.hip_events(6 * S_)
    for i in range(5):  # warm
        lay.forward(x_static, T, out_static, stream=stream)
    for i in range(S_):
        lay.forward_timed(x_static, out_static, evs[6 * i:6 * i + 6], T, stream=stream)
    torch.cuda.synchronize()
    names = ["route", "permute", "gate_up", "down", "combine"]
    stage_us = {n: 0.0 for n in names}
    for i in range(S_):
        e = evs[6 * i:6 * i + 6]
        for j, n in enumerate(names):
            stage_us[n] += L.hip_event_elapsed_ms(e[j], e[j + 1]) * 1e3 / S_
    L.hip_events_destroy(evs)
    log("[bench] stage us: " + ", ".join(f"{n} {v:.1f}" for n, v in stage_us.items()))

    # ---------------- cold replays: a 512 MiB scrub between steps (outside the events)
    cold_us = None
    if args.cold_steps > 0:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evc = L.hip_events(2)
        tot = 0.0
        with torch.cuda.stream(stream):
            for i in range(args.cold_steps):
                scrub.fill_(i & 0xFF)
                L.hip_event_record(evc[0], stream)
                lay.replay(T, stream)
                L.hip_event_record(evc[1], stream)
                tot += L.hip_event_elapsed_ms(evc[0], evc[1])
        L.hip_events_destroy(evc)
        cold_us = tot * 1e3 / args.cold_steps
        del scrub
        log(f"[bench] cold replay {cold_us:.1f} us/step")

    dominant = "gate_up"
    dom_us = stage_us[dominant]
    achieved = model[dominant] / (dom_us * 1e-6) / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{dominant}_{args.workload}.json")
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            from mixture_experts_decode_router_amd.build import source_digest
            if tj.get("source_digest") == source_digest():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    step_s = ms_per_step * 1e-3
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.wfmt == "bf16" else "nf4-b64 weights, bf16 MFMA",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; no checkpoint)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": T, "hidden": H, "experts": E,
                   "top_k": k, "inter": I, "weights": inp.wfmt,
                   "weight_layout": "row-major" if args.row_major else "tiled (packed once at load, untimed)",
                   "parallelism": "single GPU"},
        "roofline": {
            "kernel": "grouped gate/up + SiLU*up (" + ("bf16" if inp.wfmt == "bf16" else "4-bit") + ")",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": model[dominant],
            "avg_launch_us": round(dom_us, 2),
        },
        "block": {
            "algorithmic_bytes_per_step": model["block"],
            "hbm_frac": round(model["block"] / step_s / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_frac": round(model["flops"] / step_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "n_active_experts": n_act,
            "stage_us": {n: round(v, 2) for n, v in stage_us.items()},
            "gpu_event_us_per_step": round(gpu_ms * 1e3 / args.steps, 2),
            "cold_us_per_step": None if cold_us is None else round(cold_us, 2),
        },
    }

    if args.sweep and T <= 64:
        sweep = {}
        for b in buckets:
            xb = lay.upload_x(S.make(args.workload, T=b).x)
            with torch.cuda.stream(stream):
                x_static[:b].copy_(xb)
            for _ in range(5):
                lay.replay(b, stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(50):
                lay.replay(b, stream)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / 50
            c = lay.read_counts(stream=stream)
            bm = bytes_model(H, I, E, k, b, int((c > 0).sum()), inp.wfmt)
            sweep[b] = dict(us=round(dt * 1e6, 2), tokens_per_s=round(b / dt, 1),
                            hbm_frac=round(bm["block"] / dt / 1e9 / PEAK_HBM_GBS, 4))
            log(f"[bench] sweep T={b}: {dt * 1e6:.1f} us, {b / dt:,.0f} tok/s, "
                f"{sweep[b]['hbm_frac'] * 100:.1f}% HBM")
        result["sweep"] = sweep

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    lay.release_graph()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
