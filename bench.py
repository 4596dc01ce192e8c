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

Profiler summaries (under profiles/) are made from rocprofv3 CSV output:

    python bench.py --summarize stats DIR          # --kernel-trace --stats run
    python bench.py --summarize traffic FETCH_DIR WRITE_DIR --workload W
    python bench.py --summarize mfma DIR --workload W   # --pmc MfmaUtil MfmaFlopsBF16 GRBM_GUI_ACTIVE run
                                                   # two --pmc runs with --calib-copy
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
    "q4096q": "Qwen3-30B-A3B MoE layer, prefill T=4096, 4-bit blockwise weights (the q48q layer), hipGraph replay",
}
# workload -> (synthetic workload, token count or None for its own)
WORKLOAD_INPUT = {"q4096q": ("q48q", 4096)}


def make_workload(name, T=None):
    import synthetic as S
    base, t0 = WORKLOAD_INPUT.get(name, (name, None))
    return S.make(base, T=T if T is not None else t0)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bucketing_form(wfmt, T, E, k, row_major=False, lora=False, train=False):
    """Where the library buckets the routed slots for a forward of T rows (the
    rule of its forward): "direct" -- the 16-row expert kernels scan the ids
    themselves and no bucketing kernel runs (bf16 weights, no adapters, no kept
    pre-activations, 2E <= T k <= 1024 slots below the MFMA path); "router" --
    the router's select workgroup (T <= 8, T k <= 64); else "kernel"."""
    n = T * k
    mfma = wfmt == "bf16" and not row_major and n >= 32 * E
    if not mfma and wfmt == "bf16" and not lora and not train and 2 * E <= n <= 1024:
        return "direct"
    if T <= 8 and n <= 64:
        return "router"
    return "kernel"


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


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def cpu_baseline(inp, budget_s=10.0, budget_1t_s=5.0):
    """fp64 per-token oracle on this host: repeat the batch until ~budget_s on
    the BLAS threads numpy has (all the cores this process may use), then
    again on one thread for ~budget_1t_s."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    W = O.ExpertWeights(inp)
    ids, _, _ = O.route(inp.x, inp.w_router, inp.k, inp.bias)
    W.preload(np.unique(ids))                  # bf16 -> fp64 conversion, not timed

    def timed(budget):
        n_tok, reps = 0, 0
        t0 = time.perf_counter()
        while True:
            O.forward_per_token(inp, W)
            n_tok += inp.T
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return n_tok, reps, el

    n_tok, reps, el = timed(budget_s)
    one = None
    if threadpool_limits is not None and budget_1t_s > 0:
        with threadpool_limits(limits=1):
            n1, r1, e1 = timed(budget_1t_s)
        one = dict(value=round(n1 / e1, 1), unit="tokens/s", cores=1,
                   sample=f"the same batch repeated {r1}x = {n1} tokens in {e1:.1f} s on one BLAS thread")
    return dict(value=n_tok / el, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"fp64 per-token oracle (router, top-k, SwiGLU experts, combine) over the "
                       f"{inp.T}-token batch repeated {reps}x = {n_tok} tokens in {el:.1f} s; "
                       f"expert weights pre-converted to fp64 (not timed)",
                cpu_model=_cpu_model(), os_cpu_count=os.cpu_count(),
                affinity_cpus=len(os.sched_getaffinity(0)), one_thread=one)


# ---------------------------------------------------------------- profiles

CALIB_MIB = 256   # size of the plain copy that calibrates the HBM byte counters


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def _short(name):
    import re
    n = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"\((moe::|unsigned int|at::|long|int,).*", "", n)
    return n[:90]


def summarize_stats(d):
    """Markdown table of a rocprofv3 --kernel-trace --stats run (kernel_stats.csv)."""
    import csv
    rows = []
    for path in _csvs(d, "kernel_stats.csv"):
        rows += list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out)


def _counter_rows(d, counter):
    """(dispatch id, kernel name, value in KiB) of every dispatch, in dispatch order."""
    import csv
    rows = []
    for path in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(rows)


def summarize_traffic(fetch_dir, write_dir, workload):
    """HBM bytes per launch of every MoE kernel from two --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the --calib-copy copy of CALIB_MIB MiB (the largest copy kernel
    dispatch of the run)."""
    from mixture_experts_decode_router_amd.build import source_digest

    def calib(rows):
        # the --calib-copy copies are the first copy dispatches of the run
        copies = [v for _, k, v in rows if "copy" in k.lower()][:3]
        if len(copies) < 3:
            raise SystemExit("no calibration copies in the run: profile with --calib-copy")
        copies.sort()
        return CALIB_MIB * 1024.0 / copies[1]

    def means(rows):
        acc = {}
        for _, k, v in rows:
            acc.setdefault(k, []).append(v)
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    fr, wr = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    cf, cw = calib(fr), calib(wr)
    (f, nf), (w, _) = means(fr), means(wr)
    kernels = {}
    for k in sorted(set(f) | set(w)):
        if "moe::" not in k:
            continue
        fk, wk = f.get(k, 0.0), w.get(k, 0.0)
        kernels[_short(k)] = dict(dispatches=nf.get(k, 0), fetch_kib=round(fk, 1), write_kib=round(wk, 1),
                                  bytes_per_launch=int(round((fk * cf + wk * cw) * 1024)))
    return dict(workload=workload, source_digest=source_digest(), copy_mib=CALIB_MIB,
                fetch_scale=round(cf, 4), write_scale=round(cw, 4), kernels=kernels)


def measure_ceilings(torch, L, stream):
    """Achievable rates on this chip, measured beside the block: a read-only
    stream of 2 GiB with the decode GEMMs' load form (the library's read
    probe; best of three grid sizes), a plain 1 GiB device copy (bytes read +
    written per second), the bf16 MFMA issue rate on register operands (the
    library's MFMA probe, 16x16x32 and 32x32x16, 4 waves per SIMD), the
    LDS-DMA copy rate of 16-row x 64-byte tiles of a 16 MiB buffer of 4 KiB
    rows (the prefill GEMMs' gathered token copies; the library's gather
    probe, one row per lane and four lanes per row segment, 2 GiB copied) and
    the vendor library's dense bf16 GEMM at 8192^3."""
    ev = L.hip_events(2, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)

    def timed(fn, reps):
        with torch.cuda.stream(stream):
            for _ in range(2):
                fn()
            L.hip_event_record(ev[0], stream)
            for _ in range(reps):
                fn()
            L.hip_event_record(ev[1], stream)
        torch.cuda.synchronize()
        return L.hip_event_elapsed_ms(ev[0], ev[1]) * 1e-3 / reps

    nbytes = 2 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16384 * 4, dtype=torch.int32, device="cuda")
    read = {}
    for n_wg in (512, 1024, 2048, 4096):
        t = timed(lambda: L.moe_probe_read(src, nbytes, sink, n_wg, stream), 10)
        read[n_wg] = nbytes / t / 1e9
    del src, sink
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    fs = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    mfma = {}
    for shape, tag in ((0, "16x16x32"), (1, "32x32x16")):
        iters = 4000
        t = timed(lambda: L.moe_probe_mfma(fs, 1024, iters, shape, stream), 5)
        mfma[tag] = 1024 * 4 * iters * 131072 / t / 1e12
    del fs
    gsrc = torch.ones(16 << 20, dtype=torch.uint8, device="cuda")
    gsink = torch.empty(1024 * 4, dtype=torch.int32, device="cuda")
    gather = {}
    for order, tag in ((0, "row_per_lane"), (1, "four_lanes_per_row")):
        t = timed(lambda: L.moe_probe_gather(gsrc, 16 << 20, 4096, order, 512, gsink, 1024, stream), 10)
        gather[tag] = 1024 * 4 * 512 * 1024 / t / 1e9
    del gsrc, gsink
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    t_gemm = timed(lambda: torch.mm(a, b), 10)
    del a, b
    L.hip_events_destroy(ev)
    best = max(read, key=read.get)
    return {"stream_read_GBps": round(read[best], 1), "stream_read_workgroups": best,
            "device_copy_GBps": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "mfma_bf16_16x16x32_TFLOPs": round(mfma["16x16x32"], 1),
            "mfma_bf16_32x32x16_TFLOPs": round(mfma["32x32x16"], 1),
            "lds_copy_row_per_lane_GBps": round(gather["row_per_lane"], 1),
            "lds_copy_four_lanes_per_row_GBps": round(gather["four_lanes_per_row"], 1),
            "vendor_bf16_gemm_TFLOPs": round(2.0 * n ** 3 / t_gemm / 1e12, 1)}


def summarize_mfma(d, workload):
    """Per-kernel MFMA evidence from one --pmc run (MfmaUtil: % of SIMD cycles
    with the MFMA unit busy; MfmaFlopsBF16: bf16 MFMA flops per dispatch, the
    SQ_INSTS_VALU_MFMA_MOPS_BF16 count times 512)."""
    from mixture_experts_decode_router_amd.build import source_digest
    per = {}
    for name in ("MfmaUtil", "MfmaFlopsBF16", "GRBM_GUI_ACTIVE"):
        for _, k, v in _counter_rows(d, name):
            per.setdefault(k, {}).setdefault(name, []).append(v)
    kernels = {}
    for k, m in sorted(per.items()):
        if "moe::" not in k or "MfmaUtil" not in m:
            continue
        mean = {n: sum(v) / len(v) for n, v in m.items()}
        kernels[_short(k)] = dict(dispatches=len(m["MfmaUtil"]), mfma_util_pct=round(mean["MfmaUtil"], 2),
                                  mfma_flops_bf16_per_launch=int(mean.get("MfmaFlopsBF16", 0)),
                                  gui_active_cycles=int(mean.get("GRBM_GUI_ACTIVE", 0)))
    return dict(workload=workload, source_digest=source_digest(), kernels=kernels)


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
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy / vendor GEMM ceiling measurement")
    ap.add_argument("--no-lora", action="store_true", help="skip the step with rank-16 LoRA adapters")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-prenorm", action="store_true",
                    help="skip the step with the fused pre-block residual add + RMSNorm")
    ap.add_argument("--row-major", action="store_true",
                    help="keep expert weights row-major instead of the tiled layout")
    ap.add_argument("--sweep", action="store_true", help="also time every decode bucket (stderr + JSON extra)")
    ap.add_argument("--calib-copy", action="store_true",
                    help=f"run a plain {CALIB_MIB} MiB device copy first (calibrates profiler byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="'stats DIR' or 'traffic FETCH_DIR WRITE_DIR': print a profile summary, no GPU")
    args = ap.parse_args()

    if args.summarize:
        kind, dirs = args.summarize[0], args.summarize[1:]
        if kind == "stats" and len(dirs) == 1:
            print(summarize_stats(dirs[0]))
        elif kind == "traffic" and len(dirs) == 2:
            print(json.dumps(summarize_traffic(dirs[0], dirs[1], args.workload), indent=1))
        elif kind == "mfma" and len(dirs) == 1:
            print(json.dumps(summarize_mfma(dirs[0], args.workload), indent=1))
        else:
            ap.error("--summarize stats DIR | --summarize traffic FETCH_DIR WRITE_DIR | --summarize mfma DIR")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU; multi-GPU runs (--gpus > 1) are not "
              "supported (the block's expert- and tensor-parallel sharding is not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic as S
    from mixture_experts_decode_router_amd import _lib as L
    from mixture_experts_decode_router_amd.layer import MoELayer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calib_copy:
        src = torch.full((CALIB_MIB << 20,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    inp = make_workload(args.workload)
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
    # timing-only events: no system-scope fence at each record (the default
    # fence writes back caches and adds microseconds around every stage)
    evs = L.hip_events(6 * S_, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)
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
    bucketing = bucketing_form(inp.wfmt, T, E, k, row_major=args.row_major)
    log("[bench] stage us: " + ", ".join(f"{n} {v:.1f}" for n, v in stage_us.items())
        + ("" if bucketing == "kernel" else
           f" (bucketing: {bucketing}; no bucketing kernel, the permute figure is the cost of an event pair)"))

    # ---------------- per-replay spread: one event between consecutive replays
    R_ = args.stage_steps
    evr = L.hip_events(R_ + 1, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)
    L.hip_event_record(evr[0], stream)
    for i in range(R_):
        lay.replay(T, stream)
        L.hip_event_record(evr[i + 1], stream)
    torch.cuda.synchronize()
    per = np.array([L.hip_event_elapsed_ms(evr[i], evr[i + 1]) * 1e3 for i in range(R_)])
    L.hip_events_destroy(evr)
    replay_pct = {q: round(float(np.percentile(per, p)), 2) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}
    log(f"[bench] replay us p10/p50/p90: {replay_pct['p10']}/{replay_pct['p50']}/{replay_pct['p90']}")

    # ---------------- cold replays: 512 MiB scrub between steps (outside the
    # events), read-only (evicts L2 and the 256 MB last-level cache without
    # leaving dirty lines to write back during the step) and, for comparison,
    # by writing
    cold = {}
    if args.cold_steps > 0:
        scrub = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        evc = L.hip_events(2, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)
        for mode in ("read", "write"):
            tot = 0.0
            with torch.cuda.stream(stream):
                for i in range(args.cold_steps):
                    if mode == "read":
                        scrub.max()
                    else:
                        scrub.fill_(i & 0xFF)
                    L.hip_event_record(evc[0], stream)
                    lay.replay(T, stream)
                    L.hip_event_record(evc[1], stream)
                    tot += L.hip_event_elapsed_ms(evc[0], evc[1])
            cold[mode] = tot * 1e3 / args.cold_steps
        L.hip_events_destroy(evc)
        del scrub
        log(f"[bench] cold replay {cold['read']:.1f} us/step (read scrub), {cold['write']:.1f} (write scrub)")

    # ---------------- the step with the pre-block residual add + RMSNorm fused
    # into the router pass (graph replays, same weights, own workspace)
    prenorm = None
    if not args.no_prenorm and T <= 64:
        pl = lay.with_options()
        pin = S.prenorm_inputs(T, H)
        res_s, del_s, gam_s = (pl.upload_x(pin[k]) for k in ("residual", "delta", "gamma"))
        x_s = torch.empty(T, H, dtype=torch.int16, device="cuda")
        r_s = torch.empty(T, H, dtype=torch.int16, device="cuda")
        o_s = torch.empty(T, H, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        pl.capture_prenorm([T], res_s, del_s, gam_s, float(pin["eps"]), r_s, x_s, o_s, stream)
        evp = L.hip_events(2, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)
        times = {}
        for tag, g in (("fused", pl), ("block_only", lay)):
            for _ in range(10):
                g.replay(T, stream)
            L.hip_event_record(evp[0], stream)
            for _ in range(args.steps):
                g.replay(T, stream)
            L.hip_event_record(evp[1], stream)
            torch.cuda.synchronize()
            times[tag] = L.hip_event_elapsed_ms(evp[0], evp[1]) * 1e3 / args.steps
        L.hip_events_destroy(evp)
        pl.release_graph()
        prenorm = {"us_per_step": round(times["fused"], 2), "tokens_per_s": round(T / times["fused"] * 1e6, 1),
                   "block_only_us_per_step": round(times["block_only"], 2),
                   "fused_step_extra_us": round(times["fused"] - times["block_only"], 2)}
        log(f"[bench] pre-block step fused: {times['fused']:.1f} us/step vs block alone "
            f"{times['block_only']:.1f} us/step")

    # ---------------- the step with rank-16 fp32 LoRA adapters fused into the
    # expert GEMMs (graph replays, same weights, own workspace)
    lora = None
    if not args.no_lora:
        ll = lay.with_lora(S.lora_adapters(E, H, I))
        xl = ll.upload_x(inp.x)
        ol = torch.empty(T, H, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        ll.capture([T], xl, ol, stream)
        evl = L.hip_events(2, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)
        for _ in range(10):
            ll.replay(T, stream)
        L.hip_event_record(evl[0], stream)
        for _ in range(args.steps):
            ll.replay(T, stream)
        L.hip_event_record(evl[1], stream)
        torch.cuda.synchronize()
        t_l = L.hip_event_elapsed_ms(evl[0], evl[1]) * 1e3 / args.steps
        L.hip_events_destroy(evl)
        ll.release_graph()
        lora = {"rank": 16, "us_per_step": round(t_l, 2), "tokens_per_s": round(T / t_l * 1e6, 1),
                "extra_us_vs_block": round(t_l - gpu_ms * 1e3 / args.steps, 2),
                "adapter_bytes_per_step": int(n_act * 16 * 4 * (H + 2 * I + I + H))}
        log(f"[bench] with rank-16 LoRA: {t_l:.1f} us/step")

    # ---------------- backward (frozen weights, the forward's routing): input
    # and routing-weight gradients, eager, HIP events around the call
    backward = None
    if not args.no_backward and not args.row_major:
        d_out = torch.randn(T, H, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
        evb = L.hip_events(2, L.HIP_EVENT_DISABLE_SYSTEM_FENCE)
        tl = lay.with_options(train=True)   # a training forward keeps the pre-activations
        tb = 0.0
        nb = 20
        with torch.cuda.stream(stream):
            for i in range(nb + 3):
                tl.forward(x_static, T, out_static, stream=stream)
                L.hip_event_record(evb[0], stream)
                tl.backward(x_static, d_out, T, stream=stream)
                L.hip_event_record(evb[1], stream)
                torch.cuda.synchronize()
                if i >= 3:
                    tb += L.hip_event_elapsed_ms(evb[0], evb[1]) * 1e3 / nb
        # bytes the backward must move: both expert matrices of every active
        # expert again (bf16, or 4-bit codes + fp32 absmax per 64), the
        # forward's y, d_out, d_x
        w_e = 3 * I * H * 2 if inp.wfmt == "bf16" else 3 * I * H // 2 + 3 * I * H // 64 * 4
        bb = n_act * w_e + T * k * H * 4 + 2 * T * H * 4
        backward = {"us_per_step": round(tb, 2), "algorithmic_bytes": int(bb),
                    "hbm_frac": round(bb / (tb * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] backward (d_x, d_w): {tb:.1f} us, {backward['hbm_frac'] * 100:.1f}% of HBM peak")
        # with rank-16 LoRA adapters: the same plus the adapter gradients
        tll = tl.with_lora(S.lora_adapters(E, H, I))
        tbl = 0.0
        with torch.cuda.stream(stream):
            for i in range(nb + 3):
                tll.forward(x_static, T, out_static, stream=stream)
                L.hip_event_record(evb[0], stream)
                tll.backward(x_static, d_out, T, stream=stream)
                L.hip_event_record(evb[1], stream)
                torch.cuda.synchronize()
                if i >= 3:
                    tbl += L.hip_event_elapsed_ms(evb[0], evb[1]) * 1e3 / nb
        # plus the active experts' adapters read and every expert's adapter
        # gradient written (zeros where no row went)
        per_e = 16 * 4 * (2 * H + 3 * I)
        bbl = bb + n_act * per_e + E * per_e
        backward["lora"] = {"us_per_step": round(tbl, 2), "algorithmic_bytes": int(bbl),
                            "hbm_frac": round(bbl / (tbl * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] backward with LoRA gradients: {tbl:.1f} us, "
            f"{backward['lora']['hbm_frac'] * 100:.1f}% of HBM peak")
        # with the expert-weight gradients (fp32, every expert's full shape;
        # bf16 weights only: a 4-bit base is frozen)
        if inp.wfmt == "bf16":
            wg = (torch.empty(E, 2 * I, H, dtype=torch.float32, device="cuda"),
                  torch.empty(E, H, I, dtype=torch.float32, device="cuda"))
            tbw = 0.0
            with torch.cuda.stream(stream):
                for i in range(nb + 3):
                    tl.forward(x_static, T, out_static, stream=stream)
                    L.hip_event_record(evb[0], stream)
                    tl.backward(x_static, d_out, T, stream=stream, weight_grads=wg)
                    L.hip_event_record(evb[1], stream)
                    torch.cuda.synchronize()
                    if i >= 3:
                        tbw += L.hip_event_elapsed_ms(evb[0], evb[1]) * 1e3 / nb
            bbw = bb + E * 3 * I * H * 4
            backward["weight_grads"] = {"us_per_step": round(tbw, 2), "algorithmic_bytes": int(bbw),
                                        "hbm_frac": round(bbw / (tbw * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            log(f"[bench] backward with expert-weight gradients: {tbw:.1f} us, "
                f"{backward['weight_grads']['hbm_frac'] * 100:.1f}% of HBM peak")
            del wg
        L.hip_events_destroy(evb)

    # ---------------- measured ceilings of this chip in the same run
    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(torch, L, stream)
        log(f"[bench] ceilings: read stream {ceilings['stream_read_GBps']:.0f} GB/s, device copy "
            f"{ceilings['device_copy_GBps']:.0f} GB/s, MFMA 16x16x32 {ceilings['mfma_bf16_16x16x32_TFLOPs']:.0f} / "
            f"32x32x16 {ceilings['mfma_bf16_32x32x16_TFLOPs']:.0f} TFLOP/s, vendor bf16 GEMM "
            f"{ceilings['vendor_bf16_gemm_TFLOPs']:.0f} TFLOP/s")

    dominant = "gate_up"
    dom_us = stage_us[dominant]
    # the library runs the LDS-tiled MFMA kernels when the tiled layout (bf16
    # or 4-bit) has at least 32 routed rows per expert on average (prefill
    # sizes): those are bound by the matrix cores, the skinny decode kernels
    # by HBM
    mfma_path = not args.row_major and T * k >= 32 * E
    if mfma_path:
        dom_flops = 2.0 * T * k * H * 2 * I
        achieved = dom_flops / (dom_us * 1e-6) / 1e12
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = model[dominant] / (dom_us * 1e-6) / 1e9
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{dominant}_{args.workload}.json")
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            from mixture_experts_decode_router_amd.build import source_digest
            if tj.get("source_digest") == source_digest():
                traffic = tj.get("bytes_per_launch")
                if traffic is None:
                    cand = [v for kname, v in tj.get("kernels", {}).items() if kname.startswith(dominant)]
                    traffic = cand[0]["bytes_per_launch"] if len(cand) == 1 else None
        except Exception:
            traffic = None
    mfma_counter = None
    mpath = os.path.join(ROOT, "profiles", f"mfma_util_{args.workload}.json")
    if mfma_path and os.path.exists(mpath):
        try:
            mj = json.load(open(mpath))
            from mixture_experts_decode_router_amd.build import source_digest
            if mj.get("source_digest") == source_digest():
                kd = mj["kernels"].get("expert_mfma<true, false>")
                mfma_counter = kd["mfma_util_pct"] if kd else None
        except Exception:
            mfma_counter = None
    step_s = ms_per_step * 1e-3
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "value_cold": round(T / (cold["read"] * 1e-6), 1) if cold else None,
        "value_basis": "value: K back-to-back graph replays, wall clock between two synchronisations "
                       "(expert weights cannot stay in cache between steps; router weights, x and the "
                       "routing arrays can); value_cold: mean of single replays timed with HIP events, "
                       "a 512 MiB read scrub between them (outside the events) evicting L2 and the "
                       "last-level cache",
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
            "bound": bound,
            "achieved": round(achieved, 1),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": model[dominant],
            "algorithmic_flops_per_launch": 2 * T * k * H * 2 * I,
            "avg_launch_us": round(dom_us, 2),
            "mfma_busy_pct_counter": mfma_counter,
        },
        "block": {
            "algorithmic_bytes_per_step": model["block"],
            "hbm_frac": round(model["block"] / step_s / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_frac": round(model["flops"] / step_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "n_active_experts": n_act,
            "stage_us": {n: round(v, 2) for n, v in stage_us.items()},
            "bucketing": bucketing,
            "gpu_event_us_per_step": round(gpu_ms * 1e3 / args.steps, 2),
            "replay_us": replay_pct,
            "cold_us_per_step": round(cold["read"], 2) if cold else None,
            "cold_write_scrub_us_per_step": round(cold["write"], 2) if cold else None,
        },
        "ceilings": ceilings,
        "prenorm": prenorm,
        "lora": lora,
        "backward": backward,
    }

    if args.sweep and T <= 64:
        sweep = {}
        for b in buckets:
            xb = lay.upload_x(make_workload(args.workload, T=b).x)
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
