"""Benchmark of the fused MoE layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of fused_moe (routing, sort, activation quantisation for
fp8, grouped GEMM1 + SwiGLU, grouped GEMM2 + weighted combine) over one batch
of synthetic, seeded inputs already resident in HBM. The default workload is
the Mixtral-8x7B-shaped decode layer (T=32, d=4096, f=14336, E=8, top-2,
bf16). One JSON line goes to stdout. Besides the standard fields it reports:

  roofline      the dominant kernel (GEMM1 + SwiGLU) against its roofline:
                algorithmic bytes (or FLOPs) per launch over its mean duration,
                timed with HIP events on the stream it runs on;
  layer         the whole layer against the HBM and MFMA rooflines;
  ms_per_call   median, minimum and maximum of K calls timed one by one
                with HIP events (after the timed region);
  stages        mean per-stage times of the same path;
  cpu_baseline  the CPU oracle on the host cores, on a bounded token sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8_token": 5000.0, "fp8_block": 5000.0, "mxfp4": 10100.0}
METRIC = "fused-MoE tokens/s + % HBM BW (decode) / % MFMA peak (prefill), Mixtral"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_AVG_FILE = os.path.join(ROOT, "profiles", "kernel_avg.json")
MFMA_COUNTERS_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")
XCDS = 8   # accelerator dies of an MI355X, each with its own GRBM counters
# the prefill layer measured beside a decode workload (same d, f, E, k, quant)
PREFILL_OF = {"mixtral_decode": "mixtral_prefill", "mixtral_mxfp4": "mixtral_prefill_mxfp4"}
KERNEL_SOURCES = ["moe_grouped_gemm_sorting_amd/csrc/gemm_stream.hip",
                  "moe_grouped_gemm_sorting_amd/csrc/gemm_tiled.hip",
                  "moe_grouped_gemm_sorting_amd/csrc/common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the GEMM kernels' code: the sources with comments and
    whitespace taken out, so that an edit of a comment keeps the records."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_decode")
    ap.add_argument("--B", type=int, default=0)
    ap.add_argument("--stage", type=int, default=0)
    ap.add_argument("--ksplit", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's backward (moe_backward, bf16 workloads) instead of the "
                         "forward; prints its own JSON line")
    ap.add_argument("--cpu-sample", type=int, default=32, help="tokens the CPU oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU sample until this much time has run")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill sub-measurement of the decode workloads")
    ap.add_argument("--kernel-stats-from", metavar="DIR",
                    help="record the GEMM kernels' average durations from a rocprofv3 "
                         "--kernel-trace --stats run of this workload into profiles/kernel_avg.json "
                         "(no GPU needed)")
    ap.add_argument("--mfma-counters-from", nargs="+", metavar="DIR",
                    help="turn rocprofv3 --pmc runs (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, "
                         "SQ_INSTS_VALU_MFMA_MOPS_*) of this workload into MFMA utilisation of the "
                         "GEMM kernels, recorded in profiles/mfma_counters.json (no GPU needed)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --calibrate-copy` into HBM bytes per GEMM1 launch and "
                         "record them in profiles/traffic.json (no GPU needed)")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def _pmc_values(run_dir, counter):
    """Counter values per kernel name (one per dispatch) from a rocprofv3 CSV."""
    import csv
    import glob
    path = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)[0]
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def record_traffic(workload, fetch_dir, write_dir):
    """HBM bytes per GEMM1 launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    each scaled by what the same counter reads for the 1 GiB device copy."""
    import workloads
    wl = workloads.get(workload)
    import moe_grouped_gemm_sorting_amd as moe
    B, _, _ = moe.moe_select_config(wl.T, wl.d, wl.f, wl.E, wl.k, wl.quant, cu_count=256)
    want = ("k_gemm_tiled" if B >= 64 else "k_gemm_stream")
    out = {}
    for name, d, ctr in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        m = _pmc_values(d, ctr)
        # the calibration copy is the largest copy dispatch of the run
        copy = max((max(v) for k, v in m.items() if "copy" in k.lower()), default=None)
        g1 = [sum(v) / len(v) for k, v in m.items() if want in k and "true" in k]
        if copy is None or not g1:
            raise SystemExit(f"{ctr}: copy kernel or GEMM1 kernel not found in {d}")
        factor = COPY_BYTES / (copy * 1024.0)
        out[name] = {"counter_kib": g1[0], "copy_counter_kib": copy, "factor": factor,
                     "bytes": g1[0] * 1024.0 * factor}
    rec = {"kernel": f"{want} GEMM1 (B={B})", "fetch": out["fetch"], "write": out["write"],
           "bytes_per_launch": round(out["fetch"]["bytes"] + out["write"]["bytes"]),
           "source_hash": kernel_source_hash()}
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        data = {}
    data[wl.name] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1)
    print(json.dumps(rec))


def _gemm_kernel_matchers(wl):
    """The library's block size for the workload and two predicates that pick
    its GEMM1 and GEMM2 kernels out of a trace by name (the kernel and its
    template arguments follow the block size and the quant type)."""
    import moe_grouped_gemm_sorting_amd as moe
    B, _, _ = moe.moe_select_config(wl.T, wl.d, wl.f, wl.E, wl.k, wl.quant, cu_count=256)
    q = moe.QUANT[wl.quant]
    if B >= 64:
        return (B, lambda n: f"k_gemm_tiled<{q}, true, {B}," in n,
                lambda n: f"k_gemm_tiled<{q}, false, {B}," in n)
    return (B, lambda n: f"k_gemm_stream<{q}," in n and "true>" in n,
            lambda n: f"k_gemm_stream<{q}," in n and "false>" in n)


def record_kernel_avg(workload, run_dir):
    """Average GEMM1 / GEMM2 durations of `workload` (and of the prefill layer
    measured beside it) from a rocprofv3 --kernel-trace --stats CSV, recorded
    in profiles/kernel_avg.json with the kernel sources' hash."""
    import csv
    import glob

    import workloads
    paths = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    rows = list(csv.DictReader(open(paths[0])))
    try:
        data = json.load(open(KERNEL_AVG_FILE))
    except (OSError, ValueError):
        data = {}
    names = [workload] + ([PREFILL_OF[workload]] if workload in PREFILL_OF else [])
    for wn in names:
        wl = workloads.get(wn)
        B, m1, m2 = _gemm_kernel_matchers(wl)
        rec = {"B": B, "source_hash": kernel_source_hash(), "run": os.path.basename(paths[0])}
        for label, match in (("gemm1", m1), ("gemm2", m2)):
            hit = [r for r in rows if match(r["Name"])]
            if len(hit) != 1:
                raise SystemExit(f"{wn} {label}: {len(hit)} kernels match")
            r = hit[0]
            rec[label] = {"kernel": r["Name"], "calls": int(r["Calls"]),
                          "avg_us": round(float(r["AverageNs"]) / 1e3, 2),
                          "min_us": round(float(r["MinNs"]) / 1e3, 2),
                          "max_us": round(float(r["MaxNs"]) / 1e3, 2)}
        data[wn] = rec
        print(json.dumps({wn: rec}))
    with open(KERNEL_AVG_FILE, "w") as fh:
        json.dump(data, fh, indent=1)


def record_mfma_counters(workload, run_dirs):
    """MFMA utilisation of `workload`'s GEMM kernels from rocprofv3 --pmc runs
    (one or more; each counter is averaged over the kernel's dispatches):
      busy = MfmaUtil / 100, rocprofv3's derived metric: the MFMA-busy cycles
             of all SIMDs (SQ_VALU_MFMA_BUSY_CYCLES) over GRBM_GUI_ACTIVE
             times the SIMD count;
      counted FLOPs = 512 x SQ_INSTS_VALU_MFMA_MOPS_<type> (MFMA operations,
             padding rows included), per second of kernel time from the
             committed trace average, against the dtype's peak;
      clock = GRBM_GUI_ACTIVE cycles per dispatch (rocprofv3 sums them over
             the 8 XCDs; GRBM_COUNT reads the same) over 8 times the traced
             kernel time (when a run collected it): the clock the kernel ran
             at, and the counted rate against the peak scaled to that clock
             (the quoted peaks assume 2.4 GHz)."""
    import workloads
    wl = workloads.get(workload)
    B, m1, m2 = _gemm_kernel_matchers(wl)
    vals = {}
    for d in run_dirs:
        import csv
        import glob
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        for r in csv.DictReader(open(path)):
            vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    kav = committed_record(KERNEL_AVG_FILE, wl.name) or {}
    ncu = 256
    peak = MFMA_PEAK_TFLOPS[wl.quant]
    out = {"B": B, "cus": ncu, "source_hash": kernel_source_hash(), "peak_TFLOPs": peak}
    for label, match in (("gemm1", m1), ("gemm2", m2)):
        hit = [k for k in vals if match(k)]
        if len(hit) != 1:
            raise SystemExit(f"{label}: {len(hit)} kernels match")
        c = {n: float(np.mean(v)) for n, v in vals[hit[0]].items()}
        rec = {"kernel": hit[0], "counters_per_dispatch": {n: round(v) for n, v in c.items()}}
        if "MfmaUtil" in c:   # rocprofv3's derived metric, in percent
            rec["mfma_busy_frac"] = round(c["MfmaUtil"] / 100.0, 4)
        mops = [v for n, v in c.items() if n.startswith("SQ_INSTS_VALU_MFMA_MOPS")]
        if mops:
            rec["counted_flops"] = 512.0 * sum(mops)
            if kav.get(label):
                us = kav[label]["avg_us"]
                rec["counted_TFLOPs"] = round(rec["counted_flops"] / (us * 1e-6) / 1e12, 1)
                rec["counted_frac_of_peak"] = round(rec["counted_TFLOPs"] / peak, 4)
        if "GRBM_GUI_ACTIVE" in c and kav.get(label):
            ghz = c["GRBM_GUI_ACTIVE"] / XCDS / (kav[label]["avg_us"] * 1e3)
            rec["gui_active_GHz"] = round(ghz, 3)
            if "counted_TFLOPs" in rec:
                rec["counted_frac_of_clock_peak"] = round(rec["counted_TFLOPs"] / (peak * ghz / 2.4), 4)
        out[label] = rec
    # the line's roofline object reports GEMM1
    for k in ("mfma_busy_frac", "counted_flops", "counted_frac_of_peak", "gui_active_GHz",
              "counted_frac_of_clock_peak", "kernel"):
        if k in out["gemm1"]:
            out[k] = out["gemm1"][k]
    try:
        data = json.load(open(MFMA_COUNTERS_FILE))
    except (OSError, ValueError):
        data = {}
    data[wl.name] = out
    with open(MFMA_COUNTERS_FILE, "w") as fh:
        json.dump(data, fh, indent=1)
    print(json.dumps(out))


def backward_block(T, d, f, E, k):
    """The library's default sort block for the backward (streaming kernels
    for few rows per expert, tiled kernels from 64 rows per expert on)."""
    rows = T * k / E
    if rows >= 2 and d % 256 == 0 and f % 256 == 0:
        return 256 if rows >= 192 else (128 if rows >= 48 else 64)
    return 16 if rows <= 4 else 32


def bench_backward(args, wl, x, logits, ws, dev):
    """K steps of moe_backward on resident inputs (the forward's routing, a
    random output gradient). Roofline: whichever bound takes longer at its
    peak: HBM, counting each touched expert's weights read once, every
    expert's fp32 weight gradients written once, and x, dy, dx; or the bf16
    MFMAs, counting 16 d f FLOPs per assignment (the weight gradients' hi/lo
    split not included)."""
    import torch

    import moe_grouped_gemm_sorting_amd as moe

    if wl.quant != "bf16":
        print("the backward is built for bf16 layers", file=sys.stderr)
        sys.exit(2)
    ids, w = moe.moe_topk(logits, wl.k, wl.score)
    g = torch.Generator(device=dev).manual_seed(wl.seed + 7)
    dy = torch.randn(wl.T, wl.d, generator=g, device=dev).bfloat16()
    B = args.B
    nbytes = moe.moe_backward_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, B)
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step():
        moe.moe_backward(x, ws["w13"], ws["w2"], dy, ids, w, B=B, workspace=workspace)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    touched = int(torch.unique(ids).numel())
    d, f, E, T = wl.d, wl.f, wl.E, wl.T
    wbytes = touched * 3 * f * d * 2 + E * 3 * f * d * 4 + 3 * T * d * 2
    # per assignment: GEMM1 recompute 4df, dh 2df, dx 4df, dW13 4df, dW2 2df
    flops = 16 * T * wl.k * d * f
    gbs = wbytes / (ms * 1e-3) / 1e9
    log(f"[bench] moe_backward: {ms * 1e3:.1f} us/step, {T / (ms / 1e3):,.0f} tokens/s, "
        f"{gbs:.0f} GB/s against the algorithmic bytes")
    result = {
        "metric": "fused-MoE backward tokens/s (bf16; dx, dW13, dW2, routing-weight gradients)",
        "value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "d": d, "f": f, "E": E, "k": wl.k,
                   "B": B or backward_block(T, d, f, E, wl.k), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "the whole backward",
                     "algorithmic_bytes": wbytes, "flops": flops, "touched_experts": touched},
    }
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS["bf16"]
    if flops / (peak * 1e12) > wbytes / (HBM_PEAK_GBS * 1e9):
        hbm = {k: result["roofline"][k] for k in ("achieved", "peak", "unit", "frac")}
        result["roofline"].update({"bound": "mfma", "achieved": round(tflops, 1), "peak": peak,
                                   "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "hbm": hbm})
        log(f"[bench] moe_backward: {tflops:.0f} TFLOP/s = {tflops / peak:.3f} of the bf16 MFMA peak")
    print(json.dumps(result), flush=True)


def measure_forward(args, wl, x, logits, ws, dev, label):
    """Time K fused_moe steps of workload `wl` on resident inputs (after W
    warm-up steps, bracketed by device synchronisations), then each stage
    with HIP events on the library's stream; return the step time, the
    stage times and the roofline and whole-layer figures."""
    import torch

    import moe_grouped_gemm_sorting_amd as moe

    B, stage, ksplit = moe.moe_select_config(wl.T, wl.d, wl.f, wl.E, wl.k, wl.quant)
    B = args.B or B
    stage = args.stage or stage
    ksplit = args.ksplit or ksplit
    nbytes = moe.fused_moe_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, wl.quant, B, stage)
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device=dev)

    def step():
        moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, quant=wl.quant,
                      w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score,
                      B=B, stage=stage, ksplit=ksplit, out=out, workspace=workspace)

    # ---- timed region: K whole-layer steps --------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    log(f"[bench] {label} fused_moe: {ms * 1e3:.1f} us/step, {wl.T / (ms / 1e3):,.0f} tokens/s")

    # ---- each call on its own, HIP events on the library's stream: median,
    # minimum and maximum of K calls (outside the timed region) -------------
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    calls = np.array([a.elapsed_time(b) for a, b in evs])
    per_call = {"median": round(float(np.median(calls)), 4), "min": round(float(calls.min()), 4),
                "max": round(float(calls.max()), 4)}

    # ---- per-stage timing with HIP events on the library's stream -----------
    ids, w = moe.moe_topk(logits, wl.k, wl.score)
    srt = moe.moe_sort(ids, w, wl.E, B)
    h, hs = moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, B, wl.quant, ws["w13_scale"])
    g2ws = torch.empty(moe.moe_gemm2_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, B, wl.quant),
                       dtype=torch.uint8, device=dev)
    g1ws = torch.empty(max(1, moe.moe_gemm1_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, B,
                                                            wl.quant)), dtype=torch.uint8,
                       device=dev)
    stage_fns = {
        "topk": lambda: moe.moe_topk(logits, wl.k, wl.score),
        "sort": lambda: moe.moe_sort(ids, w, wl.E, B),
        "gemm1_swiglu": lambda: moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, B, wl.quant,
                                                     ws["w13_scale"], workspace=g1ws),
        "gemm2_combine": lambda: moe.moe_gemm2_combine(h, hs, ws["w2"], srt, wl.T, wl.k, B,
                                                       wl.quant, ws["w2_scale"], ksplit=ksplit,
                                                       out=out, workspace=g2ws),
    }
    stages = {}
    for name, fn in stage_fns.items():
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        stages[name] = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3  # us
    log(f"[bench] {label} stages (us): " + ", ".join(f"{k}={v:.1f}" for k, v in stages.items()))

    # ---- algorithmic work ----------------------------------------------------
    counts = srt["expert_counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    if wl.quant == "mxfp4":   # E2M1 codes two per byte + one E8M0 byte per 32
        w13_bytes = touched * 2 * wl.f * (wl.d // 2 + wl.d // 32)
    else:
        eb = 2 if wl.quant == "bf16" else 1
        w13_bytes = touched * 2 * wl.f * wl.d * eb
    if wl.quant == "fp8_token":
        w13_bytes += touched * 2 * wl.f * 4
    elif wl.quant == "fp8_block":
        w13_bytes += touched * (2 * wl.f // 128) * (wl.d // 128) * 4
    g1_bytes = w13_bytes + wl.T * wl.d * 2
    g1_flops = 4 * wl.d * wl.f * wl.T * wl.k
    layer_bytes = touched * wl.weight_bytes_per_expert() + wl.T * wl.d * 2 * 2 + wl.T * wl.E * 4
    layer_flops = wl.flops()
    g1_us = stages["gemm1_swiglu"]
    hbm_bound = (layer_bytes / HBM_PEAK_GBS) > (layer_flops / (MFMA_PEAK_TFLOPS[wl.quant] * 1e3))
    if hbm_bound:
        achieved = g1_bytes / (g1_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = g1_flops / (g1_us * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS[wl.quant]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["kernel"] = "GEMM1 + SwiGLU (moe_gemm1_swiglu)"
    roof["kernel_us"] = round(g1_us, 2)
    roof["algorithmic_per_launch"] = {"bytes": g1_bytes, "flops": g1_flops,
                                      "touched_experts": touched}
    roof["traffic"] = None
    rec = committed_record(TRAFFIC_FILE, wl.name)
    if rec:
        roof["traffic"] = rec["bytes_per_launch"]
    # the same kernel's average duration in the committed rocprofv3 trace of
    # this workload (same sources), for comparison with the HIP-event time
    kav = committed_record(KERNEL_AVG_FILE, wl.name)
    roof["rocprof_avg_us"] = None
    if kav and kav.get("gemm1"):
        roof["rocprof_avg_us"] = kav["gemm1"]["avg_us"]
        roof["rocprof_kernel"] = kav["gemm1"]["kernel"]
        roof["event_vs_rocprof"] = round(g1_us / kav["gemm1"]["avg_us"] - 1.0, 4)
        log(f"[bench] {label} GEMM1: {g1_us:.1f} us (HIP events) against {kav['gemm1']['avg_us']:.1f} us "
            f"(committed rocprofv3 average of {kav['gemm1']['kernel']})")
    counters = committed_record(MFMA_COUNTERS_FILE, wl.name)
    if counters:
        roof["mfma_counters"] = {k: counters[k] for k in ("mfma_busy_frac", "counted_flops",
                                                            "counted_frac_of_peak", "gui_active_GHz",
                                                            "counted_frac_of_clock_peak", "kernel")
                                 if k in counters}
    layer = {
        "bytes": layer_bytes, "flops": layer_flops,
        "hbm_GBs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "TFLOPs": round(layer_flops / (ms * 1e-3) / 1e12, 2),
        "mfma_frac": round(layer_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[wl.quant], 4),
    }
    return dict(ms=ms, B=B, stage=stage, ksplit=ksplit, stages=stages, roof=roof, layer=layer,
                per_call=per_call)


def committed_record(path, workload):
    """The workload's record in a committed profiles/*.json file, if it was
    taken with the current kernel sources (else None)."""
    try:
        with open(path) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if rec and rec.get("source_hash") == kernel_source_hash():
        return rec
    return None


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(args, wl, x, logits, ws):
    """The CPU oracle (test infrastructure) on the host cores: the workload's
    first tokens (a bounded sample) repeated for about --cpu-seconds on all
    threads, plus single-thread times of the tiny layer and of the sample."""
    import torch

    import oracle
    import workloads

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    n = min(args.cpu_sample, wl.T)
    tokens = np.arange(n, dtype=np.int32)
    lg = logits.cpu().numpy()
    rid, rw = oracle.route(lg, wl.k, wl.score)
    need = sorted(set(rid[tokens].ravel().tolist()))
    b16 = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)  # noqa
    w13 = [None] * wl.E
    w2 = [None] * wl.E
    s13 = [None] * wl.E if wl.quant != "bf16" else None
    s2 = [None] * wl.E if wl.quant != "bf16" else None
    for e in need:
        if wl.quant == "bf16":
            w13[e], w2[e] = b16(ws["w13"][e]), b16(ws["w2"][e])
        else:
            w13[e], w2[e] = ws["w13"][e].cpu().numpy(), ws["w2"][e].cpu().numpy()
            s13[e], s2[e] = ws["w13_scale"][e].cpu().numpy(), ws["w2_scale"][e].cpu().numpy()
    xb = b16(x)
    # repeat the sample until about cpu_seconds of CPU work have run
    reps, t0 = 0, time.perf_counter()
    while True:
        rid, rw = oracle.route(lg, wl.k, wl.score)
        oracle.moe(xb, rid, rw, w13, w2, s13, s2, quant=wl.quant, tokens=tokens, threads=threads)
        reps += 1
        sec = time.perf_counter() - t0
        if sec >= args.cpu_seconds:
            break
    # one thread: the sample once, and the whole tiny layer
    t1 = time.perf_counter()
    oracle.moe(xb, rid, rw, w13, w2, s13, s2, quant=wl.quant, tokens=tokens, threads=1)
    one = time.perf_counter() - t1
    tiny = workloads.get("tiny")
    tx, tl = tiny.activations("cpu")
    tw = tiny.weights("cpu")
    tid_, tw_ = oracle.route(tl.numpy(), tiny.k, tiny.score)
    t2 = time.perf_counter()
    oracle.moe(b16(tx), tid_, tw_, [b16(tw["w13"][e]) for e in range(tiny.E)],
               [b16(tw["w2"][e]) for e in range(tiny.E)], threads=1)
    tiny_s = time.perf_counter() - t2
    log(f"[bench] CPU oracle: {n} tokens x {reps} in {sec:.1f} s on {threads} threads; "
        f"one thread {one:.2f} s")
    return {"value": round(n * reps / sec, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {wl.T} tokens of {wl.name}, routed and run through the per-token "
                      f"fp32 expert loop {reps} times ({sec:.1f} s)",
            "cpu_model": cpu_info(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "seconds_per_sample": round(sec / reps, 3),
            "single_thread": {"sample_s": round(one, 3), "tokens_per_s": round(n / one, 3),
                              "tiny_layer_s": round(tiny_s, 4)}}


def main():
    args = parse()
    if args.traffic_from:
        record_traffic(args.workload, *args.traffic_from)
        return
    if args.kernel_stats_from:
        record_kernel_avg(args.workload, args.kernel_stats_from)
        return
    if args.mfma_counters_from:
        record_mfma_counters(args.workload, args.mfma_counters_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer is built and measured on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    wl = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] {wl.name}: T={wl.T} d={wl.d} f={wl.f} E={wl.E} k={wl.k} quant={wl.quant} "
        f"on {torch.cuda.get_device_name(0)}")
    x, logits = wl.activations(dev)
    ws = wl.weights(dev)
    torch.cuda.synchronize()
    if args.backward:
        bench_backward(args, wl, x, logits, ws, dev)
        return

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    m = measure_forward(args, wl, x, logits, ws, dev, wl.name)
    ms = m["ms"]
    tokens_per_s = wl.T / (ms / 1e3)

    # the prefill half of the metric: the Mixtral-shaped layer at T = 4096 on
    # the same weights, timed the same way
    prefill = None
    if PREFILL_OF.get(wl.name) and not args.no_prefill:
        pw = workloads.get(PREFILL_OF[wl.name])
        px, plog = pw.activations(dev)
        pm = measure_forward(args, pw, px, plog, ws, dev, pw.name)
        prefill = {"workload": pw.name, "T": pw.T, "weights": f"those of {wl.name}",
                   "value": round(pw.T / (pm["ms"] / 1e3), 1), "unit": "tokens/s",
                   "ms_per_step": round(pm["ms"], 4), "ms_per_call": pm["per_call"],
                   "B": pm["B"], "stage": pm["stage"],
                   "ksplit": pm["ksplit"], "roofline": pm["roof"], "layer": pm["layer"],
                   "stages_us": {k: round(v, 2) for k, v in pm["stages"].items()}}
        del px, plog

    cpu = None if args.no_cpu_baseline else cpu_baseline(args, wl, x, logits, ws)
    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_call": m["per_call"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "mxfp4": "mxfp4_e2m1"}.get(wl.quant, "fp8_e4m3"), "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "f": wl.f, "E": wl.E, "k": wl.k,
                   "quant": wl.quant, "score": wl.score, "B": m["B"], "stage": m["stage"],
                   "ksplit": m["ksplit"], "parallelism": "single GPU"},
        "roofline": m["roof"], "layer": m["layer"],
        "stages_us": {k: round(v, 2) for k, v in m["stages"].items()},
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
