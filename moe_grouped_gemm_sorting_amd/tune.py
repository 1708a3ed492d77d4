"""Offline sweep of the layer's configuration (block size B, stage, K-split)
per shape, written as the CSV that ``moe_load_config_table`` reads.

The AITER walk-through (section 4) tunes its GEMMs offline and keeps the
winners in a CSV keyed by shape; this is the same idea for the fused layer:
every supported (B, stage, ksplit) is timed on resident synthetic inputs of
the shape with HIP events, and the fastest is kept.

    python -m moe_grouped_gemm_sorting_amd.tune --preset mixtral --out table.csv
    python -m moe_grouped_gemm_sorting_amd.tune --shape 32,4096,14336,8,2,bf16 --out table.csv

Values do not change the timing of these kernels, so the inputs are simple
random tensors of the right formats (not the parity workloads).
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys

import torch

import moe_grouped_gemm_sorting_amd as moe

B_CHOICES = (16, 32, 64, 128, 256)
KSPLITS = (1, 2, 4, 8)
MIXTRAL_T = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)
DEEPSEEK_T = (1, 4, 16, 32, 64, 128, 256, 512)


def _weights(d, f, E, quant, dev):
    """w13 [E, 2f, d], w2 [E, d, f] and their scales in the layout of include/moe.h."""
    g = torch.Generator(device=dev).manual_seed(1)
    if quant == "mxfp4":
        w13 = torch.randint(0, 256, (E, 2 * f, d // 2), generator=g, device=dev, dtype=torch.uint8)
        w2 = torch.randint(0, 256, (E, d, f // 2), generator=g, device=dev, dtype=torch.uint8)
        s13 = torch.full((E, 2 * f, d // 32), 120, device=dev, dtype=torch.uint8)
        s2 = torch.full((E, d, f // 32), 120, device=dev, dtype=torch.uint8)
        return w13, w2, s13, s2
    w13 = torch.randn(E, 2 * f, d, generator=g, device=dev) * d ** -0.5
    w2 = torch.randn(E, d, f, generator=g, device=dev) * f ** -0.5
    if quant == "bf16":
        return w13.bfloat16(), w2.bfloat16(), None, None
    w13 = (w13 * 64).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    w2 = (w2 * 64).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    if quant == "fp8_token":
        s13 = torch.full((E, 2 * f), 1 / 64, device=dev)
        s2 = torch.full((E, d), 1 / 64, device=dev)
    else:
        s13 = torch.full((E, 2 * f // 128, d // 128), 1 / 64, device=dev)
        s2 = torch.full((E, d // 128, f // 128), 1 / 64, device=dev)
    return w13, w2, s13, s2


def _time_us(fn, iters):
    for _ in range(2):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)


def tune_shape(T, d, f, E, k, quant, score, weights, iters, dev):
    """Rows (B, stage, ksplit, us) of every supported configuration, fastest first,
    and the time of the library's built-in choice."""
    g = torch.Generator(device=dev).manual_seed(2)
    x = torch.randn(T, d, generator=g, device=dev).bfloat16()
    logits = torch.randn(T, E, generator=g, device=dev)
    w13, w2, s13, s2 = weights
    out = torch.empty(T, d, device=dev, dtype=torch.bfloat16)
    cands = [(B, 2, ks) for B in B_CHOICES for ks in KSPLITS]
    if quant == "bf16":
        cands += [(B, 1, 1) for B in (16, 32)]
    builtin = moe.moe_select_config(T, d, f, E, k, quant)
    if builtin not in cands:
        cands.append(builtin)
    rows = []
    for B, stage, ks in cands:
        nbytes = moe.fused_moe_workspace_bytes(T, d, f, E, k, quant, B, stage)
        if nbytes == 0:
            continue
        ws = torch.empty(nbytes, device=dev, dtype=torch.uint8)

        def run():
            moe.fused_moe(x, w13, w2, k, logits=logits, quant=quant, w13_scale=s13, w2_scale=s2,
                          score=score, B=B, stage=stage, ksplit=ks, out=out, workspace=ws)
        try:
            run()
        except moe.MoeError:
            continue
        rows.append((B, stage, ks, _time_us(run, iters)))
    rows.sort(key=lambda r: r[3])
    base = next((r[3] for r in rows if r[:3] == builtin), float("nan"))
    return rows, base


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--shape", action="append", default=[],
                    help="T,d,f,E,k,quant[,score] (repeatable)")
    ap.add_argument("--preset", choices=["mixtral", "deepseek", "all"],
                    help="Mixtral-shaped bf16 / fp8_token / mxfp4 layers over T = 1..4096, and/or "
                         "DeepSeek-shaped fp8_block layers over T = 1..512")
    ap.add_argument("--out", required=True)
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--all", action="store_true", help="print every candidate's time")
    args = ap.parse_args(argv)

    shapes = []
    for s in args.shape:
        p = s.split(",")
        shapes.append((*map(int, p[:5]), p[5], p[6] if len(p) > 6 else "softmax"))
    if args.preset in ("mixtral", "all"):
        for q in ("bf16", "fp8_token", "mxfp4"):
            shapes += [(T, 4096, 14336, 8, 2, q, "softmax") for T in MIXTRAL_T]
    if args.preset in ("deepseek", "all"):
        shapes += [(T, 7168, 2048, 256, 8, "fp8_block", "sigmoid") for T in DEEPSEEK_T]
    if not shapes:
        ap.error("no shapes: give --shape or --preset")

    dev = "cuda:0"
    moe.moe_load_config_table(None)   # time the built-in choice, not a previous table
    props = torch.cuda.get_device_properties(dev)
    cu = props.multi_processor_count
    name = getattr(props, "gcnArchName", props.name).split(":")[0]
    lines = [f"# tuned configurations of the fused MoE layer on {name} ({cu} CUs)",
             "# columns after ksplit: fastest time, built-in choice's time (us)",
             "cu,T,d,f,E,k,quant,B,stage,ksplit,us,us_builtin"]
    weights, wkey = None, None
    for T, d, f, E, k, quant, score in shapes:
        if wkey != (d, f, E, quant):
            weights, wkey = None, None
            torch.cuda.empty_cache()
            weights, wkey = _weights(d, f, E, quant, dev), (d, f, E, quant)
        rows, base = tune_shape(T, d, f, E, k, quant, score, weights, args.iters, dev)
        if not rows:
            print(f"[tune] T={T} d={d} f={f} E={E} k={k} {quant}: no supported configuration",
                  file=sys.stderr, flush=True)
            continue
        if args.all:
            for r in rows:
                print(f"[tune]   T={T} {quant}: B={r[0]} stage={r[1]} ksplit={r[2]} {r[3]:.1f} us", flush=True)
        B, stage, ks, us = rows[0]
        lines.append(f"{cu},{T},{d},{f},{E},{k},{quant},{B},{stage},{ks},{us:.1f},{base:.1f}")
        print(f"[tune] T={T} d={d} f={f} E={E} k={k} {quant}: B={B} stage={stage} ksplit={ks} "
              f"{us:.1f} us (built-in {base:.1f} us)", flush=True)
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"[tune] wrote {len(lines) - 3} rows to {args.out}", flush=True)


if __name__ == "__main__":
    main()
