"""Shared helpers of the GPU parity tests (the HIP library against the CPU oracle)."""
import os

import numpy as np
import torch

import oracle

DEV = "cuda:0"

# Output tolerances: relative error floored at the output RMS.
TOL = {"bf16": 2e-2, "fp8_token": 6e-2, "fp8_block": 6e-2, "mxfp4": 6e-2}


def log(msg):
    print(msg, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(b).astype(np.float64)


def rel_err(y, ref, slack=None):
    """max_i |y_i - ref_i| / max(|ref_i|, rms(ref)), plus the normwise error.

    slack maps a row of a 2-D ref to a per-column allowance (the output
    changes of that row's h rounding ties, see oracle_layer): the row's
    deviation counts only beyond it, under the same rms floor."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if rms == 0.0:
        return (float(np.abs(y - ref).max()) if y.size else 0.0), 0.0
    norm = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    dev = np.abs(y - ref)
    if slack:
        for r, a in slack.items():
            dev[r] = np.maximum(dev[r] - a, 0.0)
    return float(np.max(dev / np.maximum(np.abs(ref), rms))), norm


def host_experts(wl, ws, experts):
    """Per-expert numpy views of the device weights for the oracle (None elsewhere)."""
    E = wl.E
    w13, w2 = [None] * E, [None] * E
    s13 = [None] * E if wl.quant != "bf16" else None
    s2 = [None] * E if wl.quant != "bf16" else None
    for e in experts:
        if wl.quant == "bf16":
            w13[e] = bits(ws["w13"][e])
            w2[e] = bits(ws["w2"][e])
        else:
            w13[e] = ws["w13"][e].cpu().numpy()
            w2[e] = ws["w2"][e].cpu().numpy()
            s13[e] = ws["w13_scale"][e].cpu().numpy()
            s2[e] = ws["w2_scale"][e].cpu().numpy()
    return w13, w2, s13, s2


# Relative distance from a bf16 rounding midpoint within which the fp32 value
# of h may round either way. The oracle's fp32 sums stay within a few units
# of 2^-24 times their terms' magnitudes. The e4m3 matrix instruction
# (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales) does not add its 64
# products exactly: with every lane holding the same operand bytes, its
# results missed the exact sums by up to 4.3e-5 (2^-14.5) of the sum of the
# products' magnitudes, typically 2^-15 to 2^-17, and small products next to
# a large one were partly dropped. The GPU's h has been seen 2.13e-5 from
# its fp64 value (both GEMM1 kernels of a per-token e4m3 layer alike); the
# band is about three times that.
TIE_BAND = 2.0 ** -14


def oracle_layer(wl, x, logits, ws, tokens=None, ids=None, w=None, chunk=256, slack=None):
    """Oracle output rows (bf16 values as fp64) for `tokens` (default: all),
    computed `chunk` tokens at a time with a progress line per chunk.

    With a dict `slack` (quantised layers), each row whose h holds elements
    that the oracle reports as bf16 rounding ties (the other rounding moves
    a group scale or a code) gets slack[row] = sum over its ties of
    |output with that tie rounded the other way - output|, from the fp32
    outputs. The output is linear in each quantisation group's dequantised
    h, so any mix of the two roundings moves a row by at most about that
    sum (exactly so for ties in different groups)."""
    import time
    if ids is None:
        ids, w = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    tok = np.arange(wl.T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    need = sorted(set(ids[tok].ravel().tolist()))
    w13, w2, s13, s2 = host_experts(wl, ws, need)
    xb = bits(x)
    # Tokens go to the oracle ordered by their experts (each token's row is
    # computed on its own, so the order changes no value): threads working
    # at the same time then read the same expert weights. The thread count
    # is passed explicitly, as the process's OpenMP default can be lower.
    order = np.lexsort(tuple(ids[tok, j] for j in reversed(range(wl.k))))
    threads = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    out = np.empty((tok.size, wl.d), np.uint16)
    y32 = np.empty((tok.size, wl.d), np.float32)
    want_ties = slack is not None and wl.quant != "bf16"
    ties = {}
    t0 = time.perf_counter()
    for i in range(0, tok.size, chunk):
        sel = order[i:i + chunk]
        res = oracle.moe(xb, ids, w, w13, w2, s13, s2, quant=wl.quant, tokens=tok[sel],
                         threads=threads, tie_band=TIE_BAND if want_ties else 0.0)
        y32[sel], out[sel] = res[0], res[1]
        if want_ties:
            for p, j, n in res[2].tolist():
                ties.setdefault(int(sel[p]), []).append((j, n))
        if tok.size > chunk:
            done = min(tok.size, i + chunk)
            dt = time.perf_counter() - t0
            log(f"    oracle {wl.name}: {done}/{tok.size} tokens, {dt:.1f} s ({done / dt:.1f} tokens/s, "
                f"{threads} threads)")
    if ties:
        # one oracle call for every tie: row p of the call is a token with
        # one of its ties rounded the other way
        vt, flips, owner = [], [], []
        for r, lst in sorted(ties.items()):
            for j, n in lst:
                p = len(vt)
                vt.append(tok[r])
                owner.append(r)
                flips.append((p * wl.k + j) * wl.f + n)
        vy, _ = oracle.moe(xb, ids, w, w13, w2, s13, s2, quant=wl.quant,
                           tokens=np.asarray(vt, np.int32), threads=threads, h_flip=flips)
        for p, r in enumerate(owner):
            d = np.abs(vy[p].astype(np.float64) - y32[r])
            slack[r] = slack[r] + d if r in slack else d
        log(f"    oracle {wl.name}: {len(ties)} rows with h rounding ties ({len(vt)} ties)")
    return bf16_to_f64(out), ids, w
