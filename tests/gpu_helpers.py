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


def rel_err(y, ref):
    """max_i |y_i - ref_i| / max(|ref_i|, rms(ref)), plus the normwise error."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if rms == 0.0:
        return (float(np.abs(y - ref).max()) if y.size else 0.0), 0.0
    err = float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), rms)))
    norm = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    return err, norm


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


def oracle_layer(wl, x, logits, ws, tokens=None, ids=None, w=None, chunk=256):
    """Oracle output rows (bf16 values as fp64) for `tokens` (default: all),
    computed `chunk` tokens at a time with a progress line per chunk."""
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
    t0 = time.perf_counter()
    for i in range(0, tok.size, chunk):
        sel = order[i:i + chunk]
        _, out[sel] = oracle.moe(xb, ids, w, w13, w2, s13, s2, quant=wl.quant, tokens=tok[sel],
                                 threads=threads)
        if tok.size > chunk:
            done = min(tok.size, i + chunk)
            dt = time.perf_counter() - t0
            log(f"    oracle {wl.name}: {done}/{tok.size} tokens, {dt:.1f} s ({done / dt:.1f} tokens/s, "
                f"{threads} threads)")
    return bf16_to_f64(out), ids, w
