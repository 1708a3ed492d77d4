"""CPU oracle of the fused Mixture-of-Experts layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library never imports it, and
the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over tokens, fp32, no
BLAS, no fast-math, no FMA contraction). This module only builds it with gcc,
loads it with ctypes and marshals numpy arrays. Each function states the
passage it follows:

* :func:`route` -- top-k gating, the first stage of the fused MoE pipeline
  (AITER article, itsolotime.com/th/archives/32381, section 3).
* :func:`sort` -- token sort into expert-contiguous, block-padded groups
  (same article, section 3.1, ``_moe_sorting_impl`` and its sizing formulas).
* :func:`moe` -- per-token loop over the selected experts in fp32, SwiGLU
  expert FFN, weighted combine (same article, section 3; rocketrecap.com
  entries/19116, 5:58 and glossary "SwiGLU").
* :func:`e4m3_encode` / :func:`e4m3_decode` / :func:`quant_rows` -- OCP FP8
  E4M3FN and the amax/448 scale rule used by the fp8 layers (quant types
  per_Token and per_1x128 named in the AITER article, sections 1.1 and 3.2).
* :func:`moe_backward` -- the gradients of the bf16 layer (the training
  step named as the next milestone: rocketrecap.com/entries/19116, 10:07),
  from the chain rule of :func:`moe`; :func:`moe_backward_sampled` and
  :func:`moe_backward_expert` give selected entries and blocks of the same
  gradients in float64 for full-size layers.
* :func:`fp4_encode` / :func:`fp4_decode` / :func:`mx_quant_rows` -- MXFP4,
  the quant type per_1x32 (same article, sections 1.1, 2.2 and 3.2;
  rocketrecap.com/entries/19188 glossary "MXFP4"), with the element format,
  block size and scale rule of the published OCP MX format.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it and return its path."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.oracle_f32_to_bf16.argtypes = [f32]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = f32
        lib.oracle_e4m3_encode.argtypes = [f32]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_quant_group.argtypes = [P, i32, P, P]
        lib.oracle_quant_group.restype = f32
        lib.oracle_route.argtypes = [P, i32, i32, i32, i32, i32, P, P]
        lib.oracle_route.restype = i32
        lib.oracle_max_padded.argtypes = [i32, i32, i32, i32]
        lib.oracle_max_padded.restype = i64
        lib.oracle_max_blocks.argtypes = [i32, i32, i32, i32]
        lib.oracle_max_blocks.restype = i64
        lib.oracle_sort.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P, P]
        lib.oracle_sort.restype = i32
        lib.oracle_moe.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P,
                                   P, P, P, P, P, i32, P, P, i32, P, i64, f32, P, i64, P]
        lib.oracle_moe.restype = i32
        lib.oracle_quant_rows.argtypes = [P, i32, i32, i32, P, P]
        lib.oracle_quant_rows.restype = i32
        lib.oracle_fp4_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_fp4_decode.restype = f32
        lib.oracle_fp4_encode.argtypes = [f32]
        lib.oracle_fp4_encode.restype = ctypes.c_uint8
        lib.oracle_mx_quant_group.argtypes = [P, i32, P, P]
        lib.oracle_mx_quant_group.restype = ctypes.c_uint8
        lib.oracle_mx_quant_rows.argtypes = [P, i32, i32, P, P]
        lib.oracle_mx_quant_rows.restype = i32
        lib.oracle_moe_backward.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                            P, P, P, P, i32]
        lib.oracle_moe_backward.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    lib = _load()
    v = np.asarray(v, dtype=np.float32).ravel()
    return np.array([lib.oracle_f32_to_bf16(float(x)) for x in v], dtype=np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.oracle_e4m3_decode(int(c)) for c in codes], dtype=np.float32)


def e4m3_encode(values) -> np.ndarray:
    lib = _load()
    values = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_e4m3_encode(float(v)) for v in values], dtype=np.uint8)


def quant_group(values):
    """One shared scale: returns (codes, scale, dequantised values)."""
    lib = _load()
    v = _c(values, np.float32).ravel()
    q = np.empty(v.size, np.uint8)
    deq = np.empty(v.size, np.float32)
    s = lib.oracle_quant_group(_ptr(v), v.size, _ptr(q), _ptr(deq))
    return q, np.float32(s), deq


def fp4_decode(codes) -> np.ndarray:
    """MXFP4 E2M1 codes (low 4 bits) to fp32."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.oracle_fp4_decode(int(c)) for c in codes], dtype=np.float32)


def fp4_encode(values) -> np.ndarray:
    """fp32 to E2M1 codes (nearest, ties to the even code, saturating at +-6)."""
    lib = _load()
    values = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_fp4_encode(float(v)) for v in values], dtype=np.uint8)


def mx_quant_group(values):
    """One MXFP4 block: returns (codes one per byte, E8M0 scale code, dequantised values)."""
    lib = _load()
    v = _c(values, np.float32).ravel()
    q = np.empty(v.size, np.uint8)
    deq = np.empty(v.size, np.float32)
    c = lib.oracle_mx_quant_group(_ptr(v), v.size, _ptr(q), _ptr(deq))
    return q, int(c), deq


def mx_quant_rows(x_bf16: np.ndarray):
    """Dynamic MXFP4 quantisation of a bf16 matrix [rows, cols] (cols % 32 == 0).

    Returns (codes uint8 [rows, cols // 2], two per byte with the even column
    in the low nibble, E8M0 scales uint8 [rows, cols // 32])."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    rc = lib.oracle_mx_quant_rows(_ptr(x), rows, cols, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mx_quant_rows failed ({rc})")
    return codes, scales


def quant_rows(x_bf16: np.ndarray, group: int):
    """Dynamic e4m3 quantisation of a bf16 matrix, one scale per `group` columns.

    Returns (codes uint8 [rows, cols], scales fp32 [rows, cols // group])."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // group), np.float32)
    rc = lib.oracle_quant_rows(_ptr(x), rows, cols, group, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_quant_rows failed ({rc})")
    return codes, scales


def route(logits: np.ndarray, k: int, score: str = "softmax", renorm: bool = True):
    """Top-k routing. Returns (topk_ids int32 [T,k], topk_w fp32 [T,k])."""
    lib = _load()
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib.oracle_route(_ptr(lg), T, E, k, {"softmax": 0, "sigmoid": 1}[score], int(renorm),
                          _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return ids, w


def max_padded(T, k, E, B) -> int:
    return int(_load().oracle_max_padded(T, k, E, B))


def max_blocks(T, k, E, B) -> int:
    return int(_load().oracle_max_blocks(T, k, E, B))


def sort(topk_ids: np.ndarray, topk_w: np.ndarray, E: int, B: int) -> dict:
    """Token sort. Returns a dict of numpy arrays with the buffer names used by
    the GPU library: sorted_ids, sorted_w, sorted_expert_ids, expert_counts,
    expert_offsets, num_valid."""
    lib = _load()
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float32)
    T, k = ids.shape
    P, NB = max_padded(T, k, E, B), max_blocks(T, k, E, B)
    out = dict(sorted_ids=np.empty(P, np.int32), sorted_w=np.empty(P, np.float32),
               sorted_expert_ids=np.empty(NB, np.int32), expert_counts=np.empty(E, np.int32),
               expert_offsets=np.empty(E + 1, np.int32), num_valid=np.empty(1, np.int32))
    rc = lib.oracle_sort(_ptr(ids), _ptr(w), T, k, E, B, _ptr(out["sorted_ids"]),
                         _ptr(out["sorted_w"]), _ptr(out["sorted_expert_ids"]),
                         _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
                         _ptr(out["num_valid"]))
    if rc != 0:
        raise ValueError(f"oracle_sort failed ({rc})")
    return out


QUANT = {"bf16": 0, "fp8_token": 1, "fp8_block": 2, "mxfp4": 3}


def moe(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, w13, w2,
        w13_scale=None, w2_scale=None, quant: str = "bf16", tokens=None,
        h_exact: bool = False, threads: int = 0, h_flip=None, tie_band: float = 0.0):
    """The MoE layer output for the rows listed in `tokens` (default: all).

    w13 / w2 (and the scales) are sequences indexed by expert holding numpy
    arrays (or None for experts no listed token selects): w13[e] [2f, d],
    w2[e] [d, f]; bf16 as uint16 bits, e4m3 codes as uint8 with fp32 scales,
    or (mxfp4) E2M1 codes packed two per byte [2f, d/2] / [d, f/2] with E8M0
    scales uint8 [2f, d/32] / [d, f/32].
    Element n of the h of assignment (tokens[i], j) has the flat index
    (i * k + j) * f + n. `h_flip` lists such indices whose h is rounded to the
    other of its two nearest bf16 values. With `tie_band` > 0 the call also
    reports the elements whose fp32 h lies within tie_band * |h| of a bf16
    rounding midpoint and whose other rounding would change the scale of
    their quantisation group or, under the same scale, their own code.
    Returns (y fp32 [n, d], out bf16 bits uint16 [n, d]), and with
    tie_band > 0 also the reported elements as int64 rows (i, j, n)."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float32)
    T, d = x.shape
    k = ids.shape[1]
    E = len(w13)
    q = QUANT[quant]
    f = next(a for a in w13 if a is not None).shape[0] // 2
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    keep = []

    def table(arrs, dtype):
        t = (ctypes.c_void_p * E)()
        for e, a in enumerate(arrs):
            if a is None:
                t[e] = None
            else:
                a = _c(a, dtype)
                keep.append(a)
                t[e] = a.ctypes.data
        return t

    wdt = np.uint16 if q == 0 else np.uint8
    t13, t2 = table(w13, wdt), table(w2, wdt)
    if q:
        sdt = np.uint8 if q == 3 else np.float32
        s13, s2 = table(w13_scale, sdt), table(w2_scale, sdt)
    else:
        s13 = s2 = None
    y = np.empty((tok.size, d), np.float32)
    out = np.empty((tok.size, d), np.uint16)
    flip = np.unique(np.asarray([] if h_flip is None else h_flip, np.int64))
    cap = tok.size * k * f if tie_band > 0 else 0
    ties = np.empty(max(cap, 1), np.int64)
    n_ties = np.zeros(1, np.int64)
    rc = lib.oracle_moe(T, d, f, E, k, q, int(h_exact), _ptr(x), _ptr(ids), _ptr(w), t13, s13,
                        t2, s2, _ptr(tok), tok.size, _ptr(y), _ptr(out), int(threads),
                        _ptr(flip), flip.size, float(tie_band), _ptr(ties), cap, _ptr(n_ties))
    if rc != 0:
        raise ValueError(f"oracle_moe failed ({rc})")
    if tie_band <= 0:
        return y, out
    if n_ties[0] > cap:
        raise ValueError(f"oracle_moe reported {n_ties[0]} ties, more than the {cap} it can hold")
    t = np.sort(ties[:n_ties[0]])
    return y, out, np.stack([t // (k * f), (t // f) % k, t % f], axis=1)


def moe_backward(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, w13, w2,
                 dy_bf16: np.ndarray, h_exact: bool = False, threads: int = 0):
    """Gradients of the bf16 layer for the output gradient dy (bf16 bits [T, d]).

    w13 / w2 as in :func:`moe` (bf16 bits; None for unused experts).
    Returns (dx fp32 [T, d], dw13 list of fp32 [2f, d] or None, dw2 list of
    fp32 [d, f] or None, dtopk_w fp32 [T, k])."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float32)
    dy = _c(dy_bf16, np.uint16)
    T, d = x.shape
    k = ids.shape[1]
    E = len(w13)
    f = next(a for a in w13 if a is not None).shape[0] // 2
    keep = []

    def table(arrs, dtype):
        t = (ctypes.c_void_p * E)()
        for e, a in enumerate(arrs):
            if a is None:
                t[e] = None
            else:
                a = _c(a, dtype)
                keep.append(a)
                t[e] = a.ctypes.data
        return t

    t13, t2 = table(w13, np.uint16), table(w2, np.uint16)
    dw13 = [None if a is None else np.empty((2 * f, d), np.float32) for a in w13]
    dw2 = [None if a is None else np.empty((d, f), np.float32) for a in w2]
    g13, g2 = (ctypes.c_void_p * E)(), (ctypes.c_void_p * E)()
    for e in range(E):   # outputs are written in place: point at the arrays themselves
        g13[e] = None if dw13[e] is None else dw13[e].ctypes.data
        g2[e] = None if dw2[e] is None else dw2[e].ctypes.data
    dx = np.empty((T, d), np.float32)
    dtw = np.empty((T, k), np.float32)
    rc = lib.oracle_moe_backward(T, d, f, E, k, int(h_exact), _ptr(x), _ptr(ids), _ptr(w), t13, t2,
                                 _ptr(dy), _ptr(dx), g13, g2, _ptr(dtw), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_moe_backward failed ({rc})")
    return dx, dw13, dw2, dtw


def moe_backward_sampled(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, w13, w2,
                         dy_bf16: np.ndarray, dx_tokens=(), dw13_at=(), dw2_at=(), dtw_at=(),
                         chunk: int = 2048):
    """Selected entries of the gradients :func:`moe_backward` defines, each
    computed on its own in float64 from the chain rule (for full-size layers,
    where the whole backward is out of reach on a CPU):

      g = Wg x, u = Wu x, h = bf16(silu(g) u)   (per assignment a = t k + j),
      v = Wd^T dy[t], dh = w v, dg = dh u silu'(g), du = dh silu(g),
      dx[t] = sum_j Wg^T dg + Wu^T du,  dtopk_w[a] = <v, h>,
      dW2[e][m, n] = sum over a of expert e of w dy[t, m] h[n],
      dW13[e][n, c] = sum over a of expert e of (dg or du)[n] x[t, c].

    dx_tokens: tokens whose dx rows to return; dtw_at: flat assignments;
    dw13_at / dw2_at: (e, row, column) triples. w13 / w2: per-expert bf16
    bits [2f, d] / [d, f]. Returns (dx [len, d], dw13 [len], dw2 [len],
    dtw [len]) as float64."""
    x = bf16_bits_to_f32(np.asarray(x_bf16)).astype(np.float64)
    dy = bf16_bits_to_f32(np.asarray(dy_bf16)).astype(np.float64)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_w, dtype=np.float64)
    T, d = x.shape
    k = ids.shape[1]
    f = next(a for a in w13 if a is not None).shape[0] // 2

    def f64(b):
        return bf16_bits_to_f32(np.asarray(b)).astype(np.float64)

    def silu(z):
        return z / (1.0 + np.exp(-z))

    def silu_grad(z):
        s = 1.0 / (1.0 + np.exp(-z))
        return s * (1.0 + z * (1.0 - s))

    def bf16_round(v):
        return f64(f32_to_bf16_bits(v.astype(np.float32)))

    def columns(a, ns):
        """g, u, h, v, dg, du of assignment a at the columns ns of f."""
        t, e, w = a // k, int(ids.flat[a]), float(wts.flat[a])
        ns = np.asarray(ns)
        g = f64(w13[e][ns]) @ x[t]
        u = f64(w13[e][f + ns]) @ x[t]
        h = bf16_round(silu(g) * u)
        v = dy[t] @ f64(w2[e][:, ns])
        dh = w * v
        return g, u, h, v, dh * u * silu_grad(g), dh * silu(g)

    def all_columns(a):
        parts = [columns(a, np.arange(s, min(f, s + chunk))) for s in range(0, f, chunk)]
        return [np.concatenate([p[i] for p in parts]) for i in range(6)]

    dx = np.zeros((len(dx_tokens), d))
    for i, t in enumerate(dx_tokens):
        for j in range(k):
            a = t * k + j
            e = int(ids.flat[a])
            _, _, _, _, dg, du = all_columns(a)
            for s in range(0, f, chunk):
                sl = slice(s, min(f, s + chunk))
                dx[i] += dg[sl] @ f64(w13[e][sl]) + du[sl] @ f64(w13[e][f + sl.start:f + sl.stop])
    dtw = np.zeros(len(dtw_at))
    for i, a in enumerate(dtw_at):
        _, _, h, v, _, _ = all_columns(a)
        dtw[i] = v @ h
    dw2 = np.zeros(len(dw2_at))
    for i, (e, m, n) in enumerate(dw2_at):
        for a in np.flatnonzero(ids.ravel() == e):
            _, _, h, _, _, _ = columns(a, [n])
            dw2[i] += wts.flat[a] * dy[a // k, m] * h[0]
    dw13 = np.zeros(len(dw13_at))
    for i, (e, r, c) in enumerate(dw13_at):
        n = r % f
        for a in np.flatnonzero(ids.ravel() == e):
            _, _, _, _, dg, du = columns(a, [n])
            dw13[i] += (dg[0] if r < f else du[0]) * x[a // k, c]
    return dx, dw13, dw2, dtw


def moe_backward_expert(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, e: int,
                        w13_e, w2_e, dy_bf16: np.ndarray, rows13=(), cols13=(), rows2=(), cols2=(),
                        full_asg=(), chunk: int = 2048):
    """The gradients of :func:`moe_backward` that expert e contributes, in
    float64 from the same chain rule, taken over all of e's assignments a
    (ascending) at once with matrix products (for full-size layers):

      g = x Wg^T, u = x Wu^T, h = bf16(silu(g) u), v = dy Wd, dh = w v,
      dg = dh u silu'(g), du = dh silu(g)           (one row per assignment),
      dW13[e][r, c] = sum_a (dg if r < f else du)[a, r mod f] x[t_a, c],
      dW2[e][m, n] = sum_a w_a dy[t_a, m] h[a, n],

    and, for the assignments listed in full_asg (all of expert e), the
    routing-weight gradient <v, h> over all f and the assignment's share
    Wg^T dg + Wu^T du of dx[t_a].

    rows13 / cols13 (rows of [2f], columns of [d]) and rows2 / cols2 (rows
    of [d], columns of [f]) select the weight-gradient blocks. w13_e / w2_e:
    expert e's bf16 bits [2f, d] / [d, f]. Returns (dW13 block, dW2 block,
    {a: dtopk_w[a]}, {a: dx share [d]})."""
    x = bf16_bits_to_f32(np.asarray(x_bf16)).astype(np.float64)
    dy = bf16_bits_to_f32(np.asarray(dy_bf16)).astype(np.float64)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_w, dtype=np.float64)
    k = ids.shape[1]
    f = np.asarray(w13_e).shape[0] // 2
    asg = np.flatnonzero(ids.ravel() == e)
    tok = asg // k
    wa = wts.ravel()[asg]

    def f64(b):
        return bf16_bits_to_f32(np.asarray(b)).astype(np.float64)

    def silu(z):
        return z / (1.0 + np.exp(-z))

    def silu_grad(z):
        s = 1.0 / (1.0 + np.exp(-z))
        return s * (1.0 + z * (1.0 - s))

    def bf16_round(v):
        return f64(f32_to_bf16_bits(v.astype(np.float32))).reshape(v.shape)

    def at_columns(sel, ns):
        """g, u, h, v, dg, du of the assignments asg[sel] at the columns ns of f."""
        ns = np.asarray(ns, dtype=np.int64)
        xs = x[tok[sel]]
        g = xs @ f64(np.asarray(w13_e)[ns]).T
        u = xs @ f64(np.asarray(w13_e)[f + ns]).T
        h = bf16_round(silu(g) * u)
        v = dy[tok[sel]] @ f64(np.asarray(w2_e)[:, ns])
        dh = wa[sel, None] * v
        return g, u, h, v, dh * u * silu_grad(g), dh * silu(g)

    every = np.arange(asg.size)
    rows13, cols13 = np.asarray(rows13, np.int64), np.asarray(cols13, np.int64)
    dw13 = np.zeros((rows13.size, cols13.size))
    if rows13.size and cols13.size and asg.size:
        _, _, _, _, dg, du = at_columns(every, rows13 % f)
        lhs = np.where((rows13 < f)[None, :], dg, du)          # [assignments, rows13]
        dw13 = lhs.T @ x[tok][:, cols13]
    rows2, cols2 = np.asarray(rows2, np.int64), np.asarray(cols2, np.int64)
    dw2 = np.zeros((rows2.size, cols2.size))
    if rows2.size and cols2.size and asg.size:
        _, _, h, _, _, _ = at_columns(every, cols2)
        dw2 = (wa[:, None] * dy[tok][:, rows2]).T @ h
    dtw, dx = {}, {}
    sel = np.array([int(np.flatnonzero(asg == a)[0]) for a in full_asg], dtype=np.int64)
    if sel.size:
        d = x.shape[1]
        vh = np.zeros(sel.size)
        share = np.zeros((sel.size, d))
        for s0 in range(0, f, chunk):
            ns = np.arange(s0, min(f, s0 + chunk))
            _, _, h, v, dg, du = at_columns(sel, ns)
            vh += np.sum(v * h, axis=1)
            share += dg @ f64(np.asarray(w13_e)[ns]) + du @ f64(np.asarray(w13_e)[f + ns])
        for i, a in enumerate(full_asg):
            dtw[int(a)] = float(vh[i])
            dx[int(a)] = share[i]
    return dw13, dw2, dtw, dx
