"""Python binding of libmoe, the gfx950 fused Mixture-of-Experts library.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/moe.h``. PyTorch supplies device
memory (``torch.empty`` on the GPU) and the current stream. The functions
carry the ABI's names; importing works without a GPU, and any call fails
loudly if ``libmoe.so`` has not been built.
"""
from __future__ import annotations

import ctypes
import os
import warnings

import numpy as np
import torch

__all__ = [
    "MoeError", "QUANT", "SCORE", "load_library", "library_path",
    "moe_sort_max_padded", "moe_sort_max_blocks", "moe_topk", "moe_sort", "moe_quant_act",
    "moe_quant_act_mx",
    "moe_gemm1_workspace_bytes", "moe_gemm1_swiglu", "moe_gemm2_workspace_bytes",
    "moe_gemm2_combine", "fused_moe_workspace_bytes", "fused_moe", "moe_select_config",
    "moe_load_config_table", "DEFAULT_CONFIG_TABLE", "moe_backward_workspace_bytes", "moe_backward",
    "fused_moe_noalloc", "NOALLOC_SCRATCH_BYTES",
]

# The size of fused_moe_noalloc's static workspace (MOE_NOALLOC_SCRATCH_BYTES
# in include/moe.h).
NOALLOC_SCRATCH_BYTES = 64 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmoe.so")
# Tuned configurations measured on MI355X (written by ``tune.py``). Loaded with
# the library unless MOE_CONFIG_TABLE names another file ("" loads none).
DEFAULT_CONFIG_TABLE = os.path.join(_PKG, "configs", "mi355x.csv")
_lib = None

QUANT = {"bf16": 0, "fp8_token": 1, "fp8_block": 2, "mxfp4": 3}
SCORE = {"softmax": 0, "sigmoid": 1}
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmoe.so (built by ``moe_grouped_gemm_sorting_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m moe_grouped_gemm_sorting_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_sort_max_padded": (i64, [i32, i32, i32, i32]),
        "moe_sort_max_blocks": (i64, [i32, i32, i32, i32]),
        "moe_topk": (i32, [P, i32, i32, i32, i32, i32, P, P, P]),
        "moe_sort": (i32, [P, P, i32, i32, i32, i32, P, P, P, P, P, P, P]),
        "moe_quant_act": (i32, [P, i32, i32, i32, P, P, P]),
        "moe_quant_act_mx": (i32, [P, i32, i32, P, P, P]),
        "moe_gemm1_workspace_bytes": (sz, [i32] * 7),
        "moe_gemm1_swiglu": (i32, [i32] * 7 + [P] * 8 + [P, sz, P]),
        "moe_gemm2_workspace_bytes": (sz, [i32] * 7),
        "moe_gemm2_combine": (i32, [i32] * 8 + [P] * 9 + [P, sz, P]),
        "fused_moe_workspace_bytes": (sz, [i32] * 8),
        "fused_moe": (i32, [i32] * 8 + [P] * 8 + [i32, i32, i32, P, P, sz, P]),
        "fused_moe_noalloc": (i32, [i32] * 8 + [P] * 8 + [i32, i32, i32, P, P]),
        "moe_select_config": (i32, [i32] * 7 + [P, P, P]),
        "moe_load_config_table": (i32, [ctypes.c_char_p, P]),
        "moe_backward_workspace_bytes": (sz, [i32] * 6),
        "moe_backward": (i32, [i32] * 6 + [P] * 10 + [P, sz, P]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    table = os.environ.get("MOE_CONFIG_TABLE")
    if table:
        moe_load_config_table(table)
    elif table is None and os.path.exists(DEFAULT_CONFIG_TABLE):
        try:
            moe_load_config_table(DEFAULT_CONFIG_TABLE)
        except MoeError as e:   # the built-in rule still works
            warnings.warn(f"tuned-config table not loaded: {e}")
    return lib


# ------------------------------------------------------------------ helpers
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(rc: int):
    if rc != 0:
        msg = load_library().moe_last_error().decode(errors="replace")
        raise MoeError(rc, msg)


def _need(t, name, dtypes, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _shape(t, name, shape):
    """Raise unless tensor t (if given) has exactly `shape`."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _weight_scale_shapes(quant, E, d, f):
    """Expected shapes of (w13_scale, w2_scale) for a quant type (None for bf16)."""
    if quant == "fp8_token":
        return (E, 2 * f), (E, d)
    if quant == "fp8_block":
        return (E, 2 * f // 128, d // 128), (E, d // 128, f // 128)
    if quant == "mxfp4":
        return (E, 2 * f, d // 32), (E, d, f // 32)
    return None, None


def _h_shapes(quant, P, f):
    """Shapes of (h, h_scale) in the format moe_gemm1_swiglu writes."""
    if quant == "bf16":
        return (P, f), None
    if quant == "fp8_token":
        return (P, f), (P,)
    if quant == "fp8_block":
        return (P, f), (P, f // 128)
    return (P, f // 2), (P, f // 32)


def _check_sort(sort, T, k, E, B):
    """The sort buffers must have the sizes the library assumes for (T, k, E, B)."""
    P, NB = moe_sort_max_padded(T, k, E, B), moe_sort_max_blocks(T, k, E, B)
    if P < 0:
        raise ValueError(f"bad sort shape T={T} k={k} E={E} B={B}")
    _shape(sort["sorted_ids"], "sorted_ids", (P,))
    _shape(sort["sorted_w"], "sorted_w", (P,))
    _shape(sort["sorted_expert_ids"], "sorted_expert_ids", (NB,))
    _shape(sort["num_valid"], "num_valid", (1,))
    return P


_W8 = (torch.uint8, torch.float8_e4m3fn)


def _wdtypes(quant):
    if quant == "mxfp4":
        return (torch.uint8,)
    return (torch.bfloat16,) if quant == "bf16" else _W8


def _sdtypes(quant):
    """Scale dtype: fp32 for the e4m3 types, E8M0 bytes for MXFP4."""
    return (torch.uint8,) if quant == "mxfp4" else (torch.float32,)


def _pk(quant):
    """Elements per stored byte of weights, activations codes and h."""
    return 2 if quant == "mxfp4" else 1


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, need {nbytes}")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- ABI
def moe_sort_max_padded(T: int, k: int, E: int, B: int) -> int:
    return int(load_library().moe_sort_max_padded(T, k, E, B))


def moe_sort_max_blocks(T: int, k: int, E: int, B: int) -> int:
    return int(load_library().moe_sort_max_blocks(T, k, E, B))


def moe_topk(logits: torch.Tensor, k: int, score: str = "softmax", renorm: bool = True):
    """Top-k routing of fp32 logits [T, E]; returns (topk_ids int32, topk_w fp32), [T, k]."""
    lib = load_library()
    _need(logits, "logits", (torch.float32,))
    if logits.dim() != 2:
        raise ValueError(f"logits must be [T, E], got shape {tuple(logits.shape)}")
    T, E = logits.shape
    ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _check(lib.moe_topk(_ptr(logits), T, E, k, SCORE[score], int(renorm), _ptr(ids), _ptr(w),
                        _stream(logits)))
    return ids, w


def moe_sort(topk_ids: torch.Tensor, topk_w: torch.Tensor, E: int, B: int) -> dict:
    """Stable block-padded sort; returns sorted_ids, sorted_w, sorted_expert_ids,
    expert_counts, expert_offsets, num_valid (GPU tensors)."""
    lib = load_library()
    _need(topk_ids, "topk_ids", (torch.int32,))
    _need(topk_w, "topk_w", (torch.float32,), topk_ids.device)
    if topk_ids.dim() != 2:
        raise ValueError(f"topk_ids must be [T, k], got shape {tuple(topk_ids.shape)}")
    _shape(topk_w, "topk_w", topk_ids.shape)
    T, k = topk_ids.shape
    P, NB = moe_sort_max_padded(T, k, E, B), moe_sort_max_blocks(T, k, E, B)
    if P < 0:
        raise ValueError(f"bad sort shape T={T} k={k} E={E} B={B}")
    dev = topk_ids.device
    out = dict(sorted_ids=torch.empty(P, dtype=torch.int32, device=dev),
               sorted_w=torch.empty(P, dtype=torch.float32, device=dev),
               sorted_expert_ids=torch.empty(NB, dtype=torch.int32, device=dev),
               expert_counts=torch.empty(E, dtype=torch.int32, device=dev),
               expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               num_valid=torch.empty(1, dtype=torch.int32, device=dev))
    _check(lib.moe_sort(_ptr(topk_ids), _ptr(topk_w), T, k, E, B, _ptr(out["sorted_ids"]),
                        _ptr(out["sorted_w"]), _ptr(out["sorted_expert_ids"]),
                        _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
                        _ptr(out["num_valid"]), _stream(topk_ids)))
    return out


def moe_quant_act(x: torch.Tensor, group: int):
    """Dynamic e4m3 quantisation of bf16 x [rows, cols]; returns (codes uint8, scales fp32)."""
    lib = load_library()
    _need(x, "x", (torch.bfloat16,))
    if x.dim() != 2 or group < 1 or x.shape[1] % group:
        raise ValueError(f"x must be [rows, cols] with cols a multiple of group={group}")
    rows, cols = x.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, cols // group, dtype=torch.float32, device=x.device)
    _check(lib.moe_quant_act(_ptr(x), rows, cols, group, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def moe_quant_act_mx(x: torch.Tensor):
    """Dynamic MXFP4 quantisation of bf16 x [rows, cols]; returns (codes uint8
    [rows, cols/2], two per byte, E8M0 scales uint8 [rows, cols/32])."""
    lib = load_library()
    _need(x, "x", (torch.bfloat16,))
    if x.dim() != 2 or x.shape[1] % 32:
        raise ValueError(f"x must be [rows, cols] with cols a multiple of 32, got {tuple(x.shape)}")
    rows, cols = x.shape
    codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device)
    _check(lib.moe_quant_act_mx(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def moe_gemm1_workspace_bytes(T, d, f, E, k, B, quant="bf16") -> int:
    return int(load_library().moe_gemm1_workspace_bytes(T, d, f, E, k, B, QUANT[quant]))


def moe_gemm1_swiglu(x, w13, sort: dict, k: int, B: int, quant: str = "bf16", w13_scale=None,
                     workspace=None):
    """Stage 1: grouped gate/up GEMM + SwiGLU. Returns (h, h_scale) in the
    format of `quant` (bf16 [P, f]; e4m3 codes [P, f] + fp32 scales; or MXFP4
    codes [P, f/2] + E8M0 scales [P, f/32])."""
    lib = load_library()
    _need(x, "x", (torch.bfloat16,))
    _need(w13, "w13", _wdtypes(quant), x.device)
    if x.dim() != 2 or w13.dim() != 3:
        raise ValueError("x must be [T, d] and w13 [E, 2f, d]")
    E, f2, dk = w13.shape
    f = f2 // 2
    T, d = x.shape
    _shape(w13, "w13", (E, 2 * f, d // _pk(quant)))
    P = _check_sort(sort, T, k, E, B)
    _shape(w13_scale, "w13_scale", _weight_scale_shapes(quant, E, d, f)[0])
    dev = x.device
    q = QUANT[quant]
    if q == 0:
        h = torch.empty(P, f, dtype=torch.bfloat16, device=dev)
        h_scale = None
    elif quant == "mxfp4":
        _need(w13_scale, "w13_scale", _sdtypes(quant), dev)
        h = torch.empty(P, f // 2, dtype=torch.uint8, device=dev)
        h_scale = torch.empty(P, f // 32, dtype=torch.uint8, device=dev)
    else:
        _need(w13_scale, "w13_scale", (torch.float32,), dev)
        h = torch.empty(P, f, dtype=torch.uint8, device=dev)
        h_scale = torch.empty(P if q == 1 else P * (f // 128), dtype=torch.float32, device=dev)
    nbytes = moe_gemm1_workspace_bytes(T, d, f, E, k, B, quant)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.moe_gemm1_swiglu(T, d, f, E, k, B, q, _ptr(x), _ptr(w13), _ptr(w13_scale),
                                _ptr(sort["sorted_ids"]), _ptr(sort["sorted_expert_ids"]),
                                _ptr(sort["num_valid"]), _ptr(h), _ptr(h_scale), _ptr(ws), nbytes,
                                _stream(x)))
    if h_scale is not None and q == 2:
        h_scale = h_scale.view(P, f // 128)
    return h, h_scale


def moe_gemm2_workspace_bytes(T, d, f, E, k, B, quant="bf16") -> int:
    return int(load_library().moe_gemm2_workspace_bytes(T, d, f, E, k, B, QUANT[quant]))


def moe_gemm2_combine(h, h_scale, w2, sort: dict, T: int, k: int, B: int, quant: str = "bf16",
                      w2_scale=None, ksplit: int = 0, out=None, workspace=None):
    """Stage 2: grouped down GEMM + routing-weighted combine; returns out bf16 [T, d]."""
    lib = load_library()
    _need(w2, "w2", _wdtypes(quant))
    if w2.dim() != 3:
        raise ValueError("w2 must be [E, d, f]")
    E, d, fk = w2.shape
    f = fk * _pk(quant)
    dev = w2.device
    q = QUANT[quant]
    _need(h, "h", (torch.bfloat16,) if q == 0 else _wdtypes(quant), dev)
    if q:
        _need(w2_scale, "w2_scale", _sdtypes(quant), dev)
        _need(h_scale, "h_scale", _sdtypes(quant), dev)
    P = _check_sort(sort, T, k, E, B)
    hs, hss = _h_shapes(quant, P, f)
    _shape(h, "h", hs)
    if h_scale is not None and hss is not None and h_scale.numel() != int(np.prod(hss)):
        raise ValueError(f"h_scale has {h_scale.numel()} elements, expected {int(np.prod(hss))}")
    _shape(w2_scale, "w2_scale", _weight_scale_shapes(quant, E, d, f)[1])
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", (torch.bfloat16,), dev)
        _shape(out, "out", (T, d))
    nbytes = moe_gemm2_workspace_bytes(T, d, f, E, k, B, quant)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.moe_gemm2_combine(T, d, f, E, k, B, q, ksplit, _ptr(h), _ptr(h_scale), _ptr(w2),
                                 _ptr(w2_scale), _ptr(sort["sorted_ids"]), _ptr(sort["sorted_w"]),
                                 _ptr(sort["sorted_expert_ids"]), _ptr(sort["num_valid"]),
                                 _ptr(out), _ptr(ws), nbytes, _stream(w2)))
    return out


def fused_moe_workspace_bytes(T, d, f, E, k, quant="bf16", B=0, stage=0) -> int:
    return int(load_library().fused_moe_workspace_bytes(T, d, f, E, k, QUANT[quant], B, stage))


def fused_moe(x, w13, w2, k: int, logits=None, topk_ids=None, topk_w=None, quant: str = "bf16",
              w13_scale=None, w2_scale=None, score: str = "softmax", renorm: bool = True,
              B: int = 0, stage: int = 0, ksplit: int = 0, out=None, workspace=None):
    """The whole layer; returns out bf16 [T, d]. Pass `logits` [T, E] fp32, or
    precomputed `topk_ids` / `topk_w`."""
    lib = load_library()
    _need(x, "x", (torch.bfloat16,))
    dev = x.device
    q = QUANT[quant]
    _need(w13, "w13", _wdtypes(quant), dev)
    _need(w2, "w2", _wdtypes(quant), dev)
    if x.dim() != 2 or w13.dim() != 3:
        raise ValueError("x must be [T, d] and w13 [E, 2f, d]")
    T, d = x.shape
    E, f2, _ = w13.shape
    f = f2 // 2
    pk = _pk(quant)
    _shape(w13, "w13", (E, 2 * f, d // pk))
    _shape(w2, "w2", (E, d, f // pk))
    if logits is not None:
        _need(logits, "logits", (torch.float32,), dev)
        _shape(logits, "logits", (T, E))
    else:
        _need(topk_ids, "topk_ids", (torch.int32,), dev)
        _need(topk_w, "topk_w", (torch.float32,), dev)
        _shape(topk_ids, "topk_ids", (T, k))
        _shape(topk_w, "topk_w", (T, k))
    if q:
        _need(w13_scale, "w13_scale", _sdtypes(quant), dev)
        _need(w2_scale, "w2_scale", _sdtypes(quant), dev)
        s13, s2 = _weight_scale_shapes(quant, E, d, f)
        _shape(w13_scale, "w13_scale", s13)
        _shape(w2_scale, "w2_scale", s2)
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", (torch.bfloat16,), dev)
        _shape(out, "out", (T, d))
    nbytes = fused_moe_workspace_bytes(T, d, f, E, k, quant, B, stage)
    if nbytes == 0:
        _check(lib.fused_moe(T, d, f, E, k, q, SCORE[score], int(renorm), *([None] * 8), B, stage,
                             ksplit, None, None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.fused_moe(T, d, f, E, k, q, SCORE[score], int(renorm), _ptr(logits), _ptr(topk_ids),
                         _ptr(topk_w), _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                         _ptr(w2_scale), B, stage, ksplit, _ptr(out), _ptr(ws), nbytes, _stream(x)))
    return out


def fused_moe_noalloc(x, w13, w2, k: int, logits=None, topk_ids=None, topk_w=None,
                      quant: str = "bf16", w13_scale=None, w2_scale=None, score: str = "softmax",
                      renorm: bool = True, B: int = 0, stage: int = 0, ksplit: int = 0, out=None):
    """fused_moe on the library's static per-GPU workspace: no workspace
    argument and no device allocation inside the call (pass `out` to avoid
    the output allocation too). Returns out bf16 [T, d]."""
    lib = load_library()
    _need(x, "x", (torch.bfloat16,))
    dev = x.device
    q = QUANT[quant]
    _need(w13, "w13", _wdtypes(quant), dev)
    _need(w2, "w2", _wdtypes(quant), dev)
    if x.dim() != 2 or w13.dim() != 3:
        raise ValueError("x must be [T, d] and w13 [E, 2f, d]")
    T, d = x.shape
    E, f2, _ = w13.shape
    f = f2 // 2
    pk = _pk(quant)
    _shape(w13, "w13", (E, 2 * f, d // pk))
    _shape(w2, "w2", (E, d, f // pk))
    if logits is not None:
        _need(logits, "logits", (torch.float32,), dev)
        _shape(logits, "logits", (T, E))
    else:
        _need(topk_ids, "topk_ids", (torch.int32,), dev)
        _need(topk_w, "topk_w", (torch.float32,), dev)
        _shape(topk_ids, "topk_ids", (T, k))
        _shape(topk_w, "topk_w", (T, k))
    if q:
        _need(w13_scale, "w13_scale", _sdtypes(quant), dev)
        _need(w2_scale, "w2_scale", _sdtypes(quant), dev)
        s13, s2 = _weight_scale_shapes(quant, E, d, f)
        _shape(w13_scale, "w13_scale", s13)
        _shape(w2_scale, "w2_scale", s2)
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", (torch.bfloat16,), dev)
        _shape(out, "out", (T, d))
    _check(lib.fused_moe_noalloc(T, d, f, E, k, q, SCORE[score], int(renorm), _ptr(logits),
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(x), _ptr(w13), _ptr(w13_scale),
                                 _ptr(w2), _ptr(w2_scale), B, stage, ksplit, _ptr(out), _stream(x)))
    return out


def moe_load_config_table(path=None) -> int:
    """Load a tuned-configuration CSV (None clears the table); returns its row count."""
    lib = load_library()
    rows = ctypes.c_int()
    _check(lib.moe_load_config_table(None if path is None else os.fsencode(path), ctypes.byref(rows)))
    return rows.value


def moe_select_config(T, d, f, E, k, quant="bf16", cu_count: int = 0):
    """The library's (B, stage, ksplit) choice for a shape."""
    lib = load_library()
    B, stage, ks = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib.moe_select_config(T, d, f, E, k, QUANT[quant], cu_count, ctypes.byref(B),
                                 ctypes.byref(stage), ctypes.byref(ks)))
    return B.value, stage.value, ks.value


def moe_backward_workspace_bytes(T, d, f, E, k, B=0) -> int:
    return int(load_library().moe_backward_workspace_bytes(T, d, f, E, k, B))


def moe_backward(x, w13, w2, dy, topk_ids, topk_w, B: int = 0, workspace=None):
    """Gradients of the bf16 layer for the output gradient dy and the routing
    the forward used. Returns (dx bf16 [T, d], dw13 fp32 [E, 2f, d],
    dw2 fp32 [E, d, f], dtopk_w fp32 [T, k]). B: 16 or 32 (streaming
    kernels), 64, 128 or 256 (tiled kernels; d and f multiples of 256), or
    0 for the library's choice."""
    lib = load_library()
    dev = x.device
    _need(x, "x", (torch.bfloat16,), dev)
    _need(dy, "dy", (torch.bfloat16,), dev)
    _need(w13, "w13", (torch.bfloat16,), dev)
    _need(w2, "w2", (torch.bfloat16,), dev)
    _need(topk_ids, "topk_ids", (torch.int32,), dev)
    _need(topk_w, "topk_w", (torch.float32,), dev)
    if x.dim() != 2 or w13.dim() != 3 or topk_ids.dim() != 2:
        raise ValueError("x must be [T, d], w13 [E, 2f, d] and topk_ids [T, k]")
    T, d = x.shape
    E, f2, _ = w13.shape
    f = f2 // 2
    k = topk_ids.shape[1]
    _shape(w13, "w13", (E, 2 * f, d))
    _shape(w2, "w2", (E, d, f))
    _shape(dy, "dy", (T, d))
    _shape(topk_ids, "topk_ids", (T, k))
    _shape(topk_w, "topk_w", (T, k))
    dx = torch.empty(T, d, device=dev, dtype=torch.bfloat16)
    dw13 = torch.empty(E, 2 * f, d, device=dev, dtype=torch.float32)
    dw2 = torch.empty(E, d, f, device=dev, dtype=torch.float32)
    dtw = torch.empty(T, k, device=dev, dtype=torch.float32)
    nbytes = moe_backward_workspace_bytes(T, d, f, E, k, B)
    if nbytes == 0:
        _check(lib.moe_backward(T, d, f, E, k, B, *([None] * 10), None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.moe_backward(T, d, f, E, k, B, _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w13),
                            _ptr(w2), _ptr(dy), _ptr(dx), _ptr(dw13), _ptr(dw2), _ptr(dtw),
                            _ptr(ws), nbytes, _stream(x)))
    return dx, dw13, dw2, dtw
