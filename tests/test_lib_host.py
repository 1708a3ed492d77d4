"""Host-side checks of libmoe that need no GPU: the library loads, exports
every entry point include/moe.h declares, and validates arguments on the host
before any HIP call."""
import ctypes
import os
import re

import pytest

import moe_grouped_gemm_sorting_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.library_path()):
        pytest.skip("libmoe.so not built")
    return moe.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ["moe_topk", "moe_sort", "moe_gemm1_swiglu", "moe_gemm2_combine", "fused_moe",
                     "moe_quant_act", "moe_sort_max_padded", "moe_sort_max_blocks",
                     "moe_last_error", "moe_status_string"]:
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_sizes_follow_the_padding_formula(lib):
    for T, k, E, B in [(16, 2, 4, 32), (32, 2, 8, 32), (4096, 2, 8, 128), (128, 8, 256, 16),
                       (0, 1, 1, 16), (1, 1, 1, 1)]:
        assert moe.moe_sort_max_padded(T, k, E, B) == oracle.max_padded(T, k, E, B)
        assert moe.moe_sort_max_blocks(T, k, E, B) == oracle.max_blocks(T, k, E, B)
    assert lib.moe_sort_max_padded(-1, 1, 1, 1) == -1
    assert lib.moe_sort_max_padded(1, 3, 2, 1) == -1   # k > E


def _err(lib):
    return lib.moe_last_error().decode()


def test_validation_before_any_device_call(lib):
    S = None
    # routing: k > E, bad score, null pointers
    assert lib.moe_topk(None, 4, 4, 5, 0, 1, None, None, S) == 1
    assert lib.moe_topk(None, 4, 4, 2, 7, 1, None, None, S) == 1
    assert lib.moe_topk(None, 4, 4, 2, 0, 1, None, None, S) == 1 and "null" in _err(lib)
    assert lib.moe_topk(None, 4, 2000, 2, 0, 1, None, None, S) == 1
    # sort: bad B, null pointers
    assert lib.moe_sort(None, None, 4, 2, 4, 0, None, None, None, None, None, None, S) == 1
    assert lib.moe_sort(None, None, 4, 2, 4, 16, None, None, None, None, None, None, S) == 1
    # quant: unsupported group
    assert lib.moe_quant_act(None, 2, 256, 64, None, None, S) == 2
    assert lib.moe_quant_act(None, 2, 200, 200, None, None, S) == 2
    # gemm1: d not a multiple of 128, bad B, bad quant, null pointers, small workspace
    args = [None] * 8 + [None, 0, S]
    assert lib.moe_gemm1_swiglu(4, 100, 256, 4, 2, 16, 0, *args) == 2
    assert lib.moe_gemm1_swiglu(4, 128, 256, 4, 2, 48, 0, *args) == 1
    assert lib.moe_gemm1_swiglu(4, 128, 256, 4, 2, 16, 5, *args) == 1
    assert lib.moe_gemm1_swiglu(4, 128, 256, 4, 2, 16, 0, *args) == 1
    fake = ctypes.c_void_p(16)
    assert lib.moe_gemm1_swiglu(4, 128, 256, 4, 2, 16, 1, fake, fake, None, fake, fake, fake, fake,
                                fake, None, 0, S) == 1          # fp8 without scales
    n = lib.moe_gemm1_workspace_bytes(4, 128, 256, 4, 2, 16, 1)
    assert n > 0
    assert lib.moe_gemm1_swiglu(4, 128, 256, 4, 2, 16, 1, fake, fake, fake, fake, fake, fake, fake,
                                fake, fake, n - 1, S) == 3
    # gemm2 / fused
    assert lib.moe_gemm2_combine(4, 128, 256, 4, 2, 16, 0, 0, *([None] * 9), None, 0, S) == 1
    assert lib.fused_moe(4, 128, 256, 4, 2, 0, 0, 1, *([None] * 8), 16, 2, 0, None, None, 0, S) == 1
    n = lib.fused_moe_workspace_bytes(4, 128, 256, 4, 2, 0, 16, 2)
    assert lib.fused_moe(4, 128, 256, 4, 2, 0, 0, 1, fake, None, None, fake, fake, None, fake, None,
                         16, 2, 0, fake, fake, n - 1, S) == 3
    assert lib.fused_moe_workspace_bytes(4, 128, 256, 4, 2, 0, 16, 3) == 0
    assert lib.moe_status_string(3) == b"workspace too small"
    # MXFP4: d and f must be multiples of 256, the quantiser's columns of 32
    assert lib.moe_gemm1_swiglu(4, 128, 256, 4, 2, 16, 3, *args) == 2
    assert lib.moe_gemm1_swiglu(4, 256, 384, 4, 2, 16, 3, *args) == 2
    assert lib.moe_gemm1_swiglu(4, 256, 256, 4, 2, 16, 3, fake, fake, None, fake, fake, fake, fake,
                                fake, None, 0, S) == 1          # MXFP4 without scales
    assert lib.moe_quant_act_mx(None, 2, 48, None, None, S) == 1
    assert lib.moe_quant_act_mx(None, 2, 64, None, None, S) == 1 and "null" in _err(lib)
    assert lib.fused_moe_workspace_bytes(4, 256, 256, 4, 2, 3, 64, 2) > 0   # size query only
    # backward: tiled blocks need d, f multiples of 256; null pointers; small workspace
    assert lib.moe_backward_workspace_bytes(4, 128, 256, 4, 2, 64) == 0
    assert lib.moe_backward_workspace_bytes(4, 256, 256, 4, 2, 64) > 0
    assert lib.moe_backward_workspace_bytes(4, 256, 256, 4, 2, 48) == 0
    assert lib.moe_backward_workspace_bytes(4, 100, 256, 4, 2, 16) == 0
    n = lib.moe_backward_workspace_bytes(4, 128, 256, 4, 2, 0)
    assert n > 0 and n == lib.moe_backward_workspace_bytes(4, 128, 256, 4, 2, 16)   # 2 rows per expert
    bw = [None] * 10
    assert lib.moe_backward(4, 128, 256, 4, 2, 64, *bw, None, 0, S) == 2
    assert lib.moe_backward(4, 128, 256, 4, 2, 32, *bw, None, 0, S) == 1 and "null" in _err(lib)
    assert lib.moe_backward(4, 128, 256, 4, 2, 0, *([fake] * 10), fake, n - 1, S) == 3


def test_workspace_queries_grow_with_the_problem(lib):
    a = lib.fused_moe_workspace_bytes(32, 4096, 14336, 8, 2, 0, 32, 2)
    b = lib.fused_moe_workspace_bytes(4096, 4096, 14336, 8, 2, 0, 32, 2)
    assert 0 < a < b
    assert lib.moe_gemm2_workspace_bytes(32, 4096, 14336, 8, 2, 32, 0) >= 32 * 4096 * 4
    assert lib.moe_gemm1_workspace_bytes(32, 4096, 14336, 8, 2, 32, 0) == 0


@pytest.fixture
def no_table(lib):
    """The built-in choice: no tuned table while the test runs (the default one is reloaded)."""
    moe.moe_load_config_table(None)
    yield
    if os.path.exists(moe.DEFAULT_CONFIG_TABLE):
        moe.moe_load_config_table(moe.DEFAULT_CONFIG_TABLE)


def test_select_config_is_host_only_and_valid(lib, no_table):
    for shape in [(16, 128, 256, 4, 2, "bf16"), (32, 4096, 14336, 8, 2, "bf16"),
                  (4096, 4096, 14336, 8, 2, "bf16"), (512, 4096, 14336, 8, 2, "fp8_token"),
                  (128, 7168, 2048, 256, 8, "fp8_block"), (1, 4096, 14336, 8, 2, "bf16"),
                  (32, 4096, 14336, 8, 2, "mxfp4"), (4096, 4096, 14336, 8, 2, "mxfp4"),
                  (4096, 4096, 14592, 8, 2, "mxfp4")]:
        B, stage, ks = moe.moe_select_config(*shape, cu_count=256)
        assert B in (16, 32, 64, 128, 256) and stage in (1, 2) and ks >= 1
    # MXFP4: the streaming kernels at few rows per expert or when d or f is not
    # a multiple of 512 (the tiled kernels' pairs of K steps), else 256-row tiles
    assert moe.moe_select_config(32, 4096, 14336, 8, 2, "mxfp4", cu_count=256)[0] == 32
    assert moe.moe_select_config(4096, 4096, 14336, 8, 2, "mxfp4", cu_count=256)[0] == 256
    assert moe.moe_select_config(4096, 4096, 14592, 8, 2, "mxfp4", cu_count=256)[0] == 32
    with pytest.raises(moe.MoeError):
        moe.moe_select_config(4, 100, 256, 4, 2, "bf16", cu_count=256)


def test_config_table_fuzzy_match_on_T(lib, no_table, tmp_path):
    """Rows of the same (cu, d, f, E, k, quant): the smallest T at or above the call's T, else the
    largest; other shapes and CU counts keep the built-in rule."""
    path = tmp_path / "t.csv"
    path.write_text("# a comment\ncu,T,d,f,E,k,quant,B,stage,ksplit,us\n"
                    "256,8,4096,14336,8,2,bf16,16,1,1,1.0\n"
                    "256,64,4096,14336,8,2,bf16,32,2,3,2.0\n"
                    "256,1024,4096,14336,8,2,0,128,2,1,3.0\n"
                    "256,512,4096,14336,8,2,mxfp4,64,2,2\n")
    assert moe.moe_load_config_table(str(path)) == 4
    sel = lambda T, q="bf16", cu=256: moe.moe_select_config(T, 4096, 14336, 8, 2, q, cu_count=cu)
    assert sel(1) == (16, 1, 1) and sel(8) == (16, 1, 1)
    assert sel(9) == (32, 2, 3) and sel(64) == (32, 2, 3)
    assert sel(65) == (128, 2, 1) and sel(1024) == (128, 2, 1)
    assert sel(5000) == (128, 2, 1)                 # above every row: the largest T
    assert sel(3, "mxfp4") == (64, 2, 2)
    # another CU count or another shape: the built-in rule
    moe.moe_load_config_table(None)
    b304 = sel(64, cu=304)
    b_k4 = moe.moe_select_config(64, 4096, 14336, 8, 4, cu_count=256)
    moe.moe_load_config_table(str(path))
    assert sel(64, cu=304) == b304
    assert moe.moe_select_config(64, 4096, 14336, 8, 4, cu_count=256) == b_k4


def test_config_table_rejects_bad_rows_and_keeps_the_old_table(lib, no_table, tmp_path):
    good = tmp_path / "good.csv"
    good.write_text("256,32,4096,14336,8,2,bf16,16,2,4\n")
    assert moe.moe_load_config_table(str(good)) == 1
    for bad, status in [("256,32,4096,14336,8,2,bf16,48,2,4\n", "MOE_ERR_INVALID_ARG"),     # B
                        ("256,32,4096,14336,8,2,fp16,16,2,4\n", "MOE_ERR_INVALID_ARG"),     # quant
                        ("256,32,4096,14336,8,2,bf16,16,3,4\n", "MOE_ERR_INVALID_ARG"),     # stage
                        ("256,32,4096,14336,8,2,bf16,16\n", "MOE_ERR_INVALID_ARG"),         # short row
                        ("256,32,4096,14336,8,2,fp8_token,16,1,1\n", "MOE_ERR_UNSUPPORTED"),  # 1-stage fp8
                        ("256,32,4096,14336,8,2,fp8_block,64,2,1\n", "MOE_ERR_UNSUPPORTED"),  # tiled 1x128
                        ("256,32,4096,14592,8,2,mxfp4,64,2,1\n", "MOE_ERR_UNSUPPORTED")]:   # f % 512
        path = tmp_path / "bad.csv"
        path.write_text("256,64,4096,14336,8,2,bf16,32,2,2\n" + bad)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_load_config_table(str(path))
        assert status in str(ei.value) and "bad.csv:2" in str(ei.value)
        assert moe.moe_select_config(32, 4096, 14336, 8, 2, cu_count=256) == (16, 2, 4)
    with pytest.raises(moe.MoeError):
        moe.moe_load_config_table(str(tmp_path / "missing.csv"))


def test_packaged_config_table_loads(lib):
    """The committed table (if present) parses and names only runnable configurations."""
    if not os.path.exists(moe.DEFAULT_CONFIG_TABLE):
        pytest.skip("no packaged table")
    assert moe.moe_load_config_table(moe.DEFAULT_CONFIG_TABLE) > 0


def test_binding_shape_checks(lib):
    """The binding's cross-checks of tensor shapes (host-side, CPU tensors):
    a mismatched weight, scale, h or sort buffer raises before any library
    call could read past it."""
    import torch
    E, d, f, T, k, B = 4, 256, 512, 10, 2, 32
    assert moe._weight_scale_shapes("fp8_token", E, d, f) == ((E, 2 * f), (E, d))
    assert moe._weight_scale_shapes("fp8_block", E, d, f) == ((E, 8, 2), (E, 2, 4))
    assert moe._weight_scale_shapes("mxfp4", E, d, f) == ((E, 2 * f, 8), (E, d, 16))
    assert moe._weight_scale_shapes("bf16", E, d, f) == (None, None)
    P = moe.moe_sort_max_padded(T, k, E, B)
    assert moe._h_shapes("bf16", P, f) == ((P, f), None)
    assert moe._h_shapes("fp8_token", P, f) == ((P, f), (P,))
    assert moe._h_shapes("mxfp4", P, f) == ((P, f // 2), (P, f // 32))
    moe._shape(torch.empty(E, 2 * f, d), "w13", (E, 2 * f, d))
    moe._shape(None, "unused", (1,))
    with pytest.raises(ValueError, match="w13 has shape"):
        moe._shape(torch.empty(E, 2 * f, d // 2), "w13", (E, 2 * f, d))
    NB = moe.moe_sort_max_blocks(T, k, E, B)
    good = dict(sorted_ids=torch.empty(P, dtype=torch.int32), sorted_w=torch.empty(P),
                sorted_expert_ids=torch.empty(NB, dtype=torch.int32),
                num_valid=torch.empty(1, dtype=torch.int32))
    assert moe._check_sort(good, T, k, E, B) == P
    with pytest.raises(ValueError, match="sorted_ids"):   # a sort made with another block size
        moe._check_sort(good, T, k, E, 64)
    with pytest.raises(ValueError, match="sorted_expert_ids"):
        moe._check_sort(dict(good, sorted_expert_ids=torch.empty(NB - 1, dtype=torch.int32)), T, k, E, B)
    with pytest.raises(ValueError, match="bad sort shape"):
        moe._check_sort(good, T, 5, 4, B)
