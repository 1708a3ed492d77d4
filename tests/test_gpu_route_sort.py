"""GPU parity of routing, sorting and activation quantisation: bit-exact
against the CPU oracle (weights of the routing within 2e-6 relative)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_sorting_amd as moe
import oracle
import workloads
from gpu_helpers import DEV, bits, log

pytestmark = pytest.mark.gpu

SORT_KEYS = ["sorted_ids", "sorted_w", "sorted_expert_ids", "expert_counts", "expert_offsets",
             "num_valid"]


def _gpu_sort(ids_np, w_np, E, B):
    ids = torch.from_numpy(ids_np).to(DEV)
    w = torch.from_numpy(w_np).to(DEV)
    s = moe.moe_sort(ids, w, E, B)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in s.items()}


def _assert_sort_equal(ids, w, E, B):
    ref = oracle.sort(ids, w, E, B)
    got = _gpu_sort(ids, w, E, B)
    for key in SORT_KEYS:
        assert np.array_equal(got[key], ref[key]), f"{key} differs (E={E} B={B} T={ids.shape[0]})"
    again = _gpu_sort(ids, w, E, B)
    for key in SORT_KEYS:
        assert np.array_equal(again[key], got[key]), f"{key} not repeatable"


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_topk_and_sort_on_workload_routings(name):
    wl = workloads.get(name)
    log(f"routing+sort parity: {name}")
    _, logits = wl.activations(DEV)
    ids, w = moe.moe_topk(logits, wl.k, wl.score)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=0)
    for B in (16, 32, 64, 128):
        _assert_sort_equal(rid, rw, wl.E, B)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 2, 2), (100, 64, 6), (77, 65, 3), (9, 300, 16),
                                   (1000, 1024, 8), (513, 129, 4), (5, 16, 16)])
def test_topk_fuzz(score, T, E, k):
    g = torch.Generator(device=DEV).manual_seed(T * 7 + E)
    logits = torch.randn(T, E, generator=g, device=DEV) * 3
    # plant exact ties: duplicate a column
    if E >= 4:
        logits[:, 3] = logits[:, 1]
    ids, w = moe.moe_topk(logits, k, score)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits.cpu().numpy(), k, score)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=0)


@pytest.mark.parametrize("seed", range(12))
def test_sort_fuzz(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([1, 2, 3, 8, 33, 64, 65, 256, 1000]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([0, 1, 5, 64, 1000, 4096, 9000]))
    B = int(rng.choice([1, 16, 32, 64, 128]))
    log(f"sort fuzz seed={seed} T={T} E={E} k={k} B={B}")
    p = 1.0 / np.arange(1, E + 1) ** (1.2 if seed % 2 else 0.0)
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]) \
        if T else np.zeros((0, k), np.int64)
    ids = ids.astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    _assert_sort_equal(ids, w, E, B)


def test_sort_edge_cases():
    # everything on one expert, experts without tokens, E = 1, k = E
    ids = np.tile(np.array([[5, 2]], np.int32), (300, 1))
    _assert_sort_equal(ids, np.ones((300, 2), np.float32), 8, 16)
    _assert_sort_equal(np.zeros((7, 1), np.int32), np.ones((7, 1), np.float32), 1, 32)
    ids = np.tile(np.arange(4, dtype=np.int32)[::-1], (10, 1)).copy()
    _assert_sort_equal(ids, np.random.default_rng(0).random((10, 4)).astype(np.float32), 4, 1)
    # the largest tested sort: T*k = 65536 assignments over 1024 experts
    rng = np.random.default_rng(1)
    ids = np.stack([rng.choice(1024, 8, replace=False) for _ in range(8192)]).astype(np.int32)
    _assert_sort_equal(ids, rng.random((8192, 8)).astype(np.float32), 1024, 128)


def test_sort_at_the_largest_accepted_size():
    """T*k = 2^24 assignments, the most the library accepts (64 workgroups,
    each counting all 16.8 M of them): every output bit-exact against the
    oracle and repeatable; one assignment more is refused before any device
    work."""
    rng = np.random.default_rng(24)
    T, k, E, B = 1 << 23, 2, 8, 256
    first = rng.integers(0, E, size=T)
    ids = np.stack([first, (first + 1 + rng.integers(0, E - 1, size=T)) % E], axis=1).astype(np.int32)
    w = rng.random((T, k), dtype=np.float32)
    log(f"sort of {T * k} assignments, E={E} B={B}")
    _assert_sort_equal(ids, w, E, B)
    over = torch.zeros(((1 << 24) + 1, 1), dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError, match="2\\^24"):
        moe.moe_sort(over, torch.ones(over.shape, dtype=torch.float32, device=DEV), E, B)


@pytest.mark.parametrize("rows,cols,group", [(1, 128, 128), (3, 256, 256), (17, 4096, 4096),
                                             (128, 7168, 128), (5, 384, 128), (64, 2048, 2048)])
def test_quant_act_bit_exact(rows, cols, group):
    g = torch.Generator(device=DEV).manual_seed(rows * cols)
    x = (torch.randn(rows, cols, generator=g, device=DEV) * 4).to(torch.bfloat16)
    x[0, :5] = 0
    if rows > 2:
        x[2] = 0  # an all-zero row takes scale 1
    codes, scales = moe.moe_quant_act(x, group)
    torch.cuda.synchronize()
    rc, rs = oracle.quant_rows(bits(x), group)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_e4m3_rounding_of_every_bf16_value():
    """Every bf16 value with |v| <= 448 through the GPU quantiser with scale 1
    (a row whose amax is 448): the codes equal the oracle's e4m3 encoding,
    including the round-half-even ties that bf16 values can hit exactly."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f32(allbits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    v = vals[keep]
    n = -(-(v.size + 1) // 128) * 128
    row = np.zeros(n, np.float32)
    row[:v.size] = v
    row[v.size] = 448.0
    x = torch.from_numpy(row).to(torch.bfloat16).view(1, n).to(DEV)
    codes, scales = moe.moe_quant_act(x, n)
    torch.cuda.synchronize()
    assert float(scales[0, 0]) == 1.0
    assert np.array_equal(codes.cpu().numpy()[0, :v.size], oracle.e4m3_encode(v))


def test_empty_batch():
    """T = 0: routing returns nothing, the sort matches the oracle (every slot
    is padding, no valid block), and the whole layer returns an empty output."""
    E, k, B = 8, 2, 32
    ids, w = moe.moe_topk(torch.empty(0, E, dtype=torch.float32, device=DEV), k)
    assert ids.shape == (0, k) and w.shape == (0, k)
    _assert_sort_equal(np.zeros((0, k), np.int32), np.zeros((0, k), np.float32), E, B)
    codes, scales = moe.moe_quant_act(torch.empty(0, 256, dtype=torch.bfloat16, device=DEV), 128)
    assert codes.shape[0] == 0 and scales.shape[0] == 0
    for quant in ("bf16", "fp8_token"):
        wl = workloads.Workload("empty", T=0, d=256, f=256, E=E, k=k, quant=quant, seed=3)
        ws = wl.weights(DEV)
        x = torch.empty(0, wl.d, dtype=torch.bfloat16, device=DEV)
        logits = torch.empty(0, E, dtype=torch.float32, device=DEV)
        out = moe.fused_moe(x, ws["w13"], ws["w2"], k, logits=logits, quant=quant,
                            w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"])
        torch.cuda.synchronize()
        assert out.shape == (0, wl.d)


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (17, 4096), (128, 7168), (5, 14336)])
def test_quant_act_mx_bit_exact(rows, cols):
    """MXFP4 (per_1x32) codes and E8M0 scales equal the oracle's, including an
    all-zero block, a block at an exact power of two, E2M1 midpoints (ties)
    and blocks with tiny (subnormal-range) or huge magnitudes."""
    g = torch.Generator(device=DEV).manual_seed(rows * cols + 1)
    x = torch.randn(rows, cols, generator=g, device=DEV) * 3
    if cols >= 96:
        x[0, 0:32] = 0                                  # all-zero block: E = -127
        x[0, 32:64] = torch.tensor([4.0] + [0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.25] * 4
                                   + [-0.75, -5.0, 6.5], device=DEV)   # ties at scale 1
        x[0, 64:96] *= 1e-38                            # subnormal-range amax
    if rows > 2:
        x[2] *= 1e30
    x = x.to(torch.bfloat16)
    codes, scales = moe.moe_quant_act_mx(x)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quant_rows(bits(x))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_act_mx_worked_blocks():
    """The hand-worked MXFP4 blocks of tests/golden/mx_worked_blocks.json
    (exact powers of two, values just below a binade, a subnormal amax, an
    all-zero block): the GPU quantiser's E8M0 scales and E2M1 codes equal
    the worked values."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_blocks.json")
    blocks = json.load(open(path))["blocks"]
    rows = []
    for b in blocks:
        if "bf16_bits" in b:
            rows.append(np.array(b["bf16_bits"], np.uint16))
        else:
            v = np.array(b["values"], np.float32)
            rows.append((v.view(np.uint32) >> 16).astype(np.uint16))   # exact: the values are bf16
    x = torch.from_numpy(np.stack(rows).view(np.int16)).to(DEV).view(torch.bfloat16)
    codes, scales = moe.moe_quant_act_mx(x)
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    for r, b in enumerate(blocks):
        assert scales[r, 0] == b["scale"], b["name"]
        want = np.array(b["codes"], np.uint8)
        got = np.empty(32, np.uint8)
        got[0::2], got[1::2] = codes[r] & 15, codes[r] >> 4
        assert np.array_equal(got, want), (b["name"], got, want)


@pytest.mark.parametrize("N,E,k,B", [(511, 8, 1, 32), (512, 8, 2, 16), (1024, 8, 2, 128), (4095, 256, 5, 16),
                                     (8192, 8, 2, 256), (32769, 64, 1, 64), (40000, 1024, 8, 32),
                                     (131072, 8, 2, 256)])
def test_multi_workgroup_sort_bit_exact(N, E, k, B):
    """Sorts large enough to run on several workgroups (one per chunk of at
    least 512 assignments, each counting all assignments to find its place):
    every output bit-exact against the oracle, chunk sizes ragged and
    round, skewed and uniform routing."""
    rng = np.random.default_rng(N + E)
    T = (N + k - 1) // k
    p = rng.zipf(1.3, size=E * 4).astype(np.float64)
    p = np.bincount(rng.integers(0, E, size=E * 4), weights=p, minlength=E)[:E]
    p = p / p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p if E > k else None) for _ in range(T)])
    w = rng.random((T, k)).astype(np.float32)
    _assert_sort_equal(ids.astype(np.int32), w, E, B)
