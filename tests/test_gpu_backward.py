"""GPU parity of the backward of the bf16 layer (moe_backward) against the
oracle's chain rule, on the same routing and output gradient.

Bar: relative error floored at the RMS of the oracle's value (as for the
forward) <= 2e-2 for dx, the weight gradients of every expert and the
routing-weight gradients."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_sorting_amd as moe
import oracle
import workloads
from gpu_helpers import DEV, bits, bf16_to_f64, log, rel_err

pytestmark = pytest.mark.gpu

SHAPES = [
    workloads.get("tiny"),
    workloads.Workload("bwd_ragged", T=37, d=256, f=384, E=5, k=2, seed=51),
    workloads.Workload("bwd_skew", T=64, d=384, f=256, E=16, k=4, score="sigmoid", logits="zipf",
                       seed=52),
    workloads.Workload("bwd_single_token", T=1, d=256, f=256, E=8, k=2, seed=53),
    # 40 rows per expert: two 32-row sort blocks each, the second partly padded
    workloads.Workload("bwd_two_blocks", T=80, d=256, f=256, E=4, k=2, seed=54),
]


def _check(name, got, ref):
    err, norm = rel_err(got, ref)
    log(f"  {name}: err={err:.3e} norm={norm:.3e}")
    assert err <= 2e-2, (name, err)


# The tiled path (sort blocks of 64, 128, 256 rows; d and f multiples of 256)
TILED_SHAPES = [
    # 128 rows per expert: the default block is 128
    workloads.Workload("bwd_tiled", T=256, d=256, f=512, E=4, k=2, seed=55),
    # Zipf-skewed routing, ragged segments, a block size larger than most segments
    workloads.Workload("bwd_tiled_skew", T=300, d=512, f=256, E=6, k=2, logits="zipf", seed=56),
]


def _run_and_check(wl, B):
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ids, w = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    g = torch.Generator(device=DEV).manual_seed(wl.seed + 7)
    dy = torch.randn(wl.T, wl.d, generator=g, device=DEV).bfloat16()
    log(f"backward {wl.name} B={B}")
    dx, dw13, dw2, dtw = moe.moe_backward(x, ws["w13"], ws["w2"], dy, torch.from_numpy(ids).to(DEV),
                                          torch.from_numpy(w).to(DEV), B=B)
    torch.cuda.synchronize()
    w13 = [bits(ws["w13"][e]) for e in range(wl.E)]
    w2 = [bits(ws["w2"][e]) for e in range(wl.E)]
    rdx, r13, r2, rtw = oracle.moe_backward(bits(x), ids, w, w13, w2, bits(dy))
    _check("dx", bf16_to_f64(bits(dx)), rdx)
    _check("dw13", dw13.cpu().numpy(), np.stack(r13))
    _check("dw2", dw2.cpu().numpy(), np.stack(r2))
    _check("dtopk_w", dtw.cpu().numpy(), rtw)
    used = set(ids.ravel().tolist())
    for e in range(wl.E):
        if e not in used:
            assert not dw13[e].any() and not dw2[e].any()


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("B", [0, 16, 32])
def test_backward_matches_the_oracle(wl, B):
    _run_and_check(wl, B)


@pytest.mark.parametrize("wl", TILED_SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("B", [0, 64, 128, 256])
def test_backward_tiled_matches_the_oracle(wl, B):
    _run_and_check(wl, B)


def test_backward_rejects_tiled_blocks_on_unsupported_shapes():
    # d = 128 is not a multiple of 256: no tiled backward
    wl = workloads.get("tiny")
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ids, w = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    with pytest.raises(moe.MoeError):
        moe.moe_backward(x, ws["w13"], ws["w2"], x, torch.from_numpy(ids).to(DEV),
                         torch.from_numpy(w).to(DEV), B=64)


@pytest.mark.parametrize("name,B", [("mixtral_decode", 32), ("mixtral_decode", 0), ("mixtral_prefill", 0)])
def test_backward_full_size_sampled(name, B):
    """The Mixtral-shaped layers at full size (the decode shape on the
    streaming path with 32-row blocks and on the library's choice, the tiled
    path; the prefill shape on the tiled path) against the oracle's per-entry
    backward on sampled entries: two dx rows, four routing-weight gradients,
    twelve entries each of dW13 (gate and up rows) and dW2 in experts that
    tokens select."""
    wl = workloads.get(name)
    log(f"full-size backward: {name} B={B} (generating inputs)")
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ids, w = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    g = torch.Generator(device=DEV).manual_seed(wl.seed + 7)
    dy = torch.randn(wl.T, wl.d, generator=g, device=DEV).bfloat16()
    dx, dw13, dw2, dtw = moe.moe_backward(x, ws["w13"], ws["w2"], dy, torch.from_numpy(ids).to(DEV),
                                          torch.from_numpy(w).to(DEV), B=B)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    used = np.unique(ids)
    tokens = [0, wl.T - 1]
    asg = rng.choice(wl.T * wl.k, 4, replace=False).tolist()
    at13 = [(int(rng.choice(used)), int(rng.integers(2 * wl.f)), int(rng.integers(wl.d))) for _ in range(12)]
    at2 = [(int(rng.choice(used)), int(rng.integers(wl.d)), int(rng.integers(wl.f))) for _ in range(12)]
    w13 = [bits(ws["w13"][e]) for e in range(wl.E)]
    w2 = [bits(ws["w2"][e]) for e in range(wl.E)]
    log("  oracle on the sampled entries")
    s_dx, s13, s2, stw = oracle.moe_backward_sampled(bits(x), ids, w, w13, w2, bits(dy), dx_tokens=tokens,
                                                     dw13_at=at13, dw2_at=at2, dtw_at=asg)
    _check("dx", bf16_to_f64(bits(dx))[tokens], s_dx)
    _check("dw13", np.array([dw13[e, r, c].item() for e, r, c in at13]), s13)
    _check("dw2", np.array([dw2[e, m, n].item() for e, m, n in at2]), s2)
    _check("dtopk_w", dtw.cpu().numpy().ravel()[asg], stw)
