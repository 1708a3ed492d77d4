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


def _run_and_check(wl, B, nan_workspace=False):
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ids, w = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    g = torch.Generator(device=DEV).manual_seed(wl.seed + 7)
    dy = torch.randn(wl.T, wl.d, generator=g, device=DEV).bfloat16()
    log(f"backward {wl.name} B={B} nan_workspace={nan_workspace}")
    work = None
    if nan_workspace:
        nbytes = moe.moe_backward_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, B)
        work = torch.full((nbytes // 4 + 1,), float("nan"), device=DEV).view(torch.uint8)
    dx, dw13, dw2, dtw = moe.moe_backward(x, ws["w13"], ws["w2"], dy, torch.from_numpy(ids).to(DEV),
                                          torch.from_numpy(w).to(DEV), B=B, workspace=work)
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
    """The tiled path with its workspace filled with NaN first: the
    weight-gradient kernel sums whole 32-row chunks of each expert's segment,
    padding rows included, so it relies on the producers writing zeros into
    the padding rows of its operands; a padding row left unwritten would
    carry NaN into dW."""
    _run_and_check(wl, B, nan_workspace=True)


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
def test_backward_full_size(name, B):
    """The Mixtral-shaped layers at full size (the decode shape on the
    streaming path with 32-row blocks and on the library's choice, the tiled
    path; the prefill shape on the tiled path) against the oracle's
    per-expert float64 backward: 16 dx rows, the routing-weight gradient of
    every assignment at decode (32 sampled ones at prefill), and in every
    expert that tokens select one whole 128 x 256 tile of dW13 and one of
    dW2 (the weight-gradient kernels' tile shape), at random tile positions."""
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
    n_asg = wl.T * wl.k
    tokens = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 14, replace=False)]))
    dtw_asg = np.arange(n_asg) if n_asg <= 256 else np.sort(rng.choice(n_asg, 32, replace=False))
    full = set((tokens[:, None] * wl.k + np.arange(wl.k)).ravel().tolist()) | set(dtw_asg.tolist())
    xb, dyb = bits(x), bits(dy)
    ref_dx = np.zeros((tokens.size, wl.d))
    ref_tw = {}
    for e in np.unique(ids):
        e = int(e)
        r13 = 128 * int(rng.integers(2 * wl.f // 128))
        c13 = 256 * int(rng.integers(wl.d // 256))
        r2 = 128 * int(rng.integers(wl.d // 128))
        c2 = 256 * int(rng.integers(wl.f // 256))
        asg = [a for a in np.flatnonzero(ids.ravel() == e).tolist() if a in full]
        log(f"  oracle, expert {e}: dW13 tile ({r13}, {c13}), dW2 tile ({r2}, {c2}), {len(asg)} whole rows")
        b13, b2, tw, share = oracle.moe_backward_expert(
            xb, ids, w, e, bits(ws["w13"][e]), bits(ws["w2"][e]), dyb,
            rows13=range(r13, r13 + 128), cols13=range(c13, c13 + 256),
            rows2=range(r2, r2 + 128), cols2=range(c2, c2 + 256), full_asg=asg)
        _check(f"dw13[{e}]", dw13[e, r13:r13 + 128, c13:c13 + 256].cpu().numpy(), b13)
        _check(f"dw2[{e}]", dw2[e, r2:r2 + 128, c2:c2 + 256].cpu().numpy(), b2)
        ref_tw.update(tw)
        for a, row in share.items():
            i = np.searchsorted(tokens, a // wl.k)
            if i < tokens.size and tokens[i] == a // wl.k:
                ref_dx[i] += row
    _check("dx", bf16_to_f64(bits(dx))[tokens], ref_dx)
    _check("dtopk_w", dtw.cpu().numpy().ravel()[dtw_asg], np.array([ref_tw[int(a)] for a in dtw_asg]))
