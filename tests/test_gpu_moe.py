"""GPU parity of the grouped GEMMs and the fused layer against the CPU oracle.

Small shapes and the full-size workloads (run exactly as the benchmark
launches them) compare every output. Bar: relative error floored at the
output RMS <= 2e-2 (bf16) or 6e-2 (fp8 and MXFP4)."""
import time

import numpy as np
import pytest
import torch

import moe_grouped_gemm_sorting_amd as moe
import workloads
import oracle
from gpu_helpers import DEV, TOL, bits, bf16_to_f64, log, oracle_layer, rel_err

pytestmark = pytest.mark.gpu

SMALL = [
    workloads.get("tiny"),
    workloads.Workload("ragged_bf16", T=37, d=256, f=384, E=5, k=2, seed=21),
    workloads.Workload("wide_bf16", T=200, d=512, f=256, E=8, k=2, seed=22),
    workloads.Workload("skew_sigmoid", T=64, d=384, f=256, E=16, k=4, score="sigmoid",
                       logits="zipf", seed=23),
    workloads.Workload("tok_fp8", T=45, d=256, f=512, E=4, k=2, quant="fp8_token", seed=24),
    workloads.Workload("blk_fp8", T=33, d=384, f=256, E=12, k=3, quant="fp8_block",
                       score="sigmoid", logits="zipf", seed=25),
    workloads.Workload("tok_mx", T=40, d=256, f=512, E=4, k=2, quant="mxfp4", seed=41),
    workloads.Workload("mx_sigmoid", T=33, d=512, f=256, E=8, k=3, quant="mxfp4",
                       score="sigmoid", logits="zipf", seed=42),
    # MXFP4 on the tiled kernels (d, f multiples of 512): 128-row blocks, and
    # 600 rows per expert in 256-row blocks with a partly padded third block
    workloads.Workload("tiled_mx", T=300, d=512, f=1024, E=4, k=2, quant="mxfp4", seed=43),
    workloads.Workload("spill_mx", T=600, d=512, f=512, E=2, k=2, quant="mxfp4", seed=44),
    workloads.Workload("one_expert", T=20, d=128, f=128, E=1, k=1, seed=26),
    workloads.Workload("single_token", T=1, d=256, f=256, E=8, k=2, seed=27),
    workloads.Workload("tiled_bf16", T=300, d=512, f=384, E=4, k=2, seed=29),
    workloads.Workload("tiled_fp8", T=260, d=768, f=256, E=3, k=2, quant="fp8_token", seed=30),
    # 400 rows per expert: a second, partly padded 256-row block (padding row quarters skip
    # their MFMAs in the 256-row tiles)
    workloads.Workload("spill_bf16", T=400, d=512, f=384, E=2, k=2, seed=31),
    workloads.Workload("spill_fp8", T=400, d=512, f=384, E=2, k=2, quant="fp8_token", seed=32),
    # top-8: the tiled down projection's per-token combine sums eight rows
    workloads.Workload("top8_tiled", T=160, d=512, f=256, E=16, k=8, score="sigmoid", seed=34),
]


def _tiled_ok(wl):
    if wl.quant == "mxfp4":
        return wl.d % 512 == 0 and wl.f % 512 == 0
    return wl.quant != "fp8_block" and wl.d % 256 == 0


def _run_two_stage(wl, x, ids, w, ws, B, ksplit):
    s = moe.moe_sort(ids, w, wl.E, B)
    h, hs = moe.moe_gemm1_swiglu(x, ws["w13"], s, wl.k, B, wl.quant, ws["w13_scale"])
    return moe.moe_gemm2_combine(h, hs, ws["w2"], s, wl.T, wl.k, B, wl.quant, ws["w2_scale"],
                                 ksplit=ksplit)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_two_stage_small_all_outputs(wl):
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ref, rid, rw = oracle_layer(wl, x, logits, ws)
    ids = torch.from_numpy(rid).to(DEV)
    w = torch.from_numpy(rw).to(DEV)
    for B in (16, 32, 64, 128, 256):
        if B >= 64 and not _tiled_ok(wl):
            with pytest.raises(moe.MoeError):
                _run_two_stage(wl, x, ids, w, ws, B, 1)
            continue
        for ksplit in (1, 2, 3):
            log(f"two-stage {wl.name} B={B} ksplit={ksplit}")
            out = _run_two_stage(wl, x, ids, w, ws, B, ksplit)
            torch.cuda.synchronize()
            err, norm = rel_err(bf16_to_f64(bits(out)), ref)
            log(f"  err={err:.3e} norm={norm:.3e}")
            assert err <= TOL[wl.quant], (wl.name, B, ksplit, err)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_fused_small_all_outputs(wl):
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ref, _, _ = oracle_layer(wl, x, logits, ws)
    out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, quant=wl.quant,
                        w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score)
    torch.cuda.synchronize()
    err, norm = rel_err(bf16_to_f64(bits(out)), ref)
    log(f"fused {wl.name}: err={err:.3e} norm={norm:.3e}")
    assert err <= TOL[wl.quant]


def test_fused_with_given_routing_and_idle_experts():
    """Precomputed routing (logits = NULL) that leaves experts idle and piles
    every token on two experts, so some experts get many blocks."""
    wl = workloads.Workload("piled", T=150, d=256, f=256, E=8, k=2, seed=28)
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    rid = np.tile(np.array([[6, 1]], np.int32), (wl.T, 1))
    rid[::7] = [[1, 3]]
    rw = np.random.default_rng(0).dirichlet([1, 1], wl.T).astype(np.float32)
    ref, _, _ = oracle_layer(wl, x, logits, ws, ids=rid, w=rw)
    for B in (16, 32, 64, 128):
        out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, topk_ids=torch.from_numpy(rid).to(DEV),
                            topk_w=torch.from_numpy(rw).to(DEV), B=B, stage=2)
        torch.cuda.synchronize()
        err, _ = rel_err(bf16_to_f64(bits(out)), ref)
        assert err <= TOL["bf16"], (B, err)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_fused_full_size_all_tokens(name):
    """Every workload at full size, in the benchmark's launch configuration
    (the library's choice of block size, stage and K-split), against the
    oracle on every token."""
    wl = workloads.get(name)
    log(f"full-size parity: {name} (generating inputs)")
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, quant=wl.quant,
                        w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score)
    torch.cuda.synchronize()
    log(f"  oracle on all {wl.T} tokens")
    t0 = time.perf_counter()
    ref, _, _ = oracle_layer(wl, x, logits, ws)
    err, norm = rel_err(bf16_to_f64(bits(out)), ref)
    log(f"  err={err:.3e} norm={norm:.3e} (oracle {time.perf_counter() - t0:.1f} s)")
    assert err <= TOL[wl.quant]


def test_fused_at_the_largest_accepted_T():
    """The Mixtral-shaped bf16 layer at T = 73728, close to the largest T
    whose activation buffers stay below 2^31 elements with 256-row blocks
    ((T k + E B) f < 2^31: T <= 73874), against the oracle on tokens spread
    over the batch (the first and the last among them); T = 73875 is refused
    before any device work."""
    wl = workloads.get("mixtral_prefill").replace(T=73728, seed=77)
    log(f"largest-T parity: T={wl.T} (generating inputs)")
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, score=wl.score, B=256)
    torch.cuda.synchronize()
    tokens = np.unique(np.concatenate([[0, wl.T - 1],
                                       np.random.default_rng(5).integers(0, wl.T, size=30)]))
    ref, _, _ = oracle_layer(wl, x, logits, ws, tokens=tokens)
    got = bf16_to_f64(bits(out))[tokens]
    err, norm = rel_err(got, ref)
    log(f"  {len(tokens)} tokens: err={err:.3e} norm={norm:.3e}")
    assert err <= TOL["bf16"]
    del out
    x_over = torch.zeros(wl.T + 147, wl.d, dtype=torch.bfloat16, device=DEV)
    l_over = torch.zeros(wl.T + 147, wl.E, dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError, match="2\\^31"):
        moe.fused_moe(x_over, ws["w13"], ws["w2"], wl.k, logits=l_over, B=256)


def test_streaming_gemm2_on_reused_and_dirty_workspaces():
    """The streaming path with atomics into the fp32 accumulator: three fused
    calls on one workspace filled with 0xFF bytes first, and the two-stage
    entry point on such a workspace (the library clears what it adds into),
    each against the oracle, at two token counts."""
    for T in (32, 513):
        wl = workloads.Workload(f"fin{T}", T=T, d=512, f=1024, E=8, k=2, seed=90 + T)
        x, logits = wl.activations(DEV)
        ws = wl.weights(DEV)
        ref, ids, w = oracle_layer(wl, x, logits, ws)
        B = 16
        nbytes = moe.fused_moe_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, "bf16", B, 2)
        work = torch.full((nbytes,), 255, dtype=torch.uint8, device=DEV)
        for call in range(3):
            out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, B=B, stage=2, ksplit=2,
                                workspace=work)
            torch.cuda.synchronize()
            err, _ = rel_err(bf16_to_f64(bits(out)), ref)
            log(f"streaming GEMM2 T={T} call {call}: err={err:.3e}")
            assert err <= TOL["bf16"], (T, call, err)
        tid, tw = moe.moe_topk(logits, wl.k)
        srt = moe.moe_sort(tid, tw, wl.E, B)
        h, hs = moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, B)
        n2 = moe.moe_gemm2_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, B, "bf16")
        dirty = torch.full((n2,), 255, dtype=torch.uint8, device=DEV)
        out2 = moe.moe_gemm2_combine(h, hs, ws["w2"], srt, wl.T, wl.k, B, ksplit=2, workspace=dirty)
        torch.cuda.synchronize()
        err, _ = rel_err(bf16_to_f64(bits(out2)), ref)
        log(f"two-stage GEMM2 T={T} on a dirty workspace: err={err:.3e}")
        assert err <= TOL["bf16"], (T, err)


ONE_STAGE = [w for w in SMALL if w.quant == "bf16"] + [
    workloads.Workload("decode_t1", T=1, d=4096, f=14336, E=8, k=2, seed=31),
    workloads.Workload("decode_t4", T=4, d=4096, f=14336, E=8, k=2, seed=32),
]


@pytest.mark.parametrize("wl", ONE_STAGE, ids=lambda w: w.name)
def test_one_stage_all_outputs(wl):
    """The one-stage kernel (gate/up, SwiGLU and down per block and f-chunk)
    against the oracle, at both block sizes it takes."""
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ref, _, _ = oracle_layer(wl, x, logits, ws)
    for B in (16, 32):
        out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, score=wl.score, B=B,
                            stage=1)
        torch.cuda.synchronize()
        err, norm = rel_err(bf16_to_f64(bits(out)), ref)
        log(f"one-stage {wl.name} B={B}: err={err:.3e} norm={norm:.3e}")
        assert err <= TOL["bf16"], (B, err)


def test_one_stage_full_decode_shape_and_unsupported():
    wl = workloads.get("mixtral_decode")
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, B=32, stage=1)
    torch.cuda.synchronize()
    ref, _, _ = oracle_layer(wl, x, logits, ws)
    err, _ = rel_err(bf16_to_f64(bits(out)), ref)
    assert err <= TOL["bf16"]
    with pytest.raises(moe.MoeError):   # 64-row blocks are not taken by the one-stage kernel
        moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, B=64, stage=1)
    fp8 = workloads.Workload("fp8s1", T=4, d=256, f=256, E=4, k=2, quant="fp8_token", seed=33)
    xf, lf = fp8.activations(DEV)
    wf = fp8.weights(DEV)
    with pytest.raises(moe.MoeError):   # per-row h quantisation needs the whole row first
        moe.fused_moe(xf, wf["w13"], wf["w2"], fp8.k, logits=lf, quant="fp8_token",
                      w13_scale=wf["w13_scale"], w2_scale=wf["w2_scale"], B=16, stage=1)


@pytest.mark.parametrize("B", (64, 128, 256))
def test_stored_row_combine_is_repeatable(B):
    """With at most two K parts the tiled down projection stores each part's
    weighted rows and sums a token's rows in a fixed order: repeated calls
    give the same bits (the atomic K-split path only meets the tolerance)."""
    wl = workloads.get("mixtral_prefill").replace(name="rep", T=384, f=1024, seed=35)
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ids, w = moe.moe_topk(logits, wl.k, wl.score)
    srt = moe.moe_sort(ids, w, wl.E, B)
    h, hs = moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, B, wl.quant, ws["w13_scale"])
    outs = [moe.moe_gemm2_combine(h, hs, ws["w2"], srt, wl.T, wl.k, B, wl.quant, ws["w2_scale"],
                                  ksplit=1) for _ in range(3)]
    halves = [moe.moe_gemm2_combine(h, hs, ws["w2"], srt, wl.T, wl.k, B, wl.quant, ws["w2_scale"],
                                    ksplit=2) for _ in range(2)]
    split = moe.moe_gemm2_combine(h, hs, ws["w2"], srt, wl.T, wl.k, B, wl.quant, ws["w2_scale"],
                                  ksplit=4)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(bits(o), bits(outs[0]))
    # two stored K parts: repeatable too, and equal to one part up to rounding
    assert np.array_equal(bits(halves[1]), bits(halves[0]))
    err, _ = rel_err(bf16_to_f64(bits(halves[0])), bf16_to_f64(bits(outs[0])))
    assert err <= 1e-2
    err, _ = rel_err(bf16_to_f64(bits(split)), bf16_to_f64(bits(outs[0])))
    assert err <= 1e-2


@pytest.mark.parametrize("B", (32, 64, 128, 256))
def test_ids_outside_the_expert_range_add_nothing(B):
    """Assignments whose id is outside [0, E) (the caller's routing) are
    dropped by the sort; on every path, including the tiled down projection
    that stores weighted rows and sums them per token, they add nothing: the
    output equals the oracle's with those assignments given weight 0. The
    workspace starts out filled with NaN, so a row the combine read without
    GEMM2 having written it would show."""
    wl = workloads.Workload("bad_ids", T=300, d=512, f=512, E=4, k=2, seed=36)
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ids, w = oracle.route(logits.cpu().numpy(), wl.k, wl.score)
    bad = ids.copy()
    bad[::5, 1] = -1          # some second choices dropped
    bad[3::11, 0] = wl.E      # some first choices out of range
    bad[7] = [-3, wl.E + 2]   # a token with no valid assignment: zeros
    keep = (bad >= 0) & (bad < wl.E)
    ref, _, _ = oracle_layer(wl, x, logits, ws, ids=np.where(keep, bad, 0).astype(np.int32),
                             w=np.where(keep, w, 0).astype(np.float32))
    nbytes = moe.fused_moe_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, wl.quant, B, 2)
    work = torch.full((nbytes // 4 + 1,), float("nan"), device=DEV).view(torch.uint8)
    out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, topk_ids=torch.from_numpy(bad).to(DEV),
                        topk_w=torch.from_numpy(w).to(DEV), B=B, stage=2, workspace=work)
    # the two stages called one by one (moe_gemm2_combine marks the placed rows itself)
    srt = moe.moe_sort(torch.from_numpy(bad).to(DEV), torch.from_numpy(w).to(DEV), wl.E, B)
    h, hs = moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, B)
    g2 = torch.full((moe.moe_gemm2_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, B) // 4 + 1,),
                    float("nan"), device=DEV).view(torch.uint8)
    out2 = moe.moe_gemm2_combine(h, hs, ws["w2"], srt, wl.T, wl.k, B, workspace=g2)
    torch.cuda.synchronize()
    for o in (out, out2):
        assert torch.isfinite(o.float()).all()
        err, _ = rel_err(bf16_to_f64(bits(o)), ref)
        assert err <= TOL["bf16"], (B, err)
    assert not out[7].float().any() and not out2[7].float().any()


@pytest.mark.parametrize("T", (1, 2, 4))
def test_gemm1_k_split_few_tokens(T):
    """The single-token regime (T * k <= E) at the full Mixtral shape: with
    sort blocks of 16 or 32 rows, bf16 GEMM1 splits its reduction over d and a
    second kernel adds the parts in a fixed order before SwiGLU. Every token
    against the oracle on the two-stage path, for both block sizes and the
    library's choice; h is bit-identical over repeated calls."""
    wl = workloads.get("mixtral_decode").replace(name=f"decode_t{T}", T=T, seed=60 + T)
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ref, rid, rw = oracle_layer(wl, x, logits, ws)
    for B in (16, 32, 0):
        out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, B=B, stage=2 if B else 0)
        torch.cuda.synchronize()
        err, norm = rel_err(bf16_to_f64(bits(out)), ref)
        log(f"split GEMM1 T={T} B={B}: err={err:.3e} norm={norm:.3e}")
        assert err <= TOL["bf16"], (T, B, err)
    ids, w = torch.from_numpy(rid).to(DEV), torch.from_numpy(rw).to(DEV)
    srt = moe.moe_sort(ids, w, wl.E, 16)
    h1, _ = moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, 16)
    h2, _ = moe.moe_gemm1_swiglu(x, ws["w13"], srt, wl.k, 16)
    torch.cuda.synchronize()
    real = (srt["sorted_ids"] < wl.T * wl.k).cpu().numpy()
    assert np.array_equal(bits(h1)[real], bits(h2)[real])
