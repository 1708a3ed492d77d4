"""fused_moe_noalloc (the no-allocation variant of fused_moe, whose
workspace is the library's static per-GPU array) against fused_moe with a
caller-allocated workspace, through the C ABI: two calls in a row, the
second on a smaller input, both within the bf16 output tolerance of the
first entry point's result; the same call captured in a HIP graph, whose
every replay (with other calls on the same static array between replays)
matches the eager result; and a layer too large for the static array is
refused before any device work."""
import os
import re

import numpy as np
import pytest
import torch

import moe_grouped_gemm_sorting_amd as moe
import workloads
from gpu_helpers import DEV, TOL, bits, bf16_to_f64, log, rel_err

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_scratch_size_matches_the_header():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == moe.NOALLOC_SCRATCH_BYTES


def _both(wl, x, logits, ws, **kw):
    ref = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, quant=wl.quant,
                        w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score, **kw)
    got = moe.fused_moe_noalloc(x, ws["w13"], ws["w2"], wl.k, logits=logits, quant=wl.quant,
                                w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score, **kw)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("name,B", [("mixtral_decode", 0), ("mixtral_fp8", 64), ("deepseek_fp8", 0)])
def test_noalloc_matches_fused_moe_on_two_calls(name, B):
    wl = workloads.get(name)
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    need = moe.fused_moe_workspace_bytes(wl.T if name != "mixtral_fp8" else 64, wl.d, wl.f, wl.E,
                                         wl.k, wl.quant, B, 2 if B else 0)
    assert 0 < need <= moe.NOALLOC_SCRATCH_BYTES
    T1 = wl.T if name != "mixtral_fp8" else 64   # the first call: up to the full decode batch
    for T in (T1, max(1, T1 // 4)):              # then a smaller input on the same scratch
        xs, ls = x[:T].contiguous(), logits[:T].contiguous()
        got, ref = _both(wl, xs, ls, ws, B=B, stage=2 if B else 0)
        err, _ = rel_err(bf16_to_f64(bits(got)), bf16_to_f64(bits(ref)))
        log(f"noalloc {name} T={T} B={B}: err against fused_moe {err:.3e}")
        assert err <= TOL[wl.quant]
        assert torch.isfinite(got.float()).all()


@pytest.mark.parametrize("name", ["mixtral_decode", "deepseek_fp8"])
def test_noalloc_graph_replays_match_eager(name):
    wl = workloads.get(name)
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    kw = dict(quant=wl.quant, w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score)
    ref = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, **kw)
    # the captured call's inputs and output live in fixed buffers
    xg, lg = x.clone(), logits.clone()
    out = torch.empty_like(ref)
    # an eager call first: it finds the scratch array's address
    moe.fused_moe_noalloc(xg, ws["w13"], ws["w2"], wl.k, logits=lg, out=out, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.fused_moe_noalloc(xg, ws["w13"], ws["w2"], wl.k, logits=lg, out=out, **kw)
    torch.cuda.synchronize()
    other_x = torch.randn_like(x.float()).to(torch.bfloat16)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        err, _ = rel_err(bf16_to_f64(bits(out)), bf16_to_f64(bits(ref)))
        log(f"graph replay {rep} of {name}: err against eager fused_moe {err:.3e}")
        assert torch.isfinite(out.float()).all()
        assert err <= TOL[wl.quant]
        # eager work between replays, on the same static array
        moe.fused_moe_noalloc(other_x, ws["w13"], ws["w2"], wl.k, logits=lg, **kw)
        torch.cuda.synchronize()


def test_noalloc_refuses_layers_beyond_its_scratch():
    wl = workloads.get("mixtral_prefill").replace(T=2048)
    need = moe.fused_moe_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k, wl.quant, 0, 0)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(wl.T, wl.d, dtype=torch.bfloat16, device=DEV)
    logits = torch.zeros(wl.T, wl.E, dtype=torch.float32, device=DEV)
    w13 = torch.zeros(wl.E, 2 * wl.f, wl.d, dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros(wl.E, wl.d, wl.f, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError, match="static scratch"):
        moe.fused_moe_noalloc(x, w13, w2, wl.k, logits=logits)
