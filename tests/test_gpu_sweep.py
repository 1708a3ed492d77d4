"""A seeded sweep of layer shapes and launch choices against the CPU oracle.

Thirty-two configurations drawn once from a fixed-seed generator: token
counts from 1 to 511 (ragged against every block size), 1 to 256 experts,
top-1 to top-8, softmax and sigmoid scores over normal and Zipf logits,
every weight format, and for each a block size the shape allows (the tiled
kernels where the sizes permit them), a stage and a K-split. Each fused
layer must meet the output bar of the other parity tests."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_sorting_amd as moe
import workloads
from gpu_helpers import DEV, TOL, bits, bf16_to_f64, log, oracle_layer, rel_err

pytestmark = pytest.mark.gpu

QUANTS = ("bf16", "fp8_token", "fp8_block", "mxfp4")


def _tiled_ok(quant, d, f):
    if quant == "mxfp4":
        return d % 512 == 0 and f % 512 == 0
    return quant in ("bf16", "fp8_token") and d % 256 == 0 and f % 128 == 0


def _cases(n=32, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        q = QUANTS[i % 4]
        E = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32, 64, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 2, 3, 5, 8, 17, 33, 64, 100, 130, 257, 511]))
        unit = 512 if q == "mxfp4" else 128
        big = 1 if E >= 64 else 3
        d = unit * int(rng.integers(1, big + 1)) * (2 if q != "mxfp4" and rng.random() < 0.5 else 1)
        f = unit * int(rng.integers(1, big + 1))
        score = "sigmoid" if rng.random() < 0.3 else "softmax"
        logits = "zipf" if rng.random() < 0.3 else "normal"
        Bs = [16, 32] + ([64, 128, 256] if _tiled_ok(q, d, f) else [])
        B = int(rng.choice(Bs))
        stage = 1 if (q == "bf16" and B <= 32 and rng.random() < 0.4) else 2
        ksplit = int(rng.choice([0, 1, 2, 3]))
        wl = workloads.Workload(f"sweep{i:02d}", T=T, d=d, f=f, E=E, k=k, quant=q, score=score,
                                logits=logits, seed=3000 + i)
        out.append((wl, B, stage, ksplit))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[
    f"{w.name}-{w.quant}-T{w.T}-E{w.E}k{w.k}-d{w.d}f{w.f}-B{B}s{s}ks{ks}" for w, B, s, ks in CASES])
def test_sweep_fused_against_the_oracle(case):
    wl, B, stage, ksplit = case
    x, logits = wl.activations(DEV)
    ws = wl.weights(DEV)
    ref, _, _ = oracle_layer(wl, x, logits, ws)
    out = moe.fused_moe(x, ws["w13"], ws["w2"], wl.k, logits=logits, quant=wl.quant,
                        w13_scale=ws["w13_scale"], w2_scale=ws["w2_scale"], score=wl.score,
                        B=B, stage=stage, ksplit=ksplit)
    torch.cuda.synchronize()
    err, norm = rel_err(bf16_to_f64(bits(out)), ref)
    log(f"sweep {wl.name}: err={err:.3e} norm={norm:.3e}")
    assert torch.isfinite(out.float()).all()
    assert err <= TOL[wl.quant], (wl, B, stage, ksplit, err)
