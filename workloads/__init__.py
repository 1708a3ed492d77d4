"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic. Both the GPU library's tests/benchmark and the CPU oracle
take their inputs from here.

Recipes (one seed per workload; every expert's weights come from their own
generator seeded ``seed * 1000 + e`` so that any subset of experts can be
re-created):

* activations ``x`` [T, d]: N(0, 1) drawn in fp32, stored as bf16;
* router logits [T, E] fp32: N(0, 1); the tiny layer instead projects its bf16
  activations with a router matrix W_r [d, E] ~ N(0, 1/sqrt(d)) in fp32; the
  DeepSeek-shaped layer uses Zipf(1.1)-skewed logits
  ``-1.1 * ln(e + 1) + Gumbel(0, 1)`` so that top-1 choices follow Zipf(1.1)
  over expert ranks and top-k is a Plackett-Luce draw;
* expert weights, generated directly in the kernel layout (reduction dim
  contiguous): ``w13`` [E, 2f, d] holds the gate rows then the up rows,
  ``w2`` [E, d, f]; entries ~ N(0, 1/sqrt(fan_in)) with fan_in = d for w13 and
  f for w2;
* fp8 weights are stored as OCP e4m3 codes with fp32 scales: one scale per
  output row (``fp8_token``) or per 128x128 block (``fp8_block``), each scale
  = amax / 448 of what it covers; codes come from torch's e4m3 cast after a
  clamp to +-448 (input preparation only: the layer never quantises weights);
* MXFP4 weights (``mxfp4``) are drawn directly as stored values, with no
  rounding step: E2M1 codes uniform over all 16 codes, packed two per byte
  (even column in the low nibble), and one E8M0 scale code per 32 consecutive
  reduction elements, ``127 + floor(log2(1 / (2.25 sqrt(fan_in)))) - b`` with
  b uniform in {0, 1} (2.25 is the mean magnitude of a uniform code), so the
  entries have about the spread of the N(0, 1/sqrt(fan_in)) recipe.

Values depend on the device used to draw them (torch's CPU and GPU generators
differ); a test draws on one device and copies what the oracle needs.
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["Workload", "WORKLOADS", "get"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    quant: str = "bf16"          # "bf16" | "fp8_token" | "fp8_block" | "mxfp4"
    score: str = "softmax"       # "softmax" | "sigmoid"
    logits: str = "normal"       # "normal" | "router" | "zipf"
    seed: int = 0
    zipf_s: float = 1.1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- activations and logits --------------------------------------
    def activations(self, device="cpu"):
        """x [T, d] bf16 and router logits [T, E] fp32."""
        g = torch.Generator(device=device).manual_seed(self.seed)
        x32 = torch.randn(self.T, self.d, generator=g, device=device, dtype=torch.float32)
        x = x32.to(torch.bfloat16)
        if self.logits == "router":
            wr = torch.randn(self.d, self.E, generator=g, device=device) / math.sqrt(self.d)
            logits = x.float() @ wr
        elif self.logits == "zipf":
            u = torch.rand(self.T, self.E, generator=g, device=device, dtype=torch.float64)
            u = u.clamp_min(1e-300)
            gumbel = -torch.log(-torch.log(u))
            rank = torch.arange(1, self.E + 1, device=device, dtype=torch.float64)
            logits = (-self.zipf_s * torch.log(rank) + gumbel).to(torch.float32)
        else:
            logits = torch.randn(self.T, self.E, generator=g, device=device, dtype=torch.float32)
        return x.contiguous(), logits.contiguous()

    # ---- weights -----------------------------------------------------
    def _expert_fp32(self, e: int, device):
        g = torch.Generator(device=device).manual_seed(self.seed * 1000 + e)
        w13 = torch.randn(2 * self.f, self.d, generator=g, device=device) / math.sqrt(self.d)
        w2 = torch.randn(self.d, self.f, generator=g, device=device) / math.sqrt(self.f)
        return w13, w2

    @staticmethod
    def _codes(w, scale_full):
        q = (w / scale_full).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return q.view(torch.uint8)

    def _store(self, w):
        """One expert matrix [N, K] -> (stored tensor, scales or None)."""
        if self.quant == "bf16":
            return w.to(torch.bfloat16), None
        if self.quant == "fp8_token":
            amax = w.abs().amax(dim=1)
            s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
            return self._codes(w, s[:, None]), s.float()
        N, K = w.shape
        blocks = w.reshape(N // 128, 128, K // 128, 128)
        amax = blocks.abs().amax(dim=(1, 3))
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        full = s[:, None, :, None].expand(N // 128, 128, K // 128, 128).reshape(N, K)
        return self._codes(w, full), s.float().contiguous()

    def _expert_mx(self, e: int, device):
        g = torch.Generator(device=device).manual_seed(self.seed * 1000 + e)

        def draw(N, K):
            codes = torch.randint(0, 256, (N, K // 2), generator=g, device=device, dtype=torch.int32)
            base = 127 + math.floor(math.log2(1.0 / (2.25 * math.sqrt(K))))
            b = torch.randint(0, 2, (N, K // 32), generator=g, device=device, dtype=torch.int32)
            return codes.to(torch.uint8), (base - b).to(torch.uint8)

        a, sa = draw(2 * self.f, self.d)
        b, sb = draw(self.d, self.f)
        return dict(w13=a, w13_scale=sa, w2=b, w2_scale=sb)

    def expert(self, e: int, device="cpu"):
        """Weights of expert e: dict w13, w13_scale, w2, w2_scale (scales None for bf16)."""
        if self.quant == "mxfp4":
            return self._expert_mx(e, device)
        w13, w2 = self._expert_fp32(e, device)
        a, sa = self._store(w13)
        b, sb = self._store(w2)
        return dict(w13=a.contiguous(), w13_scale=sa, w2=b.contiguous(), w2_scale=sb)

    def weights(self, device="cpu"):
        """All experts stacked: w13 [E,2f,d], w2 [E,d,f] and scales."""
        wdt = torch.bfloat16 if self.quant == "bf16" else torch.uint8
        pk = 2 if self.quant == "mxfp4" else 1   # elements per stored byte
        w13 = torch.empty(self.E, 2 * self.f, self.d // pk, dtype=wdt, device=device)
        w2 = torch.empty(self.E, self.d, self.f // pk, dtype=wdt, device=device)
        if self.quant == "mxfp4":
            s13 = torch.empty(self.E, 2 * self.f, self.d // 32, dtype=torch.uint8, device=device)
            s2 = torch.empty(self.E, self.d, self.f // 32, dtype=torch.uint8, device=device)
        elif self.quant == "fp8_token":
            s13 = torch.empty(self.E, 2 * self.f, device=device)
            s2 = torch.empty(self.E, self.d, device=device)
        elif self.quant == "fp8_block":
            s13 = torch.empty(self.E, 2 * self.f // 128, self.d // 128, device=device)
            s2 = torch.empty(self.E, self.d // 128, self.f // 128, device=device)
        else:
            s13 = s2 = None
        for e in range(self.E):
            ex = self.expert(e, device)
            w13[e].copy_(ex["w13"])
            w2[e].copy_(ex["w2"])
            if s13 is not None:
                s13[e].copy_(ex["w13_scale"])
                s2[e].copy_(ex["w2_scale"])
        return dict(w13=w13, w13_scale=s13, w2=w2, w2_scale=s2)

    # ---- algorithmic sizes (count each touched expert's weights once) -----
    def weight_bytes_per_expert(self) -> int:
        if self.quant == "mxfp4":
            return 3 * self.d * self.f // 2 + 3 * self.d * self.f // 32
        eb = 2 if self.quant == "bf16" else 1
        b = 3 * self.d * self.f * eb
        if self.quant == "fp8_token":
            b += 4 * (2 * self.f + self.d)
        elif self.quant == "fp8_block":
            b += 4 * (2 * self.f * self.d + self.d * self.f) // (128 * 128)
        return b

    def flops(self) -> int:
        return 6 * self.d * self.f * self.T * self.k


# The workloads: a tiny layer plus Mixtral-8x7B- and DeepSeek-V3-shaped layers
# (seed = 1000 + index).
WORKLOADS = {
    "tiny": Workload("tiny", T=16, d=128, f=256, E=4, k=2, logits="router", seed=1001),
    "mixtral_decode": Workload("mixtral_decode", T=32, d=4096, f=14336, E=8, k=2, seed=1002),
    "mixtral_prefill": Workload("mixtral_prefill", T=4096, d=4096, f=14336, E=8, k=2, seed=1003),
    "mixtral_fp8": Workload("mixtral_fp8", T=512, d=4096, f=14336, E=8, k=2,
                            quant="fp8_token", seed=1004),
    "deepseek_fp8": Workload("deepseek_fp8", T=128, d=7168, f=2048, E=256, k=8,
                             quant="fp8_block", score="sigmoid", logits="zipf", seed=1005),
    # the per_1x32 (MXFP4) quant type on the Mixtral decode shape
    "mixtral_mxfp4": Workload("mixtral_mxfp4", T=32, d=4096, f=14336, E=8, k=2,
                              quant="mxfp4", seed=1006),
    "mixtral_prefill_mxfp4": Workload("mixtral_prefill_mxfp4", T=4096, d=4096, f=14336, E=8, k=2,
                                      quant="mxfp4", seed=1007),
    # the single-token decode regime (T * k <= E) on the Mixtral shape
    "mixtral_single": Workload("mixtral_single", T=1, d=4096, f=14336, E=8, k=2, seed=1008),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
