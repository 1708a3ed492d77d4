// moe_1stage.hip -- the one-stage fused MoE kernel: gate/up projection,
// SwiGLU and down projection in one launch (AITER walk-through,
// itsolotime.com/th/archives/32381, section 3.2: the one-stage path runs
// gate+up, the activation and down in a single kernel, and saves launches
// when there are few tokens).
//
// One workgroup = one sort block (B <= 32 rows of one expert) x one chunk of
// CH = 64 columns of the expert FFN:
//   phase 1: h_c = bf16(silu(A Wg[chunk]) * (A Wu[chunk]))  [B x 64]
//            (4 waves, 16 h-columns each, weight-streaming MFMA loop shared
//            with the two-stage GEMM1), kept in LDS;
//   phase 2: y = h_c Wd[:, chunk]                            [B x d]
//            (each wave one quarter of d, 16 columns at a time; the h_c
//            fragments stay in registers, Wd rows stream through);
//            acc[token] += sorted_w[slot] * y   (fp32 atomics).
// The chunks of f are partial sums of the down projection, so this is the
// two-stage path with the down projection K-split at chunk granularity: it
// trades the h round trip for rows * d * f / 64 atomics, which only pays at
// very small token counts.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int CH = 64;  // f-columns per workgroup

struct OneStageParams {
    const uint16_t *x;
    const uint16_t *w13;
    const uint16_t *w2;
    const int32_t *sorted_ids;
    const float *sorted_w;
    const int32_t *seid;
    float *acc;
    int T, d, f, k, B;
};

struct Frag {
    u32x4 lo, hi;
};

__device__ __forceinline__ Frag ld(const uint8_t *p) {
    Frag f;
    f.lo = *reinterpret_cast<const u32x4 *>(p);
    f.hi = *reinterpret_cast<const u32x4 *>(p + 16);
    return f;
}

__device__ __forceinline__ f32x4 mma2(const Frag &a, const Frag &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.lo),
                                                 __builtin_bit_cast(bf16x8, b.lo), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.hi),
                                                    __builtin_bit_cast(bf16x8, b.hi), c, 0, 0, 0);
}

// RT: 16-row tiles per block (B = 16 RT).
template <int RT>
__global__ __launch_bounds__(256) void k_moe_1stage(OneStageParams p) {
    const int blk = blockIdx.z;
    const int e = p.seid[blk];
    if (e < 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int sentinel = p.T * p.k;
    const int slot0 = blk * p.B;
    const int d = p.d, f = p.f;
    const int c0 = blockIdx.x * CH;  // first f-column of the chunk

    __shared__ __attribute__((aligned(16))) uint16_t hs[RT * 16][CH];

    // ---- phase 1: gate/up over K = d for 16 h-columns per wave ----------
    int a_of_lane[RT];
    const uint8_t *arow[RT];
    bool aok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int a = p.sorted_ids[slot0 + rt * 16 + lr];
        a_of_lane[rt] = a;
        aok[rt] = a < sentinel;
        const int t = aok[rt] ? a / p.k : 0;
        arow[rt] = reinterpret_cast<const uint8_t *>(p.x + (size_t)t * d) + lg * 32;
    }
    const int n = c0 + wave * 16 + lr;  // this lane's h-column (gate row n, up row f + n)
    const uint8_t *gw = reinterpret_cast<const uint8_t *>(p.w13 + ((size_t)e * 2 * f + n) * d) + lg * 32;
    const uint8_t *uw = reinterpret_cast<const uint8_t *>(p.w13 + ((size_t)e * 2 * f + f + n) * d) + lg * 32;
    f32x4 g[RT], u[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        g[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        u[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int nsteps = d / 64;  // 128-byte steps of bf16
    auto kof = [&](int i) { return (size_t)min(i, nsteps - 1) * 128; };
    Frag a0[RT], b0g, b0u, a1[RT], b1g, b1u;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) a0[rt] = ld(arow[rt]);
    b0g = ld(gw);
    b0u = ld(uw);
    for (int i = 0; i < nsteps; i += 2) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) a1[rt] = ld(arow[rt] + kof(i + 1));
        b1g = ld(gw + kof(i + 1));
        b1u = ld(uw + kof(i + 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            Frag a = a0[rt];
            if (!aok[rt]) a.lo = a.hi = u32x4{0, 0, 0, 0};
            g[rt] = mma2(a, b0g, g[rt]);
            u[rt] = mma2(a, b0u, u[rt]);
        }
        if (i + 1 >= nsteps) break;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) a0[rt] = ld(arow[rt] + kof(i + 2));
        b0g = ld(gw + kof(i + 2));
        b0u = ld(uw + kof(i + 2));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            Frag a = a1[rt];
            if (!aok[rt]) a.lo = a.hi = u32x4{0, 0, 0, 0};
            g[rt] = mma2(a, b1g, g[rt]);
            u[rt] = mma2(a, b1u, u[rt]);
        }
    }
    // SwiGLU; lane holds rows 4 lg + i of each row tile, column lr
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            hs[rt * 16 + lg * 4 + i][wave * 16 + lr] = f32_to_bf16_bits(silu(g[rt][i]) * u[rt][i]);
    __syncthreads();

    // ---- phase 2: y = h_c Wd[:, chunk] for this wave's quarter of d ------
    // The A fragments (h rows, K = the 64 chunk columns = one 128-byte step)
    // are loaded once; lane l serves row l % 16 and bytes 32 (l / 16) .. +32.
    Frag ha[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        ha[rt] = ld(reinterpret_cast<const uint8_t *>(&hs[rt * 16 + lr][0]) + lg * 32);
    // rows' destinations (tokens) and weights, for the lane's output rows
    int tok[RT][4];
    float wt[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a = __shfl(a_of_lane[rt], lg * 4 + i, 64);
            tok[rt][i] = a < sentinel ? a / p.k : -1;
            wt[rt][i] = a < sentinel ? p.sorted_w[slot0 + rt * 16 + lg * 4 + i] : 0.0f;
        }
    const int ncols = d / 4;  // per wave
    const int nbeg = wave * ncols;
    const uint8_t *dw = reinterpret_cast<const uint8_t *>(p.w2 + (size_t)e * d * f + c0) + lg * 32;
    auto wrow = [&](int t) { return dw + (size_t)(nbeg + min(t, ncols / 16 - 1) * 16 + lr) * f * 2; };
    const int ntile = ncols / 16;
    Frag w0 = ld(wrow(0)), w1;
    auto emit = [&](const Frag &w, int t) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 y = mma2(ha[rt], w, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok[rt][i] >= 0)
                    atomic_add_f32(p.acc + (size_t)tok[rt][i] * d + nbeg + t * 16 + lr, wt[rt][i] * y[i]);
        }
    };
    for (int t = 0; t < ntile; t += 2) {
        w1 = ld(wrow(t + 1));
        __builtin_amdgcn_sched_barrier(0);
        emit(w0, t);
        if (t + 1 >= ntile) break;
        w0 = ld(wrow(t + 2));
        __builtin_amdgcn_sched_barrier(0);
        emit(w1, t + 1);
    }
}

}  // namespace

bool onestage_supported(const GemmShape &sh) {
    return sh.quant == 0 && (sh.B == 16 || sh.B == 32) && sh.f % CH == 0 && sh.d % 64 == 0;
}

hipError_t launch_moe_1stage(const GemmShape &sh, const void *x, const void *w13, const void *w2,
                             const int32_t *sorted_ids, const float *sorted_w,
                             const int32_t *sorted_expert_ids, float *acc, hipStream_t s) {
    OneStageParams p{};
    p.x = static_cast<const uint16_t *>(x);
    p.w13 = static_cast<const uint16_t *>(w13);
    p.w2 = static_cast<const uint16_t *>(w2);
    p.sorted_ids = sorted_ids;
    p.sorted_w = sorted_w;
    p.seid = sorted_expert_ids;
    p.acc = acc;
    p.T = sh.T; p.d = sh.d; p.f = sh.f; p.k = sh.k; p.B = sh.B;
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + sh.B - 1) / sh.B;
    const dim3 grid(sh.f / CH, 1, NB);
    if (sh.B == 16)
        k_moe_1stage<1><<<grid, 256, 0, s>>>(p);
    else if (sh.B == 32)
        k_moe_1stage<2><<<grid, 256, 0, s>>>(p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
