// gemm_tiled.hip -- LDS-tiled grouped GEMMs for large sort blocks (B = 64, 128).
//
// The compute-bound regime of the grouped GEMMs (many rows per expert, e.g.
// prefill): grouped GEMMs in place of masked dense GEMMs (rocketrecap.com/
// entries/19116, talk summary at 5:58), run as the two stages of the AITER
// walk-through (itsolotime.com/th/archives/32381, section 3.2).
//
// Workgroup tile: one sort block (BM = B rows of one expert) x 256 weight
// rows (GEMM1: 128 gate rows + the 128 matching up rows, so SwiGLU fuses into
// the epilogue; GEMM2: 256 output columns), K in steps of 128 bytes per row.
// 8 waves in a 2 x 4 arrangement, each owning (BM/2) x 64 of the tile, with
// v_mfma_f32_32x32x16_bf16 or, for e4m3, v_mfma_scale_f32_32x32x64_f8f6f4
// with unit scales (per-row / per-channel fp32 scales go in the epilogue).
//
// Operands are staged through LDS, double-buffered, one barrier per K step.
// Each 128-byte row segment is stored as 8 chunks of 16 bytes whose position
// is XOR-swizzled per row (see swz), so that a fragment read (32 rows, one
// chunk column) spreads over all banks.
//
// Tile order: tiles are enumerated block-group-major (GM sort blocks x all
// column tiles), and workgroup i, which the hardware places on XCD i % 8,
// takes logical tile (i % 8) * ceil(tiles / 8) + i / 8. Neighbouring tiles,
// which share activation rows and weight rows, therefore run on the same XCD
// and share its L2. The tile count comes from num_valid on the device, so
// no XCD is left with the padding blocks.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TILE_N = 256;     // weight rows per workgroup
constexpr int ROWB = 128;       // bytes per row per K step
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
constexpr int GROUP_M = MOE_GROUP_M;  // sort blocks per tile group
#ifndef MOE_TILED_NSTAGE
#define MOE_TILED_NSTAGE 2
#endif
constexpr int NSTAGE = MOE_TILED_NSTAGE;  // K steps of global loads in flight

struct TiledParams {
    const uint8_t *a;
    const float *a_scale;
    const uint8_t *w;
    const float *w_scale;
    const int32_t *sorted_ids;
    const float *sorted_w;
    const int32_t *seid;
    const int32_t *num_valid;
    void *out;
    float *out_scale;
    int T, d, f, k, B;
    int kchunk;
    float *zero;
    size_t zero_n;
};

// Chunk position of (row, chunk) inside the row's 128 bytes. A fragment read
// takes one chunk column of consecutive rows: any 8 consecutive rows land on 8
// different positions (32-bank LDS, 8 lanes per cycle) and any 16 on 16
// different (row parity, position) pairs (64 banks, 16 lanes per cycle).
#ifndef MOE_SWIZZLE
#define MOE_SWIZZLE 1
#endif
__device__ __forceinline__ int swz(int row, int chunk) {
#if MOE_SWIZZLE == 1
    return chunk ^ (row & 7) ^ ((row >> 3) & 1);
#else
    return chunk ^ ((row >> 1) & 7);
#endif
}

__device__ __forceinline__ f32x16 mma32_bf16(const u32x4 &a, const u32x4 &b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// e4m3 x e4m3 over K = 64 (32 bytes per lane: two LDS chunks) with unit
// E8M0 scales; A and B use the same lane/byte layout.
__device__ __forceinline__ f32x16 mma32_fp8(const u32x4 &a0, const u32x4 &a1, const u32x4 &b0,
                                            const u32x4 &b1, f32x16 acc) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                      (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
}

// BM: rows per sort block (64 or 128). QUANT 0 (bf16) or 1 (e4m3, per-row
// activation scale and per-channel weight scale applied in the epilogue).
// WAVES: 4 (2 x 2 waves, each (BM/2) x 128) or 8 (2 x 4 waves, each
// (BM/2) x 64, two waves per SIMD so that one wave's MFMAs cover the other's
// LDS and barrier waits).
template <int QUANT, bool GEMM1, int BM, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_tiled(TiledParams p) {
    constexpr int NTHR = 64 * WAVES;
    constexpr int ES = QUANT == 0 ? 2 : 1;
    constexpr int KS = ROWB / ES;               // K elements per step
    constexpr int A_CHUNKS = BM * 8 / NTHR;     // 16-byte chunks per thread per step
    constexpr int B_CHUNKS = TILE_N * 8 / NTHR;
    constexpr int RPASS = NTHR / 8;             // rows covered by one pass of the threads
    constexpr int WN = WAVES / 2;               // waves along the weight rows
    constexpr int RT = BM / 64;                 // 32-row tiles per wave
    constexpr int CT = TILE_N / WN / 32;        // 32-column tiles per wave
    constexpr int BUF = (BM + TILE_N) * ROWB;   // bytes per LDS buffer
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (p.zero) {
        const size_t nwg = (size_t)gridDim.x * gridDim.y;
        const size_t wg = blockIdx.x + (size_t)gridDim.x * blockIdx.y;
        float4 *z = reinterpret_cast<float4 *>(p.zero);
        for (size_t i = wg * NTHR + tid; i < p.zero_n / 4; i += nwg * NTHR)
            z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // ---- which tile -------------------------------------------------------
    const int ntiles = GEMM1 ? p.f / 128 : p.d / TILE_N;
    // tiles of BM rows; the sort block B is a multiple of BM, so a tile never
    // straddles two experts
    const int nblocks = *p.num_valid / BM;
    const int total = nblocks * ntiles;
    const int per_xcd = (total + 7) / 8;
    const int j = blockIdx.x >> 3;
    if (j >= per_xcd) return;
    const int logical = (blockIdx.x & 7) * per_xcd + j;
    if (logical >= total) return;
    const int group = logical / (GROUP_M * ntiles);
    const int gm = min(GROUP_M, nblocks - group * GROUP_M);
    const int r = logical - group * GROUP_M * ntiles;
    const int nt = r / gm;
    const int blk = group * GROUP_M + r % gm;
    const int e = p.seid[blk * BM / p.B];
    if (e < 0) return;

    const int sentinel = p.T * p.k;
    // a tile of padding only (the tail of a larger sort block)
    if (p.sorted_ids[blk * BM] >= sentinel) return;
    const int K = GEMM1 ? p.d : p.f;
    const int Ntot = GEMM1 ? 2 * p.f : p.d;
    const int slot0 = blk * BM;
    const int kbeg = blockIdx.y * p.kchunk;
    const int kend = min(K, kbeg + p.kchunk);

    // ---- global -> LDS staging assignment ---------------------------------
    // thread t moves chunk (t & 7) of rows (t >> 3) + RPASS i.
    const int cchunk = tid & 7, crow = tid >> 3;
    // 32-bit byte offsets from wave-uniform bases keep the address registers
    // few (the host guarantees every operand matrix is below 4 GiB).
    uint32_t aoff[A_CHUNKS];
    bool aok[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int row = crow + RPASS * i;
        const int slot = slot0 + row;
        if (GEMM1) {
            const int a = p.sorted_ids[slot];
            aok[i] = a < sentinel;
            const int t = aok[i] ? a / p.k : 0;
            aoff[i] = (uint32_t)t * (uint32_t)(K * ES) + cchunk * 16;
        } else {
            aok[i] = true;
            aoff[i] = (uint32_t)slot * (uint32_t)(K * ES) + cchunk * 16;
        }
    }
    uint32_t boff[B_CHUNKS];
    const uint8_t *wexp = p.w + (size_t)e * Ntot * K * ES;
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
        const int row = crow + RPASS * i;   // 0..255
        int n;
        if (GEMM1)
            n = (row < 128 ? 0 : p.f - 128) + nt * 128 + row;
        else
            n = nt * TILE_N + row;
        boff[i] = (uint32_t)n * (uint32_t)(K * ES) + cchunk * 16;
    }
    struct Stage {
        u32x4 a[A_CHUNKS], b[B_CHUNKS];
    };
    // kk is clamped by the caller; the loads are unconditional so that the
    // wait counts in the unrolled loop stay exact.
    auto gload = [&](Stage &st, int kk) {
        const uint8_t *ab = p.a + (size_t)kk * ES;
        const uint8_t *bb = wexp + (size_t)kk * ES;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) st.a[i] = *reinterpret_cast<const u32x4 *>(ab + aoff[i]);
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) st.b[i] = *reinterpret_cast<const u32x4 *>(bb + boff[i]);
    };
    auto lstore = [&](const Stage &st, int buf) {
        uint8_t *base = lds + buf * BUF;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            // padding rows are zeroed here, where the data has arrived anyway
            // (masking right after the load would stall the prefetch)
            const int row = crow + RPASS * i;
            *reinterpret_cast<u32x4 *>(base + row * ROWB + swz(row, cchunk) * 16) =
                aok[i] ? st.a[i] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int row = crow + RPASS * i;
            *reinterpret_cast<u32x4 *>(base + (BM + row) * ROWB + swz(row, cchunk) * 16) = st.b[i];
        }
    };

    // ---- compute assignment -------------------------------------------------
    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 31, lh = lane >> 5;
    int arow[RT], brow[CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) arow[rt] = wm * (BM / 2) + rt * 32 + lr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        // GEMM1: the first CT/2 tiles are gate rows, the last CT/2 the matching up rows
        if (GEMM1)
            brow[ct] = (ct < CT / 2 ? 0 : 128) + wn * (128 / WN) + (ct % (CT / 2)) * 32 + lr;
        else
            brow[ct] = wn * (TILE_N / WN) + ct * 32 + lr;
    }
    f32x16 acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0.0f;

    auto frags_at = [&](const uint8_t *base, int chunk, u32x4 (&fa)[RT], u32x4 (&fb)[CT]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            fa[rt] = *reinterpret_cast<const u32x4 *>(base + arow[rt] * ROWB + swz(arow[rt], chunk) * 16);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            fb[ct] = *reinterpret_cast<const u32x4 *>(base + (BM + brow[ct]) * ROWB +
                                                      swz(brow[ct], chunk) * 16);
    };
    // bf16: 4 sub-steps of K = 16 (lane half lh takes chunk 2s + lh); the
    // fragments of sub-step s+1 are read while the MFMAs of sub-step s run.
    // e4m3: 2 sub-steps of K = 64 (lane half lh takes chunks 4s + 2lh and
    // 4s + 2lh + 1). The next step's staged operands (`st`, already in
    // registers) are written to the other LDS buffer right after the first
    // fragment reads, so that the LDS writes overlap the MFMAs instead of
    // forming a burst before the barrier.
    auto compute = [&](int buf, const Stage &st) {
        const uint8_t *base = lds + buf * BUF;
        if constexpr (QUANT == 0) {
            u32x4 fa0[RT], fb0[CT], fa1[RT], fb1[CT];
            frags_at(base, lh, fa0, fb0);
            lstore(st, buf ^ 1);
#pragma unroll
            for (int sub = 0; sub < 4; sub += 2) {
                frags_at(base, 2 * (sub + 1) + lh, fa1, fb1);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = mma32_bf16(fa0[rt], fb0[ct], acc[rt][ct]);
                if (sub + 2 < 4) frags_at(base, 2 * (sub + 2) + lh, fa0, fb0);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = mma32_bf16(fa1[rt], fb1[ct], acc[rt][ct]);
            }
        } else {
            u32x4 fa0[RT], fb0[CT], fa1[RT], fb1[CT];
            u32x4 ga0[RT], gb0[CT], ga1[RT], gb1[CT];
            frags_at(base, 2 * lh, fa0, fb0);
            frags_at(base, 2 * lh + 1, fa1, fb1);
            lstore(st, buf ^ 1);
            frags_at(base, 4 + 2 * lh, ga0, gb0);
            frags_at(base, 4 + 2 * lh + 1, ga1, gb1);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    acc[rt][ct] = mma32_fp8(fa0[rt], fa1[rt], fb0[ct], fb1[ct], acc[rt][ct]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    acc[rt][ct] = mma32_fp8(ga0[rt], ga1[rt], gb0[ct], gb1[ct], acc[rt][ct]);
        }
    };

    // ---- main loop -------------------------------------------------------
    // LDS holds step j (double-buffered); NSTAGE register sets hold steps
    // j+1 .. j+NSTAGE in flight, so a global load has about NSTAGE steps of
    // compute to land. One iteration: load step j+NSTAGE into the set that
    // held step j, compute step j, move step j+1 from its set into the other
    // LDS buffer, barrier. Unrolled by 2*NSTAGE so every set / buffer index is
    // a compile-time constant; loads past the end are clamped to the last
    // step (cache hits) to keep the wait counts exact.
    const int nsteps = (kend - kbeg) / KS;
    if (nsteps > 0) {
        auto kof = [&](int i) { return kbeg + min(i, nsteps - 1) * KS; };
        Stage r[NSTAGE];
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s) gload(r[s], kof(s));
        lstore(r[0], 0);
        __syncthreads();
        constexpr int UNR = 2 * NSTAGE;
        int j = 0;
        for (; j + UNR <= nsteps; j += UNR) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                gload(r[u % NSTAGE], kof(j + u + NSTAGE));
                __builtin_amdgcn_sched_barrier(0);
                compute(u & 1, r[(u + 1) % NSTAGE]);
                __syncthreads();
            }
        }
        // the remaining steps (fewer than UNR), same pattern
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (j + u < nsteps) {
                gload(r[u % NSTAGE], kof(j + u + NSTAGE));
                __builtin_amdgcn_sched_barrier(0);
                compute(u & 1, r[(u + 1) % NSTAGE]);
                __syncthreads();
            }
        }
    }

    // ---- epilogue -----------------------------------------------------------
    // 32x32 accumulator layout: lane holds column (lane & 31) and rows
    // 8 * (v / 4) + 4 * (lane >> 5) + (v & 3), v = 0..15.
    if constexpr (GEMM1) {
        const int f = p.f;
        uint16_t *h = reinterpret_cast<uint16_t *>(p.out);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * (BM / 2) + rt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                const int slot = slot0 + row;
                float sx = 1.0f;
                if constexpr (QUANT == 1) {
                    const int a = p.sorted_ids[slot];
                    sx = a < sentinel ? p.a_scale[a / p.k] : 0.0f;
                }
                float m = 0.0f;
#pragma unroll
                for (int c = 0; c < CT / 2; ++c) {
                    const int n = nt * 128 + wn * (128 / WN) + c * 32 + lr;
                    float g = acc[rt][c][v], u = acc[rt][c + CT / 2][v];
                    if constexpr (QUANT == 1) {
                        g = g * sx * p.w_scale[(size_t)e * Ntot + n];
                        u = u * sx * p.w_scale[(size_t)e * Ntot + f + n];
                    }
                    const uint16_t hb = f32_to_bf16_bits(silu(g) * u);
                    h[(size_t)slot * f + n] = hb;
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(hb)));
                }
                if constexpr (QUANT == 1) {
#pragma unroll
                    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                    if (lr == 0) atomic_max_nonneg(p.out_scale + slot, m);
                }
            }
        }
    } else {
        float *accg = reinterpret_cast<float *>(p.out);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * (BM / 2) + rt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                const int slot = slot0 + row;
                const int a = p.sorted_ids[slot];
                if (a >= sentinel) continue;
                float wgt = p.sorted_w[slot];
                if constexpr (QUANT == 1) wgt *= p.a_scale[slot];
                float *dst = accg + (size_t)(a / p.k) * p.d;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int n = nt * TILE_N + wn * (TILE_N / WN) + ct * 32 + lr;
                    float y = acc[rt][ct][v];
                    if constexpr (QUANT == 1) y *= p.w_scale[(size_t)e * Ntot + n];
                    atomic_add_f32(dst + n, wgt * y);
                }
            }
        }
    }
}

#ifndef MOE_TILED_WAVES
#define MOE_TILED_WAVES 8
#endif

template <int QUANT, bool GEMM1>
hipError_t dispatch_bm(const TiledParams &p, int BM, dim3 grid, hipStream_t s) {
    constexpr int W = MOE_TILED_WAVES;
    if (BM == 64)
        k_gemm_tiled<QUANT, GEMM1, 64, W><<<grid, 64 * W, 0, s>>>(p);
    else if (BM == 128)
        k_gemm_tiled<QUANT, GEMM1, 128, W><<<grid, 64 * W, 0, s>>>(p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool GEMM1>
hipError_t dispatch(const TiledParams &p, int quant, int BM, dim3 grid, hipStream_t s) {
    if (quant == 0) return dispatch_bm<0, GEMM1>(p, BM, grid, s);
    if (quant == 1) return dispatch_bm<1, GEMM1>(p, BM, grid, s);
    return hipErrorInvalidValue;
}

unsigned grid_tiles(int NB, int ntiles) {
    const unsigned total = (unsigned)NB * (unsigned)ntiles;
    return (total + 7) / 8 * 8;
}

}  // namespace

bool tiled_gemm_supported(const GemmShape &sh) {
    return (sh.B == 64 || sh.B == 128 || sh.B == 256) && (sh.quant == 0 || sh.quant == 1) &&
           sh.f % 128 == 0 && sh.d % 256 == 0;
}

// Rows per kernel tile: 64 or 128, a divisor of the sort block B (a 256-row
// sort block runs as two 128-row tiles); other values pick min(B, 128).
int tile_rows(int B, int bm) {
    if (bm <= 0 || bm > B || B % bm || bm > 128) bm = B < 128 ? B : 128;
    return bm;
}

hipError_t launch_tiled_gemm1(const Gemm1Args &g, int bm, hipStream_t s) {
    const GemmShape &sh = g.sh;
    TiledParams p{};
    p.a = static_cast<const uint8_t *>(g.a);
    p.a_scale = g.a_scale;
    p.w = static_cast<const uint8_t *>(g.w13);
    p.w_scale = g.w13_scale;
    p.sorted_ids = g.sorted_ids;
    p.seid = g.sorted_expert_ids;
    p.num_valid = g.num_valid;
    p.out = g.h;
    p.out_scale = g.h_scale;
    p.T = sh.T; p.d = sh.d; p.f = sh.f; p.k = sh.k; p.B = sh.B;
    p.kchunk = sh.d;
    p.zero = g.zero;
    p.zero_n = g.zero_n;
    bm = tile_rows(sh.B, bm);
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + bm - 1) / bm;
    const dim3 grid(grid_tiles(NB, sh.f / 128), 1);
    return dispatch<true>(p, sh.quant, bm, grid, s);
}

hipError_t launch_tiled_gemm2(const Gemm2Args &g, int bm, int ksplit, hipStream_t s) {
    const GemmShape &sh = g.sh;
    TiledParams p{};
    p.a = static_cast<const uint8_t *>(g.h);
    p.a_scale = g.h_scale;
    p.w = static_cast<const uint8_t *>(g.w2);
    p.w_scale = g.w2_scale;
    p.sorted_ids = g.sorted_ids;
    p.sorted_w = g.sorted_w;
    p.seid = g.sorted_expert_ids;
    p.num_valid = g.num_valid;
    p.out = g.acc;
    p.T = sh.T; p.d = sh.d; p.f = sh.f; p.k = sh.k; p.B = sh.B;
    const int KS = sh.quant == 0 ? 64 : 128;
    const int steps = sh.f / KS;
    if (ksplit < 1) ksplit = 1;
    if (ksplit > steps) ksplit = steps;
    const int steps_per = (steps + ksplit - 1) / ksplit;
    p.kchunk = steps_per * KS;
    ksplit = (steps + steps_per - 1) / steps_per;
    bm = tile_rows(sh.B, bm);
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + bm - 1) / bm;
    const dim3 grid(grid_tiles(NB, sh.d / TILE_N), ksplit);
    return dispatch<false>(p, sh.quant, bm, grid, s);
}

}  // namespace moe
