// gemm_tiled.hip -- LDS-tiled grouped GEMMs for large sort blocks (B = 64, 128, 256).
//
// The compute-bound regime of the grouped GEMMs (many rows per expert, e.g.
// prefill): grouped GEMMs in place of masked dense GEMMs (rocketrecap.com/
// entries/19116, talk summary at 5:58), run as the two stages of the AITER
// walk-through (itsolotime.com/th/archives/32381, section 3.2).
//
// Workgroup tile: BM rows of one expert (BM = 64 or 128; a 256-row sort block
// runs as two tiles) x 256 weight rows (GEMM1: 128 gate rows + the 128
// matching up rows, so SwiGLU fuses into the epilogue; GEMM2: 256 output
// columns), K in steps of 128 bytes per row. 8 waves in a 2 x 4 arrangement,
// each owning (BM/2) x 64 of the tile, with v_mfma_f32_32x32x16_bf16 or, for
// e4m3, v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales (per-row /
// per-channel fp32 scales go in the epilogue).
//
// Operand staging: gfx950's global_load_lds_dwordx4 moves 16 bytes per lane
// from global memory straight into LDS (lane l's bytes land at M0 + 16 l), so
// no registers or LDS-store instructions carry the operands. Three LDS stages
// form a ring: while step j is multiplied out of one stage, the loads of
// steps j+1 and j+2 are in flight into the other two, one barrier per step.
// The loads are issued from inline assembly, with the vmcnt waits written out,
// because the compiler, which cannot tell the stages apart, would otherwise
// wait for every outstanding load at each barrier.
//
// Each 128-byte row segment is stored as 8 chunks of 16 bytes whose position
// is XOR-swizzled per row (see swz), so that a fragment read (32 rows, one
// chunk column) spreads over all banks; a load lane picks the global chunk
// that belongs at its fixed LDS position.
//
// Tile order: tiles are enumerated block-group-major (GM sort blocks x all
// column tiles), and workgroup i, which the hardware places on XCD i % 8,
// takes logical tile (i % 8) * ceil(tiles / 8) + i / 8. Neighbouring tiles,
// which share activation rows and weight rows, therefore run on the same XCD
// and share its L2. The tile count comes from num_valid on the device, so
// no XCD is left with the padding blocks.
//
// Epilogue: the tile's per-row metadata (destination token, routing weight,
// activation scale) is fetched into LDS before the K loop. GEMM1 writes the
// bf16 h tile into LDS and copies it out in 16-byte row segments (and, for
// e4m3, takes each row's amax there with one atomic per row and tile); GEMM2
// adds its weighted rows into the fp32 accumulator with atomics.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TILE_N = 256;     // weight rows per workgroup
constexpr int ROWB = 128;       // bytes per row per K step
constexpr int WAVES = 8;
constexpr int NTHR = 64 * WAVES;
constexpr int HROW = 272;       // bytes per row of the staged h tile (256 + 16 against bank conflicts)
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
constexpr int GROUP_M = MOE_GROUP_M;  // sort blocks per tile group
#ifndef MOE_TILED_SCHED
#define MOE_TILED_SCHED 0
#endif

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

// Chunk position of (row, chunk) inside the row's 128 bytes (an involution
// in chunk). A fragment read takes one chunk column of consecutive rows: any
// 8 consecutive rows land on 8 different positions (32-bank LDS, 8 lanes per
// cycle) and any 16 on 16 different (row parity, position) pairs (64 banks,
// 16 lanes per cycle).
__device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ (row & 7) ^ ((row >> 3) & 1);
}

// 32-bit LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)p;
}

// One wave-wide LDS DMA: lane l copies the 16 bytes at base + off into LDS
// bytes [m0 + 16 l, m0 + 16 l + 16). m0 must be wave-uniform. The s_nop
// covers the wait state an M0 write needs before an LDS DMA reads it.
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are pending
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
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

// BM: rows per tile (64 or 128). QUANT 0 (bf16) or 1 (e4m3, per-row
// activation scale and per-channel weight scale applied in the epilogue).
template <int QUANT, bool GEMM1, int BM>
__global__ __launch_bounds__(NTHR) void k_gemm_tiled(TiledParams p) {
    constexpr int ES = QUANT == 0 ? 2 : 1;
    constexpr int KS = ROWB / ES;               // K elements per step
    constexpr int ROWS = BM + TILE_N;           // LDS rows per stage (activations first)
    constexpr int BUF = ROWS * ROWB;            // bytes per stage
    constexpr int NQ = ROWS / 8 / WAVES;        // DMA instructions per wave per step
    constexpr int NQA = BM / 8 / WAVES;         // ... of which activation rows
    constexpr int RT = BM / 64;                 // 32-row tiles per wave
    constexpr int CT = 2;                       // 32-column tiles per wave
    constexpr int NBUF = BM >= 256 ? 2 : 3;     // LDS stages (160 KB of LDS per CU)
    static_assert(BM % (8 * WAVES) == 0, "tile rows");
    static_assert(BM * HROW <= NBUF * BUF, "h staging");
    __shared__ __attribute__((aligned(16))) uint8_t lds[NBUF * BUF];
    __shared__ __attribute__((aligned(16))) int row_tok[BM];     // token, or -1 for padding
    __shared__ __attribute__((aligned(16))) float row_scale[BM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // GEMM1 of the fused path clears GEMM2's accumulator on the way (at the
    // end, so that no stores are pending during the K loop)
    auto clear_zero = [&]() {
        if (!p.zero) return;
        const size_t nwg = (size_t)gridDim.x * gridDim.y;
        const size_t wg = blockIdx.x + (size_t)gridDim.x * blockIdx.y;
        float4 *z = reinterpret_cast<float4 *>(p.zero);
        for (size_t i = wg * NTHR + tid; i < p.zero_n / 4; i += nwg * NTHR)
            z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    };

    // ---- which tile -------------------------------------------------------
    const int ntiles = GEMM1 ? p.f / 128 : p.d / TILE_N;
    // tiles of BM rows; the sort block B is a multiple of BM, so a tile never
    // straddles two experts
    const int nblocks = *p.num_valid / BM;
    const int total = nblocks * ntiles;
    const int per_xcd = (total + 7) / 8;
    const int jx = blockIdx.x >> 3;
    const int logical = (blockIdx.x & 7) * per_xcd + jx;
    if (jx >= per_xcd || logical >= total) {
        clear_zero();
        return;
    }
    const int group = logical / (GROUP_M * ntiles);
    const int gm = min(GROUP_M, nblocks - group * GROUP_M);
    const int r = logical - group * GROUP_M * ntiles;
    const int nt = r / gm;
    const int blk = group * GROUP_M + r % gm;
    const int e = p.seid[blk * BM / p.B];
    const int sentinel = p.T * p.k;
    // a tile of padding only (the tail of a larger sort block)
    if (e < 0 || p.sorted_ids[blk * BM] >= sentinel) {
        clear_zero();
        return;
    }
    const int K = GEMM1 ? p.d : p.f;
    const int Ntot = GEMM1 ? 2 * p.f : p.d;
    const int slot0 = blk * BM;
    const int kbeg = blockIdx.y * p.kchunk;
    const int kend = min(K, kbeg + p.kchunk);

    // ---- per-row metadata for the epilogue ---------------------------------
    if (tid < BM) {
        const int slot = slot0 + tid;
        const int a = p.sorted_ids[slot];
        const bool ok = a < sentinel;
        row_tok[tid] = ok ? a / p.k : -1;
        float sc = 1.0f;
        if constexpr (GEMM1) {
            if constexpr (QUANT == 1) sc = ok ? p.a_scale[a / p.k] : 0.0f;
        } else {
            sc = ok ? p.sorted_w[slot] : 0.0f;
            if constexpr (QUANT == 1) sc *= p.a_scale[slot];
        }
        row_scale[tid] = sc;
    }
    const int lr = lane & 31, lh = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    // per-channel weight scales of this lane's columns (e4m3)
    float wsc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        wsc[ct] = 1.0f;
        if constexpr (QUANT == 1) {
            const int n = GEMM1 ? ct * p.f + nt * 128 + wn * 32 + lr : nt * TILE_N + wn * 64 + ct * 32 + lr;
            wsc[ct] = p.w_scale[(size_t)e * Ntot + n];
        }
    }

    // ---- LDS DMA sources -----------------------------------------------------
    // Instruction i of wave w fills stage rows 8 (w + 8 i) .. +7; lane l
    // writes row 8 (w + 8 i) + l / 8 at chunk position l % 8, which holds the
    // row's logical chunk swz(row, l % 8). 32-bit byte offsets from
    // wave-uniform bases keep the address registers few (the host guarantees
    // every operand matrix is below 4 GiB). Padding rows read token 0's row:
    // their products are never used (each output row depends on its own A row
    // only), and the epilogue writes zeros for them.
    const uint8_t *wexp = p.w + (size_t)e * Ntot * K * ES;
    uint32_t goff[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int row = 8 * (wave + WAVES * i) + (lane >> 3);
        const int chunk = swz(row, lane & 7);
        if (i < NQA) {
            int src;
            if constexpr (GEMM1) {
                const int a = p.sorted_ids[slot0 + row];
                src = a < sentinel ? a / p.k : 0;
            } else {
                src = slot0 + row;
            }
            goff[i] = (uint32_t)src * (uint32_t)(K * ES) + chunk * 16;
        } else {
            const int rb = row - BM;   // 0..255
            const int n = GEMM1 ? (rb < 128 ? 0 : p.f - 128) + nt * 128 + rb : nt * TILE_N + rb;
            goff[i] = (uint32_t)n * (uint32_t)(K * ES) + chunk * 16;
        }
    }
    const uint32_t m0w = lds_addr(lds) + (uint32_t)wave * 1024u;
    auto issue = [&](int buf, int kk) {
        const uint8_t *ab = p.a + (size_t)kk * ES;
        const uint8_t *bb = wexp + (size_t)kk * ES;
#pragma unroll
        for (int i = 0; i < NQ; ++i)
            dma16(i < NQA ? ab : bb, goff[i], m0w + (uint32_t)(buf * BUF + i * WAVES * 1024));
    };

    // ---- compute assignment -------------------------------------------------
    int arow[RT], brow[CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) arow[rt] = wm * (BM / 2) + rt * 32 + lr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        // GEMM1: tile 0 is gate rows, tile 1 the matching up rows
        brow[ct] = GEMM1 ? ct * 128 + wn * 32 + lr : wn * 64 + ct * 32 + lr;
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
    // 4s + 2lh + 1), all fragments read up front.
    auto compute = [&](int buf) {
        const uint8_t *base = lds + buf * BUF;
        if constexpr (QUANT == 0) {
            u32x4 fa0[RT], fb0[CT], fa1[RT], fb1[CT];
            frags_at(base, lh, fa0, fb0);
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
#if MOE_TILED_SCHED
            // reads of sub-step s+1 interleaved with the MFMAs of sub-step s
            __builtin_amdgcn_sched_group_barrier(0x100, RT + CT, 0);
#pragma unroll
            for (int i = 0; i < 3 * RT * CT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, RT * CT, 0);
#endif
        } else {
            u32x4 fa0[RT], fb0[CT], fa1[RT], fb1[CT];
            u32x4 ga0[RT], gb0[CT], ga1[RT], gb1[CT];
            frags_at(base, 2 * lh, fa0, fb0);
            frags_at(base, 2 * lh + 1, fa1, fb1);
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
#if MOE_TILED_SCHED
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RT + CT), 0);
#pragma unroll
            for (int i = 0; i < RT * CT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, RT * CT, 0);
#endif
        }
    };

    // ---- main loop -------------------------------------------------------
    // With S = NBUF stages, step j: issue the loads of step j+S-1 into stage
    // (j+S-1) % S (read during step j-1, which every wave has finished:
    // barrier), multiply stage j % S, wait for this wave's loads of step j+1,
    // barrier (so all of step j+1 has landed and stage j % S is free).
    // Unrolled by S so that the stage offsets are constants; loads past the
    // end are clamped to the last step, which keeps the wait counts exact and
    // lands in a stage nobody reads.
    const int nsteps = (kend - kbeg) / KS;
    if (nsteps > 0) {
        auto kof = [&](int i) { return kbeg + min(i, nsteps - 1) * KS; };
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) issue(b, kof(b));
        wait_vmem<NQ * (NBUF - 2)>();
        __syncthreads();
        auto step = [&](int j, int b) {
            issue((b + NBUF - 1) % NBUF, kof(j + NBUF - 1));
            compute(b);
            wait_vmem<NQ * (NBUF - 2)>();
            __syncthreads();
        };
        int j = 0;
        for (; j + NBUF <= nsteps; j += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) step(j + b, b);
        }
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b)
            if (j + b < nsteps) step(j + b, b);
    }
    wait_vmem<0>();
    __syncthreads();   // the clamped loads have landed; metadata is visible

    // ---- epilogue -----------------------------------------------------------
    // 32x32 accumulator layout: lane holds column (lane & 31) and rows
    // 8 * (v / 4) + 4 * (lane >> 5) + (v & 3), v = 0..15.
    if constexpr (GEMM1) {
        uint8_t *hs = lds;   // [BM][HROW] bf16 h tile
        const int hcol = wn * 32 + lr;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row0 = wm * (BM / 2) + rt * 32 + 8 * q + 4 * lh;
                const int4 tok4 = *reinterpret_cast<const int4 *>(&row_tok[row0]);
                float4 sc4 = make_float4(1.f, 1.f, 1.f, 1.f);
                if constexpr (QUANT == 1) sc4 = *reinterpret_cast<const float4 *>(&row_scale[row0]);
                const int tk[4] = {tok4.x, tok4.y, tok4.z, tok4.w};
                const float sx[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float g = acc[rt][0][4 * q + i], u = acc[rt][1][4 * q + i];
                    if constexpr (QUANT == 1) {
                        g = g * sx[i] * wsc[0];
                        u = u * sx[i] * wsc[1];
                    }
                    const uint16_t hb = tk[i] >= 0 ? f32_to_bf16_bits(silu(g) * u) : (uint16_t)0;
                    *reinterpret_cast<uint16_t *>(hs + (row0 + i) * HROW + hcol * 2) = hb;
                }
            }
        }
        __syncthreads();
        // 16 lanes per row, 16 bytes each: the tile's 256-byte row segments
        uint8_t *h = reinterpret_cast<uint8_t *>(p.out);
#pragma unroll
        for (int it = 0; it < BM * 16 / NTHR; ++it) {
            const int idx = tid + NTHR * it, row = idx >> 4, c = idx & 15;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(hs + row * HROW + c * 16);
            *reinterpret_cast<u32x4 *>(h + ((size_t)(slot0 + row) * p.f + nt * 128) * 2 + c * 16) = val;
            if constexpr (QUANT == 1) {
                float m = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(val[w] & 0xffffu)));
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(val[w] >> 16)));
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                if (c == 0) atomic_max_nonneg(p.out_scale + slot0 + row, m);
            }
        }
    } else {
        float *accg = reinterpret_cast<float *>(p.out);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row0 = wm * (BM / 2) + rt * 32 + 8 * q + 4 * lh;
                const int4 tok4 = *reinterpret_cast<const int4 *>(&row_tok[row0]);
                const float4 sc4 = *reinterpret_cast<const float4 *>(&row_scale[row0]);
                const int tk[4] = {tok4.x, tok4.y, tok4.z, tok4.w};
                const float sw[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (tk[i] < 0) continue;
                    float *dst = accg + (size_t)tk[i] * p.d + nt * TILE_N + wn * 64 + lr;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        atomic_add_f32(dst + ct * 32, sw[i] * (acc[rt][ct][4 * q + i] * wsc[ct]));
                }
            }
        }
    }
    clear_zero();
}

template <int QUANT, bool GEMM1>
hipError_t dispatch_bm(const TiledParams &p, int BM, dim3 grid, hipStream_t s) {
    if (BM == 64)
        k_gemm_tiled<QUANT, GEMM1, 64><<<grid, NTHR, 0, s>>>(p);
    else if (BM == 128)
        k_gemm_tiled<QUANT, GEMM1, 128><<<grid, NTHR, 0, s>>>(p);
    else if (QUANT == 0 && BM == 256)
        k_gemm_tiled<0, GEMM1, 256><<<grid, NTHR, 0, s>>>(p);
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

// Rows per kernel tile: 64, 128 or (bf16) 256, a divisor of the sort block
// B; other values pick min(B, 128).
int tile_rows(int B, int bm, int quant) {
    const int maxbm = quant == 0 ? 256 : 128;
    if (bm <= 0 || bm > B || B % bm || bm > maxbm) bm = B < 128 ? B : 128;
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
    bm = tile_rows(sh.B, bm, sh.quant);
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
    bm = tile_rows(sh.B, bm, sh.quant);
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + bm - 1) / bm;
    const dim3 grid(grid_tiles(NB, sh.d / TILE_N), ksplit);
    return dispatch<false>(p, sh.quant, bm, grid, s);
}

}  // namespace moe
