// gemm_tiled.hip -- LDS-tiled grouped GEMMs for large sort blocks (B = 64, 128, 256).
//
// The compute-bound regime of the grouped GEMMs (many rows per expert, e.g.
// prefill): grouped GEMMs in place of masked dense GEMMs (rocketrecap.com/
// entries/19116, talk summary at 5:58), run as the two stages of the AITER
// walk-through (itsolotime.com/th/archives/32381, section 3.2).
//
// Workgroup tile: BM rows of one expert (BM = 64, 128 or 256, a divisor of
// the sort block) x TN weight rows (TN = 256, or 128 for 256-row tiles;
// GEMM1 takes TN/2 gate rows and the TN/2 matching up rows, so SwiGLU fuses
// into the epilogue; GEMM2 takes TN output columns), K in steps of 128 bytes
// per row. 8 waves in a WM x WN grid (WN = TN/64), each owning (BM/WM) x 64
// of the tile as 32x32 accumulators, with v_mfma_f32_32x32x16_bf16 or, for
// e4m3, v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales (per-row /
// per-channel fp32 scales go in the epilogue). Waves whose rows are all
// padding skip their MFMAs.
//
// Operand staging: gfx950's global_load_lds_dwordx4 moves 16 bytes per lane
// from global memory straight into LDS (lane l's bytes land at M0 + 16 l), so
// no registers or LDS-store instructions carry the operands; activation rows
// go through the buffer form, whose range check lets padding rows read
// nothing. Three LDS stages (two for 256 x 256 tiles) form a ring: while step
// j is multiplied out of one stage, the loads of the next steps are in
// flight into the others, one barrier per step.
// The loads are issued from inline assembly, with the vmcnt waits written out,
// because the compiler, which cannot tell the stages apart, would otherwise
// wait for every outstanding load at each barrier.
//
// Each 128-byte row segment is stored as 8 chunks of 16 bytes whose position
// is XOR-swizzled per row (see swz), so that a fragment read (32 rows, one
// chunk column) spreads over all banks; a load lane picks the global chunk
// that belongs at its fixed LDS position.
//
// Tile order: workgroup i, which the hardware places on XCD i % 8, takes
// logical tile (i % 8) * ceil(tiles / 8) + i / 8, so every XCD works through
// one contiguous range of logical tiles and neighbouring tiles share its L2.
// Logical tiles go strip by strip: a strip is S consecutive column tiles
// (S = 4 for GEMM1, 2 for GEMM2) times every sort block, with the strip's
// column tiles innermost. An XCD's range is then a band of the weight
// columns over all blocks, and the tiles running at once on it share a few
// weight column tiles and each activation block across S of them. Against
// the block-group order (8 sort blocks x all column tiles, kept as the
// alternative for S = 0), this cut the layer time by 2.5 % (bf16, T = 4096)
// to 6 % (MXFP4, T = 4096) and up to 9 % at T = 1024..2048, where an XCD's
// in-flight tiles otherwise re-fetch the same activation blocks from beyond
// L2 round after round. The tile count comes from num_valid on the device,
// so no XCD is left with the padding blocks.
//
// Epilogue: the tile's per-row metadata (assignment, routing weight,
// activation scale) is loaded before the K loop and kept in registers until
// after it. GEMM1 writes the bf16 h tile into LDS and copies its real rows
// out in 16-byte row segments (and, for e4m3, takes each row's amax there
// with one atomic per row and tile). GEMM2 either stores its weighted rows at
// their K part and assignment (a combine kernel sums each token's rows) or
// adds them into the token's fp32 accumulator row with atomics.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
// column tiles per strip of the tile order (0: block-group order)
#ifndef MOE_TILED_STRIP1
#define MOE_TILED_STRIP1 4
#endif
#ifndef MOE_TILED_STRIP2
#define MOE_TILED_STRIP2 2
#endif
// 1: raise the wave's priority while it issues a sub-step's MFMAs (bf16)
#ifndef MOE_TILED_PRIO
#define MOE_TILED_PRIO 0
#endif
constexpr int GROUP_M = MOE_GROUP_M;  // sort blocks per tile group (block-group order)
constexpr int ROWB = 128;       // bytes per row per K step
// K rotation: bit 2q for GEMM1 of quant q, bit 2q+1 for GEMM2
#ifndef MOE_TILED_ROTATE
#define MOE_TILED_ROTATE 0xC
#endif
constexpr int CH = ROWB / 16;   // 16-byte chunks per row segment
// bytes per row per K step for 128- and 256-row tiles

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
    int rotate;     // start each tile's K loop at a step that depends on its column tile
    int strip;      // > 0: column-strip tile order with strips of this many column tiles
    float *zero;
    size_t zero_n;
    float *yrows;   // GEMM2 without K-split: weighted rows [T*k, d] by assignment, stored (no atomics)
    // quant 3 (MXFP4): E8M0 scales of A [rows, K/32] and of the weights
    // [E, N, K/32]; GEMM1 writes h's [P, f/32]
    const uint8_t *a_mx, *w_mx;
    uint8_t *out_mx;
    // GEMM1, bf16 only: when set, the raw gate / up sums of the real rows go
    // to raw_out [P, 2f] fp32 (gate at column n, up at f + n) and no h is
    // written (the backward's recompute of the forward sums, and its
    // v = Wd^T dy with Wd^T split into two halves)
    float *raw_out;
    // rows of the activation operand a (tokens for GEMM1, sort slots for
    // GEMM2): the range its buffer descriptor allows
    uint32_t a_rows;
};

// Chunk position of (row, chunk) inside the row's 128 bytes (an involution
// in chunk). A fragment read takes one chunk column of 16 consecutive rows
// per LDS cycle (64 banks of 4 bytes = 16 chunks), which land on 16
// different (row parity, position) pairs.
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
// M0 is listed as clobbered although the compiler reserves it: nothing else
// in these kernels reads M0 (no other LDS DMA, message or relative-move
// instruction; checked in the generated assembly), so the warning is
// silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}
// The same through a buffer descriptor (raw, stride 0): a lane whose offset
// lies past the descriptor's num_records reads nothing from memory and
// writes zeros to its 16 LDS bytes, which is how padding rows skip their
// traffic while every lane still issues the instruction (the wait counts
// stay fixed).
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(rsrc), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Buffer descriptor of n bytes from base: stride 0, no swizzle, the data
// format the gfx9 family takes for untyped dword loads.
__device__ __forceinline__ i32x4 buf_rsrc(const void *base, uint32_t n) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = 0x00020000;
    return r;
}
// offset of a lane that must read nothing (past any num_records: operand
// matrices are below 4 GiB and whole 128-byte rows)
constexpr uint32_t DMA_SKIP = 0xFFFFFFF0u;

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

// E2M1 x E2M1 over K = 64 (16 bytes per lane: one LDS chunk, which is one
// 32-element MX block) with the lanes' E8M0 scales in byte OPSEL of xa / xb.
template <int OPSEL>
__device__ __forceinline__ f32x16 mma32_fp4(const u32x4 &a, const u32x4 &b, uint32_t xa, uint32_t xb,
                                            f32x16 acc) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, OPSEL, (int)xa, OPSEL, (int)xb);
}

// BM: rows per tile (64, 128 or 256); TN: weight rows per tile (256, or 128
// for 256-row tiles; GEMM1 takes TN/2 gate rows and the TN/2 matching up
// rows). QUANT 0 (bf16) or 1 (e4m3, per-row activation scale and
// per-channel weight scale applied in the epilogue). The 8 waves form a
// WM x WN grid, each wave owning (BM / WM) rows x 64 weight rows.
// BT (bf16 only): the weights are stored [K][N] (N contiguous) instead of
// [N][K]: the backward's products with Wd^T and W13^T read the forward's
// weights in place. A stage then holds the tile's 64 K rows of TN columns
// (TN * 2 bytes each, 16-byte chunk c of K row r at position
// c ^ 4 (r % 4)) and the MFMA B fragments come from two transposing reads
// ds_read_tr16_b64 each: within a 16-lane group, lane 4j + q points at
// K row k0 + j and columns c0 + 4q .. c0 + 4q + 3, and lane i receives K rows
// k0 .. k0 + 3 of column c0 + i. The four K rows a half-wave reads then sit
// in four different 64-byte bank groups.
template <int QUANT, bool GEMM1, int BM, int TN, int WAVES, bool BT = false>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_tiled(TiledParams p) {
    static_assert(!BT || QUANT == 0, "weights stored [K][N] are bf16 only");
    constexpr int NTHR = 64 * WAVES;
    constexpr bool MX = QUANT == 3;             // MXFP4: E2M1 two per byte, E8M0 per 32
    auto eb = [](size_t n) -> size_t { return QUANT == 0 ? 2 * n : (MX ? n / 2 : n); };  // bytes of n elements
    constexpr int KS = QUANT == 0 ? 64 : (MX ? 256 : 128);  // K elements per 128-byte step
    constexpr int ROWS = BM + TN;               // LDS rows per stage (activations first)
    constexpr int BUF = ROWS * ROWB;            // bytes per stage
    constexpr int NQ = BUF / 1024 / WAVES;      // DMA instructions per wave per step
    constexpr int NQA = BM * ROWB / 1024 / WAVES;  // ... of which activation rows
    constexpr int WN = TN / 64, WM = WAVES / WN;
    constexpr int RT = BM / WM / 32;            // 32-row tiles per wave
    constexpr int CT = 2;                       // 32-column tiles per wave
    // LDS stages (of 160 KB of LDS)
    constexpr int NBUF = BUF <= 48 * 1024 ? 3 : 2;
    // MXFP4 scales: per pair of K steps, 16 bytes per tile row (8 per step),
    // in two slots after the stages
    constexpr int SSLOT = MX ? ROWS * 16 : 0;
    constexpr int HROW = TN + 16;               // bytes per row of the staged h tile (+16 against bank conflicts)
    static_assert(BM % (8 * WAVES) == 0 && TN % 64 == 0 && RT >= 1 && BM <= NTHR, "tile shape");
    static_assert(BM * HROW <= NBUF * BUF, "h staging");
    static_assert(!MX || ROWS <= NTHR, "one scale row per thread");
    __shared__ __attribute__((aligned(16))) uint8_t lds[NBUF * BUF + 2 * SSLOT];
    __shared__ __attribute__((aligned(16))) int row_asg[BM];     // assignment t*k+j, or -1 for padding
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
    const int ntiles = GEMM1 ? p.f / (TN / 2) : p.d / TN;
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
    int nt, blk;
    if (p.strip > 0) {
        // strips of p.strip column tiles x every block, the strip's column
        // tiles innermost
        const int strip = logical / (p.strip * nblocks);
        const int gn = min(p.strip, ntiles - strip * p.strip);
        const int r = logical - strip * p.strip * nblocks;
        blk = r / gn;
        nt = strip * p.strip + r % gn;
    } else {
        const int group = logical / (GROUP_M * ntiles);
        const int gm = min(GROUP_M, nblocks - group * GROUP_M);
        const int r = logical - group * GROUP_M * ntiles;
        nt = r / gm;
        blk = group * GROUP_M + r % gm;
    }
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

    // ---- prologue ------------------------------------------------------------
    // Order matters: the compiler waits for its own loads with vmcnt counts
    // that know nothing of the DMA, so every load whose result is used before
    // the K loop is issued first; the weight DMA (which needs only the
    // expert) goes out while they are in flight; the activation DMA, whose
    // row addresses need the sorted ids, comes last, so that the K loop's
    // wait counts cover exactly the DMA. Epilogue metadata stays in registers
    // until after the K loop.
    const int lr = lane & 31, lh = lane >> 5;
    // waves w and w + 4 share a SIMD: they get the same columns and row
    // blocks BM/2 apart, so that when the second half of a tile is padding
    // (whose MFMAs are skipped) every SIMD still has one busy wave
    const int wn = wave % WN, wm = wave / WN;
    const uint8_t *wexp = p.w + eb((size_t)e * Ntot * K);
    const uint32_t kbytes = (uint32_t)eb(K);

    // Instruction i of wave w fills the stage's kilobyte w + 8 i, i.e. 8
    // rows; lane l writes row 8 (w + 8 i) + l / 8 at chunk position l % 8,
    // which holds the row's logical chunk swz(row, l % 8). 32-bit byte
    // offsets from wave-uniform bases keep the address registers few (the
    // host guarantees every operand matrix is below 4 GiB). Padding rows read
    // token 0's row: their products are never used (each output row depends
    // on its own A row only), and the epilogue writes zeros for them.
    int arow_src[NQA];
#pragma unroll
    for (int i = 0; i < NQA; ++i) {
        const int row = 8 * (wave + WAVES * i) + (lane >> 3);
        arow_src[i] = p.sorted_ids[slot0 + row];   // the assignment, or padding (>= sentinel)
    }
    // MXFP4 scale rows: wave w copies tile rows 64 w .. 64 w + 63 (all
    // activation rows or all weight rows, BM being a multiple of 64), lane l
    // row 64 w + l, 16 bytes (a pair of K steps) at a time
    const bool xwave = MX && 64 * wave < ROWS;
    const bool xwave_a = 64 * wave < BM;
    int xsrc = 0;
    if constexpr (MX) {
        const int row = 64 * wave + lane;
        if (xwave_a) {
            xsrc = GEMM1 ? p.sorted_ids[slot0 + row] : slot0 + row;
        } else {
            const int rb = row - BM;
            xsrc = GEMM1 ? (rb < TN / 2 ? 0 : p.f - TN / 2) + nt * (TN / 2) + rb : nt * TN + rb;
        }
    }
    // live 32-row groups of the tile: padding sits at the end of the
    // expert's segment, so they form a prefix (bit g: row 32 g is real)
    const uint64_t live32 =
        __ballot(lane < BM / 32 && p.sorted_ids[slot0 + 32 * min(lane, BM / 32 - 1)] < sentinel);
    int meta_a = sentinel;
    float meta_w = 0.0f, meta_s = 1.0f;
    if (tid < BM) {
        meta_a = p.sorted_ids[slot0 + tid];
        if constexpr (!GEMM1) {
            meta_w = p.sorted_w ? p.sorted_w[slot0 + tid] : 1.0f;
            if constexpr (QUANT == 1) meta_s = p.a_scale[slot0 + tid];
        }
    }
    // per-channel weight scales of this lane's columns (e4m3)
    float wsc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        wsc[ct] = 1.0f;
        if constexpr (QUANT == 1) {
            const int n = GEMM1 ? ct * p.f + nt * (TN / 2) + wn * 32 + lr : nt * TN + wn * 64 + ct * 32 + lr;
            wsc[ct] = p.w_scale[(size_t)e * Ntot + n];
        }
    }

    uint32_t goff[NQ];
#pragma unroll
    for (int i = NQA; i < NQ; ++i) {
        if constexpr (BT) {
            // instruction i fills K rows 2q and 2q + 1 of the B region
            // (q = its kilobyte there); lane l: K row 2q + l / 32, chunk
            // position l % 32, which holds the row's logical 8-column chunk
            // (l % 32) ^ 4 (K row % 4)
            const int q = wave + WAVES * (i - NQA);
            const int kr = 2 * q + (lane >> 5);
            const int lc = 8 * ((lane & 31) ^ ((kr & 3) << 2));   // column in the tile, 0..TN-1
            const int n = GEMM1 ? (lc < TN / 2 ? 0 : p.f - TN / 2) + nt * (TN / 2) + lc : nt * TN + lc;
            goff[i] = (uint32_t)kr * (uint32_t)(Ntot * 2) + (uint32_t)n * 2;
        } else {
            const int row = 8 * (wave + WAVES * i) + (lane >> 3);
            const int rb = row - BM;   // 0..TN-1
            const int n = GEMM1 ? (rb < TN / 2 ? 0 : p.f - TN / 2) + nt * (TN / 2) + rb : nt * TN + rb;
            goff[i] = (uint32_t)n * kbytes + swz(row, lane & 7) * 16;
        }
    }
    const uint32_t m0w = lds_addr(lds) + (uint32_t)wave * 1024u;
    // MXFP4 scale copies: pair q of K steps (steps 2q, 2q + 1 of this K
    // range) into slot q % 2
    const uint8_t *xbase = MX ? (xwave_a ? p.a_mx : p.w_mx + (size_t)e * Ntot * (K / 32)) : nullptr;
    uint32_t xoff = 0;
    auto issue_scales = [&](int q) {
        if constexpr (MX) {
            if (xwave)
                dma16(xbase, xoff + (uint32_t)(kbeg / 32 + 16 * q),
                      lds_addr(lds) + (uint32_t)(NBUF * BUF + (q & 1) * SSLOT) + (uint32_t)wave * 1024u);
        }
    };
    const uint32_t abytes = p.a_rows * kbytes;
    auto issue_part = [&](int buf, int kk, int i0, int i1) {
        // activation rows through a descriptor of the bytes from column kk on
        const uint32_t ak = (uint32_t)eb(kk);
        const i32x4 ar = buf_rsrc(p.a + ak, abytes - ak);
        // [N][K] weights advance along the row, [K][N] weights by kk rows
        const uint8_t *bb = BT ? wexp + (size_t)kk * Ntot * 2 : wexp + eb(kk);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            if (i < i0 || i >= i1) continue;
            const uint32_t m0 = m0w + (uint32_t)(buf * BUF + i * WAVES * 1024);
            if (i < NQA)
                dma16_buf(ar, goff[i], m0);
            else
                dma16(bb, goff[i], m0);
        }
    };
    static_assert(NBUF <= 3, "the first K step's wait count assumes at most 3 stages");
    const int nsteps = (kend - kbeg) / KS;
    // K steps in the order rot, rot+1, ..., nsteps-1, 0, ..., rot-1: tiles of
    // different column tiles then read different 128-byte columns of their
    // weight rows at any moment, which spreads the HBM traffic over channels
    // and banks (rows a power of two apart otherwise meet in the same ones).
    // Tiles of one column tile keep the same order, so the sort blocks of an
    // expert still share each weight step in L2.
    const int rot = (p.rotate && nsteps > 0 && !MX) ? nt % nsteps : 0;
    auto kof = [&](int i) {
        int st = min(i, nsteps - 1) + rot;
        if (st >= nsteps) st -= nsteps;
        return kbeg + st * KS;
    };
    // weight rows of the first NBUF-1 steps
    if (nsteps > 0) {
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) issue_part(b, kof(b), NQA, NQ);
    }
    // activation rows (the compiler's wait for the sorted ids is here);
    // padding rows read nothing and land as zeros
#pragma unroll
    for (int i = 0; i < NQA; ++i) {
        const int row = 8 * (wave + WAVES * i) + (lane >> 3);
        const int src = GEMM1 ? arow_src[i] / p.k : slot0 + row;
        goff[i] = arow_src[i] < sentinel ? (uint32_t)src * kbytes + swz(row, lane & 7) * 16 : DMA_SKIP;
    }
    if constexpr (MX) {
        int src = xsrc;
        if (GEMM1 && xwave_a) src = src < sentinel ? src / p.k : 0;
        xoff = (uint32_t)src * (uint32_t)(K / 32);
    }
    const bool meta_ok = meta_a < sentinel;
    const int meta_asg = meta_ok ? meta_a : -1;
    if constexpr (GEMM1) {
        if constexpr (QUANT == 1) meta_s = meta_ok ? p.a_scale[meta_a / p.k] : 0.0f;
    } else {
        meta_s = meta_ok ? meta_w * meta_s : 0.0f;
    }

    // ---- compute assignment -------------------------------------------------
    int arow[RT], brow[CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) arow[rt] = wm * (BM / WM) + rt * 32 + lr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        // GEMM1: tile 0 is gate rows, tile 1 the matching up rows
        brow[ct] = GEMM1 ? ct * (TN / 2) + wn * 32 + lr : wn * 64 + ct * 32 + lr;
    }
    // the wave's rows hold no assignment (padding is at the end of each
    // expert's segment, so the first row decides): skip its MFMAs
    const bool wave_live = (live32 >> (wm * (BM / WM) / 32)) & 1;
    f32x16 acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0.0f;

    // (weight fragments first: a sub-step's first MFMA takes fb[0] and fa[0],
    // and the activation fragments follow in the order the MFMAs take them)
    auto frags_at = [&](const uint8_t *base, int chunk, u32x4 (&fa)[RT], u32x4 (&fb)[CT]) {
        if constexpr (BT) {
            // K rows 8 chunk .. 8 chunk + 7 of column brow[ct]: two transposing
            // reads of four K rows each (the lane's 16-lane group starts at
            // column brow[ct] - lane % 16)
            const uint32_t bbase = lds_addr(base) + (uint32_t)(BM * ROWB);
            const int li = lane & 15, tj = li >> 2, tq = li & 3;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int col = brow[ct] - li + 4 * tq;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = 8 * chunk + 4 * hh + tj;
                    const int pos = (col >> 3) ^ ((kr & 3) << 2);
                    const uint32_t addr = bbase + (uint32_t)(kr * (TN * 2) + pos * 16 + (col & 7) * 2);
                    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)addr);
                    fb[ct][2 * hh] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                    fb[ct][2 * hh + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
                }
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                fb[ct] = *reinterpret_cast<const u32x4 *>(base + (BM + brow[ct]) * ROWB +
                                                          swz(brow[ct], chunk) * 16);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            fa[rt] = *reinterpret_cast<const u32x4 *>(base + arow[rt] * ROWB + swz(arow[rt], chunk) * 16);
    };
    // bf16: CH/2 sub-steps of K = 16 (lane half lh takes chunk 2s + lh); the
    // fragments of sub-step s+1 are read while the MFMAs of sub-step s run.
    // e4m3: CH/4 sub-steps of K = 64 (lane half lh takes chunks 4s + 2lh and
    // 4s + 2lh + 1); the second sub-step's fragments are read between the
    // first one's MFMAs (two reads after each).
    // MXFP4: 4 sub-steps of K = 64; lane half lh takes chunk 4 lh + s, i.e.
    // MX block 4 lh + s of the step, so the lane's four E8M0 scales of the
    // step are one dword of the scale row (byte s for sub-step s): dword
    // 2 (j % 2) + lh of the row's 16 bytes in slot (j / 2) % 2, read once per
    // step together with the first sub-step's fragments.
    // bf16 and MXFP4: the instruction order of a sub-step that also reads the next
    // sub-step's fragments: one LDS read after each of the first MFMAs, so
    // the reads' latency hides behind them. Left to itself the compiler
    // reuses one set of fragment registers and waits for each read right
    // before the MFMA that needs it. The pattern applies to the code since
    // the last sched_barrier, which closes it: MFMAs do not move across
    // sub-steps, where the same accumulators would form dependent chains.
    constexpr int NRD = RT + (BT ? 2 : 1) * CT;   // LDS reads of one sub-step's fragments
    auto interleave = [&]() {
        constexpr int PAIRS = NRD < RT * CT ? NRD : RT * CT;
#pragma unroll
        for (int i = 0; i < PAIRS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, RT * CT - PAIRS, 0);
        if constexpr (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](int buf, int j, int par) {
        if (!wave_live) return;
        const uint8_t *base = lds + buf * BUF;
        if constexpr (MX) {
            // the first sub-step's fragments and the step's scale dwords
            // (dword 2 (j % 2) + lh of each row's 16 bytes in slot (j / 2) % 2),
            // all in flight together, in the order the first MFMAs take them
            // (weight column tile 0 and its scale, activation row tile 0 and
            // its scale, then the others: the first MFMA waits for four reads)
            u32x4 fa[2][RT], fb[2][CT];
            const uint8_t *sb = lds + NBUF * BUF + ((j >> 1) & 1) * SSLOT + (2 * (j & 1) + lh) * 4;
            uint32_t xa[RT], xb[CT];
            auto read_a = [&](int rt) {
                fa[0][rt] = *reinterpret_cast<const u32x4 *>(base + arow[rt] * ROWB + swz(arow[rt], 4 * lh) * 16);
                xa[rt] = *reinterpret_cast<const uint32_t *>(sb + arow[rt] * 16);
            };
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                fb[0][ct] = *reinterpret_cast<const u32x4 *>(base + (BM + brow[ct]) * ROWB +
                                                             swz(brow[ct], 4 * lh) * 16);
                xb[ct] = *reinterpret_cast<const uint32_t *>(sb + (BM + brow[ct]) * 16);
                if (ct == 0) read_a(0);
            }
#pragma unroll
            for (int rt = 1; rt < RT; ++rt) read_a(rt);
            __builtin_amdgcn_sched_barrier(0);
            static_for<4>([&](auto sc) {
                constexpr int sub = decltype(sc)::value;
                if constexpr (sub + 1 < 4) frags_at(base, 4 * lh + sub + 1, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        acc[rt][ct] = mma32_fp4<sub>(fa[sub & 1][rt], fb[sub & 1][ct], xa[rt], xb[ct], acc[rt][ct]);
                interleave();
            });
        } else if constexpr (QUANT == 0) {
            constexpr int NSUB = CH / 2;
            u32x4 fa[2][RT], fb[2][CT];
            frags_at(base, lh, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
                if (sub + 1 < NSUB) frags_at(base, 2 * (sub + 1) + lh, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
                if constexpr (MOE_TILED_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        acc[rt][ct] = mma32_bf16(fa[sub & 1][rt], fb[sub & 1][ct], acc[rt][ct]);
                if constexpr (MOE_TILED_PRIO) __builtin_amdgcn_s_setprio(0);
                interleave();
            }
        } else {
            constexpr int NSUB = CH / 4;
            u32x4 fa[NSUB][2][RT], fb[NSUB][2][CT];
            // one sub-step's fragments (two chunks per row tile) in the order
            // its MFMAs take them: weight column tile 0, activation row tile
            // 0, then the others
            auto read_sub = [&](int sub) {
                const int c0 = 4 * sub + 2 * lh;
                auto read_a = [&](int rt) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        fa[sub][h][rt] = *reinterpret_cast<const u32x4 *>(base + arow[rt] * ROWB +
                                                                          swz(arow[rt], c0 + h) * 16);
                };
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        fb[sub][h][ct] = *reinterpret_cast<const u32x4 *>(base + (BM + brow[ct]) * ROWB +
                                                                          swz(brow[ct], c0 + h) * 16);
                    if (ct == 0) read_a(0);
                }
#pragma unroll
                for (int rt = 1; rt < RT; ++rt) read_a(rt);
            };
            // the next sub-step's reads go out between this one's MFMAs
            read_sub(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
                if (sub + 1 < NSUB) read_sub(sub + 1);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        acc[rt][ct] = mma32_fp8(fa[sub][0][rt], fa[sub][1][rt], fb[sub][0][ct],
                                                fb[sub][1][ct], acc[rt][ct]);
                if (sub + 1 < NSUB) {
                    constexpr int NR = 2 * (RT + CT), NM = RT * CT;
#pragma unroll
                    for (int i = 0; i < NM; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, NR / NM, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- main loop -------------------------------------------------------
    // With S = NBUF stages, step j: issue the loads of step j+S-1 into stage
    // (j+S-1) % S (read during step j-1, which every wave has finished:
    // barrier), multiply stage j % S, wait for this wave's loads of step j+1,
    // barrier (so all of step j+1 has landed and stage j % S is free).
    // Unrolled by S (MXFP4 with three stages: by 6, so that the stage and the
    // parity of the step are both constants) so that the stage offsets and
    // wait counts are constants; loads past the end are clamped to the last
    // step, which keeps the wait counts exact and lands in a stage nobody
    // reads. MXFP4 scale pairs go out with the loads of their first (even)
    // step, so a step's wait allows one more outstanding load after an
    // issue of scales (waves that copy scale rows only).
    // Activation load i of every wave covers rows [64 i, 64 i + 64) of the
    // tile, so only the first NQAL = ceil(real rows / 64) of them carry real
    // rows; the others are not issued. Their LDS rows keep stale bytes, which
    // reach only the accumulators of padding rows (never stored). The loop
    // is instantiated per NQAL so that every wait count stays a constant.
    auto kloop = [&](auto nqal_c) {
        constexpr int NQAL = decltype(nqal_c)::value;
        constexpr int NQL = NQAL + (NQ - NQA);   // loads per wave per step
        constexpr int UNR = (MX && NBUF % 2) ? 2 * NBUF : NBUF;
        if (nsteps <= 0) return;
        // scales of the first pair before the activation rows, which the
        // first wait leaves outstanding
        issue_scales(0);
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) issue_part(b, kof(b), 0, NQAL);
        // stage 0 has landed once only the activation rows of the later
        // prologue stages are pending (everything older has completed)
        wait_vmem<NQAL * (NBUF - 2)>();
        __syncthreads();
        // b: position in the unrolled group (the group starts at an even step)
        auto step = [&](int j, auto bc) {
            constexpr int b = decltype(bc)::value;
            constexpr int nb = (b + NBUF - 1) % NBUF;
            // MXFP4 (even step count, no rotation): the issued step is even
            constexpr bool SC = MX && (b + NBUF - 1) % 2 == 0;
            const int jj = j + NBUF - 1, kk = kof(jj);
            issue_part(nb, kk, 0, NQAL);
            issue_part(nb, kk, NQA, NQ);
            const bool sc = SC && jj < nsteps;
            if (sc) issue_scales(jj / 2);
            compute(b % NBUF, j, b % 2);
            if (NBUF > 2 && sc && xwave)
                wait_vmem<(NQL + 1) * (NBUF - 2)>();
            else
                wait_vmem<NQL * (NBUF - 2)>();
            __syncthreads();
        };
        int j = 0;
        for (; j + UNR <= nsteps; j += UNR)
            static_for<UNR>([&](auto bc) { step(j + decltype(bc)::value, bc); });
        static_for<UNR - 1>([&](auto bc) {
            if (j + decltype(bc)::value < nsteps) step(j + decltype(bc)::value, bc);
        });
    };
    const int nqal = min(NQA, (__popcll(live32) + 1) / 2);
    static_for<NQA>([&](auto ic) {
        if (nqal == decltype(ic)::value + 1) kloop(IC<decltype(ic)::value + 1>{});
    });
    if (tid < BM) {
        row_asg[tid] = meta_asg;
        row_scale[tid] = meta_s;
    }
    wait_vmem<0>();
    __syncthreads();   // the clamped loads have landed; metadata is visible

    // ---- epilogue -----------------------------------------------------------
    // 32x32 accumulator layout: lane holds column (lane & 31) and rows
    // 8 * (v / 4) + 4 * (lane >> 5) + (v & 3), v = 0..15.
    if constexpr (GEMM1 && QUANT == 0) {
        if (p.raw_out) {
            const size_t f2 = 2 * (size_t)p.f;
            const int col = nt * (TN / 2) + wn * 32 + lr;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * (BM / WM) + rt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    if (row_asg[row] < 0) continue;
                    float *dst = p.raw_out + (size_t)(slot0 + row) * f2 + col;
                    dst[0] = acc[rt][0][v];
                    dst[p.f] = acc[rt][1][v];
                }
            clear_zero();
            return;
        }
    }
    if constexpr (GEMM1) {
        uint8_t *hs = lds;   // [BM][HROW] bf16 h tile
        const int hcol = wn * 32 + lr;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row0 = wm * (BM / WM) + rt * 32 + 8 * q + 4 * lh;
                const int4 tok4 = *reinterpret_cast<const int4 *>(&row_asg[row0]);
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
        uint8_t *h = reinterpret_cast<uint8_t *>(p.out);
        if constexpr (MX) {
            // one thread per (row, 32-column MX block): the block's amax
            // gives its E8M0 scale, the codes go out as 16 bytes
            constexpr int NBK = TN / 2 / 32;
            for (int idx = tid; idx < BM * NBK; idx += NTHR) {
                const int row = idx / NBK, bk = idx % NBK;
                if (row_asg[row] < 0) continue;
                float v[32];
                float m = 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 q = *reinterpret_cast<const u32x4 *>(hs + row * HROW + bk * 64 + c * 16);
                    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[8 * c + 2 * i] = bf16_bits_to_f32(w4[i] & 0xffffu);
                        v[8 * c + 2 * i + 1] = bf16_bits_to_f32(w4[i] >> 16);
                    }
                }
#pragma unroll
                for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
                const int E = mx_block_exp(m);
                const float inv = mx_inv_scale(E);
                uint32_t cw[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float sv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) sv[i] = v[8 * c + i] * inv;
                    cw[c] = e2m1_pack8(sv);
                }
                const size_t slot = (size_t)slot0 + row;
                const int col0 = nt * (TN / 2) + bk * 32;
                *reinterpret_cast<u32x4 *>(h + slot * (p.f / 2) + col0 / 2) = u32x4{cw[0], cw[1], cw[2], cw[3]};
                p.out_mx[slot * (p.f / 32) + col0 / 32] = (uint8_t)(E + 127);
            }
            clear_zero();
            return;
        }
        // TN/16 lanes per row, 16 bytes each: the tile's TN-byte row segments
        constexpr int RC = TN / 16;
#pragma unroll
        for (int it = 0; it < BM * RC / NTHR; ++it) {
            const int idx = tid + NTHR * it, row = idx / RC, c = idx % RC;
            // padding rows are not stored (their h rows are unspecified); a
            // row's RC lanes are consecutive, so they skip together
            if (row_asg[row] < 0) continue;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(hs + row * HROW + c * 16);
            *reinterpret_cast<u32x4 *>(h + ((size_t)(slot0 + row) * p.f + nt * (TN / 2)) * 2 + c * 16) = val;
            if constexpr (QUANT == 1) {
                float m = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(val[w] & 0xffffu)));
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(val[w] >> 16)));
                }
#pragma unroll
                for (int o = 1; o < RC; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                if (c == 0) atomic_max_nonneg(p.out_scale + slot0 + row, m);
            }
        }
    } else {
        // rows weighted by routing weight (and activation scale); with
        // yrows each row is stored at its assignment, else added atomically
        // into the token's accumulator row
        float *accg = reinterpret_cast<float *>(p.out);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row0 = wm * (BM / WM) + rt * 32 + 8 * q + 4 * lh;
                const int4 asg4 = *reinterpret_cast<const int4 *>(&row_asg[row0]);
                const float4 sc4 = *reinterpret_cast<const float4 *>(&row_scale[row0]);
                const int as[4] = {asg4.x, asg4.y, asg4.z, asg4.w};
                const float sw[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (as[i] < 0) continue;
                    const int col = nt * TN + wn * 64 + lr;
                    if (p.yrows) {
                        float *dst = p.yrows + ((size_t)blockIdx.y * p.T * p.k + as[i]) * p.d + col;
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) dst[ct * 32] = sw[i] * (acc[rt][ct][4 * q + i] * wsc[ct]);
                    } else {
                        float *dst = accg + (size_t)(as[i] / p.k) * p.d + col;
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct)
                            atomic_add_f32(dst + ct * 32, sw[i] * (acc[rt][ct][4 * q + i] * wsc[ct]));
                    }
                }
            }
        }
    }
    clear_zero();
}

// bf16 with weights stored [K][N] (the backward): the 256-column tiles
template <bool GEMM1>
hipError_t dispatch_kn(const TiledParams &p, int BM, int TN, dim3 grid, hipStream_t s) {
    if (TN != 256) return hipErrorInvalidValue;
    if (BM == 64)
        k_gemm_tiled<0, GEMM1, 64, 256, 8, true><<<grid, 512, 0, s>>>(p);
    else if (BM == 128)
        k_gemm_tiled<0, GEMM1, 128, 256, 8, true><<<grid, 512, 0, s>>>(p);
    else if (BM == 256)
        k_gemm_tiled<0, GEMM1, 256, 256, 8, true><<<grid, 512, 0, s>>>(p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int QUANT, bool GEMM1>
hipError_t dispatch_shape(const TiledParams &p, int BM, int TN, dim3 grid, hipStream_t s) {
    if (BM == 64 && TN == 256)
        k_gemm_tiled<QUANT, GEMM1, 64, 256, 8><<<grid, 512, 0, s>>>(p);
    else if (BM == 128 && TN == 256)
        k_gemm_tiled<QUANT, GEMM1, 128, 256, 8><<<grid, 512, 0, s>>>(p);
    else if (BM == 256 && TN == 128)
        k_gemm_tiled<QUANT, GEMM1, 256, 128, 8><<<grid, 512, 0, s>>>(p);
    else if (BM == 256 && TN == 256) {
        if constexpr (QUANT == 0 || QUANT == 3)
            k_gemm_tiled<QUANT, GEMM1, 256, 256, 8><<<grid, 512, 0, s>>>(p);
        else
            return hipErrorInvalidValue;
    } else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool GEMM1>
hipError_t dispatch(const TiledParams &p, int quant, int BM, int TN, dim3 grid, hipStream_t s) {
    if (quant == 0) return dispatch_shape<0, GEMM1>(p, BM, TN, grid, s);
    if (quant == 1) return dispatch_shape<1, GEMM1>(p, BM, TN, grid, s);
    if (quant == 3) return dispatch_shape<3, GEMM1>(p, BM, TN, grid, s);
    return hipErrorInvalidValue;
}

unsigned grid_tiles(int NB, int ntiles) {
    const unsigned total = (unsigned)NB * (unsigned)ntiles;
    return (total + 7) / 8 * 8;
}

}  // namespace

// MXFP4 runs K in pairs of 128-byte steps (512 elements), so d and f must
// be multiples of 512
bool tiled_gemm_supported(const GemmShape &sh) {
    if (!(sh.B == 64 || sh.B == 128 || sh.B == 256)) return false;
    if (sh.quant == 3) return sh.f % 512 == 0 && sh.d % 512 == 0;
    return (sh.quant == 0 || sh.quant == 1) && sh.f % 128 == 0 && sh.d % 256 == 0;
}

// Tile shape (rows BM, weight rows TN) for sort blocks of B rows; bm / tn
// > 0 request a shape, which must be one of the instantiated ones and BM must
// divide B. The library's choice: a 64/128-row block is one 64/128 x 256 tile;
// a 256-row block runs bf16 and MXFP4 as 256 x 256 tiles (a third fewer
// operand bytes per MFMA than 128 x 256) and e4m3 as 256 x 128 tiles (whose weight columns
// each cover a whole expert of up to 256 rows, so every weight byte leaves
// HBM once).
struct TileShape {
    int bm, tn;
};

TileShape tile_shape(int B, int quant, bool gemm1, int bm, int tn) {
    auto valid = [&](int m, int n) {
        if (m <= 0 || m > B || B % m) return false;
        return (n == 256 && (m == 64 || m == 128 || (m == 256 && quant != 1))) || (n == 128 && m == 256);
    };
    if (valid(bm, tn)) return {bm, tn};
    if (B < 256) return {B, 256};
    if (quant == 1) return {256, 128};
    return {256, 256};
}

int tiled_tile_cols(int B, int quant, bool gemm1, int bm, int tn) {
    return tile_shape(B, quant, gemm1, bm, tn).tn;
}

int tiled_tile_rows(int B, int quant, bool gemm1, int bm, int tn) {
    return tile_shape(B, quant, gemm1, bm, tn).bm;
}

hipError_t launch_tiled_gemm1(const Gemm1Args &g, int bm, int tn, hipStream_t s) {
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
    p.rotate = MOE_TILED_ROTATE & (1 << (2 * sh.quant));
    p.strip = MOE_TILED_STRIP1;
    p.zero = g.zero;
    p.zero_n = g.zero_n;
    p.a_mx = g.a_mx;
    p.w_mx = g.w13_mx;
    p.out_mx = g.h_mx;
    p.raw_out = sh.quant == 0 ? g.gu_out : nullptr;
    p.a_rows = (uint32_t)sh.T;
    const TileShape ts = tile_shape(sh.B, sh.quant, true, bm, tn);
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + ts.bm - 1) / ts.bm;
    const dim3 grid(grid_tiles(NB, sh.f / (ts.tn / 2)), 1);
    if (g.w_kn) {
        if (sh.quant != 0) return hipErrorInvalidValue;
        return dispatch_kn<true>(p, ts.bm, ts.tn, grid, s);
    }
    return dispatch<true>(p, sh.quant, ts.bm, ts.tn, grid, s);
}

// K steps (128 bytes per row) per part of a requested split; MXFP4 parts
// hold whole pairs of steps.
static int tiled_steps_per_part(int f, int quant, int ksplit) {
    const int steps = f / (quant == 0 ? 64 : (quant == 3 ? 256 : 128));
    ksplit = ksplit < 1 ? 1 : (ksplit > steps ? steps : ksplit);
    int steps_per = (steps + ksplit - 1) / ksplit;
    if (quant == 3) steps_per += steps_per & 1;
    return steps_per;
}

// Parts of K for a requested split: ceil(steps / steps per part), each
// non-empty.
int tiled_gemm2_parts(int f, int quant, int ksplit) {
    const int steps = f / (quant == 0 ? 64 : (quant == 3 ? 256 : 128));
    const int steps_per = tiled_steps_per_part(f, quant, ksplit);
    return (steps + steps_per - 1) / steps_per;
}

hipError_t launch_tiled_gemm2(const Gemm2Args &g, int bm, int tn, int ksplit, hipStream_t s) {
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
    p.yrows = g.yrows;
    p.a_mx = g.h_mx;
    p.w_mx = g.w2_mx;
    p.T = sh.T; p.d = sh.d; p.f = sh.f; p.k = sh.k; p.B = sh.B;
    const int KS = sh.quant == 0 ? 64 : (sh.quant == 3 ? 256 : 128);
    const int steps_per = tiled_steps_per_part(sh.f, sh.quant, ksplit);
    p.kchunk = steps_per * KS;
    p.rotate = MOE_TILED_ROTATE & (2 << (2 * sh.quant));
    p.strip = MOE_TILED_STRIP2;
    ksplit = tiled_gemm2_parts(sh.f, sh.quant, ksplit);
    const TileShape ts = tile_shape(sh.B, sh.quant, false, bm, tn);
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + ts.bm - 1) / ts.bm;
    p.a_rows = (uint32_t)P;
    const dim3 grid(grid_tiles(NB, sh.d / ts.tn), ksplit);
    if (g.w_kn) {
        if (sh.quant != 0) return hipErrorInvalidValue;
        return dispatch_kn<false>(p, ts.bm, ts.tn, grid, s);
    }
    return dispatch<false>(p, sh.quant, ts.bm, ts.tn, grid, s);
}

}  // namespace moe
