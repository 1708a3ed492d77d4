// gemm_stream.hip -- weight-streaming grouped GEMMs for small sort blocks.
//
// Grouped GEMM over the sorted assignment list (grouped GEMMs in place of
// masked dense GEMMs: rocketrecap.com/entries/19116, talk summary at 5:58;
// the two stages of the AITER walk-through, itsolotime.com/th/archives/32381,
// section 3.2). One workgroup = one sort block (B <= 32 rows, all of one
// expert) x a slice of output columns; 4 waves split the columns.
//
// Both operands have the reduction dimension contiguous, so every lane loads
// its MFMA fragments straight from global memory: lane l serves row/column
// l % 16 and two 16-byte pieces of each 128-byte K step (lane group l / 16
// picks which), i.e. a wave reads whole 128-byte lines of 16 rows. The same
// K permutation is used for both operands, so the MFMA sums are the plain
// dot products (v_mfma_f32_16x16x32_bf16 twice, or one
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales, per step). MXFP4
// (E2M1, 256 elements per 128-byte step) takes two scaled MFMAs per step
// whose per-lane E8M0 scales are the lane's two 32-element blocks, so the
// block scaling happens inside the MFMA; the scales come in 8-step chunks.
// No LDS: weights are used by exactly one workgroup, which is the decode
// (weight-streaming, HBM-bound) regime. GEMM1 starts each workgroup's K loop
// at a step given by its column tile: weight rows 8 KiB apart would otherwise
// all be read at the same 128-byte column at once, which piles the requests
// onto the same HBM channels.
//
//   GEMM1: C[slot, n] over K = d, n in gate rows n0.. and up rows f + n0..,
//          epilogue h = silu(gate) * up -> bf16 (quant 0/1) or e4m3 per
//          1x128 block (quant 2); quant 1 also records the row amax.
//   GEMM2: C[slot, n] over K = f (optionally K-split across blockIdx.y),
//          epilogue acc[token, n] += sorted_w[slot] * C (fp32 atomics).
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct StreamParams {
    const uint8_t *a;        // A base (bytes)
    const float *a_scale;
    const uint8_t *w;        // weights base (bytes) [E, N_total, K]
    const float *w_scale;
    const int32_t *sorted_ids;
    const float *sorted_w;
    const int32_t *seid;
    void *out;               // GEMM1: h ; GEMM2: acc fp32 [T, d]
    float *out_scale;        // GEMM1 quant 1: row amax [P]; quant 2: h_scale [P, f/128]
    const uint8_t *a_mx;     // quant 3: E8M0 scales of A [rows, K/32]
    const uint8_t *w_mx;     // quant 3: E8M0 scales of the weights [E, N, K/32]
    uint8_t *out_mx;         // GEMM1 quant 3: E8M0 scales of h [P, f/32]
    int a_rows;              // quant 3: rows of a_mx (GEMM1: T tokens, GEMM2: P slots)
    // backward (bf16 GEMM1 only): gu_out receives the raw gate / up sums
    // [P, 2f] fp32 next to h. With bwd set the kernel computes v = Wd^T dy
    // (A = dy rows by token, weights Wd^T [E, f, d] split into "gate" rows
    // 0..f/2 and "up" rows f/2..f) and its epilogue turns v into the SwiGLU
    // input gradients dg, du [P, 2f] bf16 (from gu and the slot's routing
    // weight) and adds <v, h> into the routing-weight gradient of the
    // assignment (fp32 atomics); bwd_f is the layer's f.
    float *gu_out;
    // GEMM1 split over K (bf16): part blockIdx.y writes its raw gate / up sums
    // of every real row to gu_part [parts][T*k][2f] fp32 by assignment
    // (gate at column n, up at f + n) instead of h; a reduction kernel adds
    // the parts in a fixed order and applies SwiGLU
    float *gu_part;
    int bwd, bwd_f;
    const float *bwd_gu;
    const uint16_t *bwd_h;
    uint16_t *bwd_dgu;
    uint16_t *bwd_dgu_lo;    // bf16(g - bf16(g)) of each gradient: with bwd_dgu, about 16 bits
    float *bwd_dtw;
    int T, d, f, k, B;
    int kchunk;              // K elements per blockIdx.y
    int rotate;              // start the K loop at a step given by the column tile
    float *zero;             // optional fp32 buffer cleared by the grid on the way
    size_t zero_n;           // its length (a multiple of 4)
};

// Element formats: 0 bf16, 1/2 e4m3, 3 MXFP4 (E2M1, two per byte)
template <int QUANT>
struct Elem {
    static constexpr int kstep = QUANT == 0 ? 64 : (QUANT == 3 ? 256 : 128);  // K elements per 128-byte step
    // bytes of n consecutive elements
    static constexpr size_t off(size_t n) { return QUANT == 0 ? 2 * n : (QUANT == 3 ? n / 2 : n); }
};

struct Frag {
    u32x4 lo, hi;  // the lane's two 16-byte pieces of one row's 128-byte K step
};

// Where lane group lg (lane / 16) finds its two pieces in a 128-byte K step:
// bytes 32 lg and 32 lg + 16, except for MXFP4, whose pieces sit at 16 lg and
// 64 + 16 lg. An MXFP4 lane group then owns 32-element blocks lg and 4 + lg
// of every step, so its E8M0 scales are byte lg of consecutive scale dwords
// (see mx_chunk_to_lanes). Either way a wave's load covers whole 64-byte
// halves of 16 rows' lines, and both operands use the same K permutation.
template <int QUANT>
struct Piece {
    static constexpr int first(int lg) { return QUANT == 3 ? 16 * lg : 32 * lg; }
    static constexpr int second = QUANT == 3 ? 64 : 16;
};

#ifndef MOE_STREAM_NT
#define MOE_STREAM_NT 0
#endif
// K rotation: bit 0 GEMM1, bit 1 GEMM2
#ifndef MOE_STREAM_ROTATE
#define MOE_STREAM_ROTATE 1
#endif

template <int SECOND>
__device__ __forceinline__ Frag load_frag(const uint8_t *p) {
    Frag f;
    f.lo = *reinterpret_cast<const u32x4 *>(p);
    f.hi = *reinterpret_cast<const u32x4 *>(p + SECOND);
    return f;
}

// Weight operands: every weight tile of a wave shares one per-lane offset
// (row within the tile, piece of the step) and adds a wave-uniform offset
// (tile row, K step) from the expert's base, so the wave keeps no 64-bit
// pointer per tile. The bf16 / e4m3 loop uses global loads with a scalar
// base and a 32-bit lane offset (buffer loads measured 4 % slower in the
// bf16 down projection); the MXFP4 loop reads data and scales through
// buffer resources (no difference measured there). The slice must stay
// below 2 GiB.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void *base, size_t bytes) {
    // word 3 of a raw (unswizzled, stride 0) gfx9 resource: 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Nontemporal loads (MOE_STREAM_NT, the slc bit) would keep the weights, read
// once per call, from evicting activations from the caches, but measured
// slower; they are off.
template <int SECOND>
__device__ __forceinline__ Frag load_frag_buf(Rsrc r, int voff, int soff) {
    constexpr int aux = MOE_STREAM_NT ? 2 : 0;
    Frag f;
    f.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, aux));
    f.hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + SECOND, soff, aux));
    return f;
}

// acc += A . B over one 128-byte K step.
template <int QUANT>
__device__ __forceinline__ f32x4 mma_step(const Frag &a, const Frag &b, f32x4 acc) {
    if constexpr (QUANT == 0) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.lo),
                                                       __builtin_bit_cast(bf16x8, b.lo), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.hi),
                                                       __builtin_bit_cast(bf16x8, b.hi), acc, 0, 0, 0);
    } else {
        // one e4m3 MFMA over the whole 128-byte step (K = 128) with unit
        // E8M0 scales (127 = 2^0); both operands use the same lane/byte
        // layout, so the sum is the plain dot product
        typedef int i32x8 __attribute__((ext_vector_type(8)));
        const i32x8 av = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w,
                          (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
        const i32x8 bv = {(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w,
                          (int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
    }
    return acc;
}

#ifndef MOE_STREAM_DEPTH
#define MOE_STREAM_DEPTH 2
#endif

template <int QUANT, int RT, int NT>
struct StepBuf {
    Frag a[RT], b[NT];
    float sa[RT][4], sw[NT];
};

// The K loop of one wave: a ring of DEPTH fragment buffers, fully unrolled so
// every buffer index is a compile-time constant; the loads of step k + DEPTH-1
// are issued before the MFMAs of step k. Only the first RTL row tiles hold
// real rows. Block scales (QUANT 2) travel with their fragments.
// Weight tile nt of step kk is read at wexp + wtile[nt] + bytes of kk + wvoff.
template <int QUANT, int RT, int RTL, int NT>
__device__ __forceinline__ void stream_kloop(f32x4 (&acc)[RT][NT], const uint8_t *const (&arow)[RT],
                                             const uint8_t *wexp, int wvoff, const int (&wtile)[NT],
                                             const float *const (&sap)[RT][4],
                                             const float *const (&swp)[NT], int kbeg, int kend,
                                             int rot) {
    constexpr int KS = Elem<QUANT>::kstep;
    constexpr int DEPTH = MOE_STREAM_DEPTH;
    StepBuf<QUANT, RT, NT> bf[DEPTH];
    auto load = [&](StepBuf<QUANT, RT, NT> &b, int kk) {
#pragma unroll
        for (int rt = 0; rt < RTL; ++rt) b.a[rt] = load_frag<16>(arow[rt] + Elem<QUANT>::off(kk));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            b.b[nt] = load_frag<16>(wexp + (uint32_t)(wtile[nt] + (int)Elem<QUANT>::off(kk) + wvoff));
        if constexpr (QUANT == 2) {
            const int kb = kk / 128;
#pragma unroll
            for (int rt = 0; rt < RTL; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) b.sa[rt][i] = sap[rt][i][kb];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b.sw[nt] = swp[nt][kb];
        }
    };
    auto compute = [&](const StepBuf<QUANT, RT, NT> &b) {
#pragma unroll
        for (int rt = 0; rt < RTL; ++rt) {
            const Frag &a = b.a[rt];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (QUANT == 2) {
                    const f32x4 part = mma_step<QUANT>(a, b.b[nt], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rt][nt][i] += part[i] * (b.sa[rt][i] * b.sw[nt]);
                } else {
                    acc[rt][nt] = mma_step<QUANT>(a, b.b[nt], acc[rt][nt]);
                }
            }
        }
    };
    // Straight-line steady state (every load unconditional, so the wait
    // counts stay exact): prefetches past the last step are clamped to it and
    // hit the cache.
    const int nsteps = (kend - kbeg) / KS;
    if (nsteps <= 0) return;
    rot %= nsteps;
    auto kof = [&](int i) {
        int st = min(i, nsteps - 1) + rot;
        if (st >= nsteps) st -= nsteps;
        return kbeg + st * KS;
    };
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s) load(bf[s], kof(s));
    int i = 0;
    for (; i + DEPTH <= nsteps; i += DEPTH) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            load(bf[(s + DEPTH - 1) % DEPTH], kof(i + s + DEPTH - 1));
            // keep the prefetch above the MFMAs (the scheduler would
            // otherwise sink the loads below them)
            __builtin_amdgcn_sched_barrier(0);
            compute(bf[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s)
        if (i + s < nsteps) compute(bf[s]);
}

// MXFP4 scales. A scale row holds one E8M0 byte per 32-element block, 8 per
// K step; with the MXFP4 piece layout, dword 2j of a chunk of 8 steps holds
// the scales of lane groups 0..3 for the first MFMA of step j (byte lg) and
// dword 2j + 1 those for the second. Lane group lg loads dwords 4 lg .. 4 lg + 3
// of the chunk (16 bytes); this turns them into the lane's own bytes: on
// return d[m] = [first(2m), second(2m), first(2m+1), second(2m+1)] of lane
// group lg, and the MFMA picks the byte by op_sel. One 16-byte scale load per
// tile covers 8 steps.
__device__ __forceinline__ void mx_chunk_to_lanes(uint32_t (&d)[4]) {
    // in the lane: t_b = byte b of d0, d1, d2, d3 (what lane group b needs
    // from this lane group); v_perm byte selectors index {src0 : src1} with
    // src1 as bytes 0..3
    const uint32_t u0 = __builtin_amdgcn_perm(d[1], d[0], 0x06020400u);  // d0.b0 d1.b0 d0.b2 d1.b2
    const uint32_t u1 = __builtin_amdgcn_perm(d[1], d[0], 0x07030501u);  // d0.b1 d1.b1 d0.b3 d1.b3
    const uint32_t u2 = __builtin_amdgcn_perm(d[3], d[2], 0x06020400u);
    const uint32_t u3 = __builtin_amdgcn_perm(d[3], d[2], 0x07030501u);
    const uint32_t t0 = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
    const uint32_t t1 = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
    const uint32_t t2 = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
    const uint32_t t3 = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
    // across the four 16-lane rows (lane groups): register m of row r takes
    // register r of row m. permlane32_swap exchanges rows 2-3 of its first
    // operand with rows 0-1 of its second, permlane16_swap rows 1 and 3 of
    // the first with rows 0 and 2 of the second.
    const auto s02 = __builtin_amdgcn_permlane32_swap(t0, t2, false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(t1, t3, false, false);
    const auto q01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    const auto q23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    d[0] = q01[0];
    d[1] = q01[1];
    d[2] = q23[0];
    d[3] = q23[1];
}

// The MXFP4 K loop: steps of 128 bytes (K = 256), two scaled E2M1 MFMAs
// (format 4, K = 128 each) per step and tile pair, block scales applied
// inside the MFMA. Chunks of 8 steps, each with one scale load per tile
// issued a step ahead; the data ring is the same as stream_kloop's with
// DEPTH 2. Chunks start at a chunk given by rot; a last, partial chunk
// skips its missing steps (prefetches are clamped to the last step, and
// scale bytes past the end of a row are never used).
template <int RT, int RTL, int NT>
__device__ __forceinline__ void stream_kloop_mx(f32x4 (&acc)[RT][NT], const uint8_t *const (&arow)[RT],
                                                Rsrc wr, int wvoff, const int (&wtile)[NT], Rsrc axr,
                                                const int (&axvoff)[RT], Rsrc wxr, int wxvoff,
                                                const int (&wxtile)[NT], int kbeg, int kend, int rot) {
    constexpr int KS = 256, CH = 8, SECOND = Piece<3>::second;
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const int nsteps = (kend - kbeg) / KS;
    if (nsteps <= 0) return;
    const int nch = (nsteps + CH - 1) / CH;
    rot %= nch;
    const int xbase = kbeg / 32;
    Frag fa[2][RT], fb[2][NT];
    uint32_t ra[RT][4], rb[NT][4];  // chunk in flight
    uint32_t xa[RT][4], xb[NT][4];  // chunk in use
    auto chunk = [&](int i) {
        const int c = i + rot;
        return c >= nch ? c - nch : c;
    };
    auto load_scales = [&](int c) {
        const int so = xbase + 64 * c;
#pragma unroll
        for (int rt = 0; rt < RTL; ++rt) {
            const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(axr, axvoff[rt], so, 0));
            ra[rt][0] = v.x; ra[rt][1] = v.y; ra[rt][2] = v.z; ra[rt][3] = v.w;
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const u32x4 v =
                __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wxr, wxvoff, wxtile[nt] + so, 0));
            rb[nt][0] = v.x; rb[nt][1] = v.y; rb[nt][2] = v.z; rb[nt][3] = v.w;
        }
    };
    auto load_data = [&](int buf, int st) {
        const int kb = (kbeg + st * KS) / 2;  // bytes
#pragma unroll
        for (int rt = 0; rt < RTL; ++rt) fa[buf][rt] = load_frag<SECOND>(arow[rt] + kb);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) fb[buf][nt] = load_frag_buf<SECOND>(wr, wvoff, wtile[nt] + kb);
    };
    load_scales(chunk(0));
    load_data(0, CH * chunk(0));
    for (int i = 0; i < nch; ++i) {
        const int c = chunk(i);
        const int cn = chunk(min(i + 1, nch - 1));
#pragma unroll
        for (int rt = 0; rt < RTL; ++rt) {
#pragma unroll
            for (int m = 0; m < 4; ++m) xa[rt][m] = ra[rt][m];
            mx_chunk_to_lanes(xa[rt]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int m = 0; m < 4; ++m) xb[nt][m] = rb[nt][m];
            mx_chunk_to_lanes(xb[nt]);
        }
        static_for<CH>([&](auto sc) {
            constexpr int st = decltype(sc)::value;
            constexpr int cur = st & 1, m = st / 2, sel = 2 * (st & 1);
            if constexpr (st == CH - 1) load_scales(cn);
            load_data(cur ^ 1, st == CH - 1 ? CH * cn : min(CH * c + st + 1, nsteps - 1));
            // keep the prefetch above the MFMAs
            __builtin_amdgcn_sched_barrier(0);
            if (CH * c + st < nsteps) {
#pragma unroll
                for (int rt = 0; rt < RTL; ++rt) {
                    const Frag &a = fa[cur][rt];
                    const i32x8 alo = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w, 0, 0, 0, 0};
                    const i32x8 ahi = {(int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w, 0, 0, 0, 0};
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const Frag &b = fb[cur][nt];
                        const i32x8 blo = {(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w, 0, 0, 0, 0};
                        const i32x8 bhi = {(int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w, 0, 0, 0, 0};
                        acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            alo, blo, acc[rt][nt], 4, 4, sel, (int)xa[rt][m], sel, (int)xb[nt][m]);
                        acc[rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            ahi, bhi, acc[rt][nt], 4, 4, sel + 1, (int)xa[rt][m], sel + 1, (int)xb[nt][m]);
                    }
                }
            }
        });
    }
}

// RT: 16-row tiles per block (B = 16 * RT). CT: 16-column tiles per wave
// (GEMM1: CT gate tiles + CT matching up tiles).
template <int QUANT, int RT, int CT, bool GEMM1>
__global__ __launch_bounds__(256) void k_gemm_stream(StreamParams p) {
    constexpr int NT = GEMM1 ? 2 * CT : CT;
    static_assert(QUANT != 3 || !GEMM1 || CT == 2, "an MXFP4 h block is one wave's 32 columns");

    if (p.zero) {
        // clear the next stage's accumulator, 16 bytes per thread per pass
        const size_t nwg = (size_t)gridDim.x * gridDim.y * gridDim.z;
        const size_t wg = blockIdx.x + (size_t)gridDim.x * (blockIdx.y + (size_t)gridDim.y * blockIdx.z);
        float4 *z = reinterpret_cast<float4 *>(p.zero);
        for (size_t i = wg * 256 + threadIdx.x; i < p.zero_n / 4; i += nwg * 256)
            z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int blk = blockIdx.z;
    const int e = p.seid[blk];
    if (e < 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int sentinel = p.T * p.k;
    const int K = GEMM1 ? p.d : p.f;
    const int Ntot = GEMM1 ? 2 * p.f : p.d;   // weight rows per expert
    const int n0 = (blockIdx.x * 4 + wave) * CT * 16;
    const int kbeg = blockIdx.y * p.kchunk;
    const int kend = min(K, kbeg + p.kchunk);
    const int slot0 = blk * p.B;

    // rows of this lane's A fragments, and which 16-row tiles hold real rows.
    // A padding row (sentinel slot) of GEMM1 reads token 0: MFMA output rows
    // are independent, and the epilogue's results for padding slots are never
    // consumed, so the row needs no mask.
    const uint8_t *arow[RT];
    bool arow_ok[RT];
    bool live[RT];
    int a_of_lane[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int slot = slot0 + rt * 16 + lr;
        const int a = p.sorted_ids[slot];
        a_of_lane[rt] = a;
        live[rt] = p.sorted_ids[slot0 + rt * 16] < sentinel;
        if (GEMM1) {
            arow_ok[rt] = a < sentinel;
            const int t = arow_ok[rt] ? a / p.k : 0;
            arow[rt] = p.a + Elem<QUANT>::off((size_t)t * K) + Piece<QUANT>::first(lg);
        } else {
            arow_ok[rt] = true;
            arow[rt] = p.a + Elem<QUANT>::off((size_t)slot * K) + Piece<QUANT>::first(lg);
        }
    }
    // first weight row of each tile (wave-uniform)
    int wrow0[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wrow0[nt] = (GEMM1 && nt >= CT ? p.f : 0) + n0 + (nt % CT) * 16;
    const int kbytes = (int)Elem<QUANT>::off(K);
    const uint8_t *wexp = p.w + Elem<QUANT>::off((size_t)e * Ntot * K);
    const Rsrc wr = make_rsrc(wexp, (size_t)Ntot * kbytes);
    const int wvoff = lr * kbytes + Piece<QUANT>::first(lg);
    int wtile[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wtile[nt] = wrow0[nt] * kbytes;

    f32x4 acc[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // per-row scale rows for the 1x128 / 128x128 block-scaled product
    int srow[RT][4];
    if constexpr (QUANT == 2) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = lg * 4 + i;
                if (GEMM1) {
                    const int a = __shfl(a_of_lane[rt], r, 64);
                    srow[rt][i] = a < sentinel ? a / p.k : -1;
                } else {
                    srow[rt][i] = slot0 + rt * 16 + r;
                }
            }
    }

    // scale rows of the block-scaled product (sentinel rows read token 0's
    // scales; their products land in padding rows, which nothing consumes)
    const float *sap[RT][4];
    const float *swp[NT];
    if constexpr (QUANT == 2) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sap[rt][i] = p.a_scale + (size_t)max(srow[rt][i], 0) * (K / 128);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int nrow = (GEMM1 && nt >= CT ? p.f : 0) + n0 + (nt % CT) * 16;
            swp[nt] = p.w_scale + ((size_t)e * (Ntot / 128) + nrow / 128) * (K / 128);
        }
    }
    // K steps start at a step given by the column tile: weight rows a power
    // of two apart otherwise meet in the same HBM channels at the same moment
    const int rot = p.rotate ? (int)blockIdx.x : 0;
    if constexpr (QUANT == 3) {
        // scale rows: A by token (GEMM1; padding rows read token 0) or slot,
        // weights by the tile's rows; lane group lg reads bytes 16 lg .. of
        // each 64-byte chunk
        int axvoff[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = GEMM1 ? (arow_ok[rt] ? a_of_lane[rt] / p.k : 0) : slot0 + rt * 16 + lr;
            axvoff[rt] = r * (K / 32) + 16 * lg;
        }
        const Rsrc axr = make_rsrc(p.a_mx, (size_t)p.a_rows * (K / 32));
        const Rsrc wxr = make_rsrc(p.w_mx + (size_t)e * Ntot * (K / 32), (size_t)Ntot * (K / 32));
        const int wxvoff = lr * (K / 32) + 16 * lg;
        int wxtile[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wxtile[nt] = wrow0[nt] * (K / 32);
        if (RT == 2 && live[RT - 1])
            stream_kloop_mx<RT, RT, NT>(acc, arow, wr, wvoff, wtile, axr, axvoff, wxr, wxvoff, wxtile, kbeg,
                                        kend, rot);
        else
            stream_kloop_mx<RT, 1, NT>(acc, arow, wr, wvoff, wtile, axr, axvoff, wxr, wxvoff, wxtile, kbeg,
                                       kend, rot);
    } else {
        if (RT == 2 && live[RT - 1])
            stream_kloop<QUANT, RT, RT, NT>(acc, arow, wexp, wvoff, wtile, sap, swp, kbeg, kend, rot);
        else
            stream_kloop<QUANT, RT, 1, NT>(acc, arow, wexp, wvoff, wtile, sap, swp, kbeg, kend, rot);
    }

    // ------------------------------------------------------------ epilogue
    if constexpr (GEMM1 && QUANT == 0) {
        if (p.gu_part) {
            const size_t f2 = 2 * (size_t)p.f;
            float *part = p.gu_part + (size_t)blockIdx.y * sentinel * f2;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int a = __shfl(a_of_lane[rt], lg * 4 + i, 64);
                    if (a >= sentinel) continue;   // padding rows are not stored
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const int n = n0 + ct * 16 + lr;
                        part[(size_t)a * f2 + n] = acc[rt][ct][i];
                        part[(size_t)a * f2 + p.f + n] = acc[rt][CT + ct][i];
                    }
                }
            return;
        }
        if (p.bwd) {
            const int fb = p.bwd_f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = lg * 4 + i;
                    const int a = __shfl(a_of_lane[rt], r, 64);
                    const int slot = slot0 + rt * 16 + r;
                    const bool ok = a < sentinel;   // the same for the row's 16 lanes
                    const float w = ok ? p.sorted_w[slot] : 0.0f;
                    float dwp = 0.0f;
#pragma unroll
                    for (int half = 0; half < 2; ++half)
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) {
                            if (!ok) continue;
                            const int col = half * p.f + n0 + ct * 16 + lr;
                            const float v = acc[rt][half * CT + ct][i];
                            const size_t gi = (size_t)slot * 2 * fb + col;
                            const float g = p.bwd_gu[gi], u = p.bwd_gu[gi + fb];
                            dwp += v * bf16_bits_to_f32(p.bwd_h[(size_t)slot * fb + col]);
                            const float dh = w * v;
                            const float dg = dh * u * silu_grad(g), du = dh * silu(g);
                            const uint16_t gh = f32_to_bf16_bits(dg), uh = f32_to_bf16_bits(du);
                            p.bwd_dgu[gi] = gh;
                            p.bwd_dgu[gi + fb] = uh;
                            p.bwd_dgu_lo[gi] = f32_to_bf16_bits(dg - bf16_bits_to_f32(gh));
                            p.bwd_dgu_lo[gi + fb] = f32_to_bf16_bits(du - bf16_bits_to_f32(uh));
                        }
#pragma unroll
                    for (int o = 8; o > 0; o >>= 1) dwp += __shfl_xor(dwp, o, 64);
                    if (ok && lr == 0) atomic_add_f32(p.bwd_dtw + a, dwp);
                }
            return;
        }
    }
    if constexpr (GEMM1) {
        const int f = p.f;
        __shared__ float amax_lds[4][RT * 16];
        float hv[RT][CT][4];
        float rmax[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = lg * 4 + i;
                const int a = __shfl(a_of_lane[rt], r, 64);
                const int t = a < sentinel ? a / p.k : 0;
                const float sx = (QUANT == 1 && a < sentinel) ? p.a_scale[t] : 1.0f;
                float m = 0.0f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float g = acc[rt][ct][i], u = acc[rt][CT + ct][i];
                    if constexpr (QUANT == 1) {
                        const int n = n0 + ct * 16 + lr;
                        g = g * sx * p.w_scale[(size_t)e * Ntot + n];
                        u = u * sx * p.w_scale[(size_t)e * Ntot + f + n];
                    }
                    if (QUANT == 0 && p.gu_out) {
                        const int slot = slot0 + rt * 16 + r;
                        const int n = n0 + ct * 16 + lr;
                        p.gu_out[(size_t)slot * 2 * f + n] = g;
                        p.gu_out[(size_t)slot * 2 * f + f + n] = u;
                    }
                    const float h = bf16_bits_to_f32(f32_to_bf16_bits(silu(g) * u));
                    hv[rt][ct][i] = h;
                    m = fmaxf(m, fabsf(h));
                }
                if constexpr (QUANT != 0) {
#pragma unroll
                    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                }
                rmax[rt][i] = m;
            }
        if constexpr (QUANT == 2) {
            if (lr == 0)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) amax_lds[wave][rt * 16 + lg * 4 + i] = rmax[rt][i];
            __syncthreads();
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slot = slot0 + rt * 16 + lg * 4 + i;
                float s = 1.0f;
                if constexpr (QUANT == 2) {
                    const int r = rt * 16 + lg * 4 + i;
                    const float am = fmaxf(fmaxf(amax_lds[0][r], amax_lds[1][r]),
                                           fmaxf(amax_lds[2][r], amax_lds[3][r]));
                    s = am == 0.0f ? 1.0f : am / 448.0f;
                    // one 128-column block per workgroup (4 waves x CT x 16 = 128)
                    if (wave == 0 && lr == 0)
                        p.out_scale[(size_t)slot * (f / 128) + (blockIdx.x * 4 * CT * 16) / 128] = s;
                }
                if constexpr (QUANT == 1) {
                    if (lr == 0) atomic_max_nonneg(p.out_scale + slot, rmax[rt][i]);
                }
                if constexpr (QUANT == 3) {
                    // one MXFP4 block: the wave's 32 columns n0 .. n0+31 of the row;
                    // even lanes pack their code with the odd neighbour's
                    const int E = mx_block_exp(rmax[rt][i]);
                    const float inv = mx_inv_scale(E);
                    uint8_t *h = reinterpret_cast<uint8_t *>(p.out);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const uint32_t c = e2m1_code(hv[rt][ct][i] * inv);
                        const uint32_t hi = (uint32_t)__shfl_xor((int)c, 1, 64);
                        if ((lr & 1) == 0)
                            h[(size_t)slot * (f / 2) + (n0 + ct * 16 + lr) / 2] = (uint8_t)(c | (hi << 4));
                    }
                    if (lr == 0) p.out_mx[(size_t)slot * (f / 32) + n0 / 32] = (uint8_t)(E + 127);
                    continue;
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int n = n0 + ct * 16 + lr;
                    if constexpr (QUANT == 2) {
                        uint8_t *h = reinterpret_cast<uint8_t *>(p.out);
                        h[(size_t)slot * f + n] = (uint8_t)f32x2_to_e4m3x2(hv[rt][ct][i] / s, 0.0f);
                    } else {
                        uint16_t *h = reinterpret_cast<uint16_t *>(p.out);
                        h[(size_t)slot * f + n] = f32_to_bf16_bits(hv[rt][ct][i]);
                    }
                }
            }
    } else {
        float *accg = reinterpret_cast<float *>(p.out);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (!live[rt]) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = lg * 4 + i;
                const int slot = slot0 + rt * 16 + r;
                const int a = __shfl(a_of_lane[rt], r, 64);
                if (a >= sentinel) continue;
                float wgt = p.sorted_w ? p.sorted_w[slot] : 1.0f;
                if constexpr (QUANT == 1) wgt *= p.a_scale[slot];
                float *dst = accg + (size_t)(a / p.k) * p.d;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int n = n0 + ct * 16 + lr;
                    float y = acc[rt][ct][i];
                    if constexpr (QUANT == 1) y *= p.w_scale[(size_t)e * Ntot + n];
                    atomic_add_f32(dst + n, wgt * y);
                }
            }
        }
    }
}

template <int QUANT, int RT, int CT, bool GEMM1>
hipError_t run(const StreamParams &p, dim3 grid, hipStream_t s) {
    k_gemm_stream<QUANT, RT, CT, GEMM1><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
}

template <bool GEMM1, int QUANT>
hipError_t dispatch_rt_ct(const StreamParams &p, int RT, int CT, dim3 grid, hipStream_t s) {
    if constexpr (QUANT == 3 && GEMM1) {
        if (CT != 2) return hipErrorInvalidValue;
        if (RT == 1) return run<3, 1, 2, true>(p, grid, s);
        if (RT == 2) return run<3, 2, 2, true>(p, grid, s);
        return hipErrorInvalidValue;
    } else {
        if (RT == 1) {
            if (CT == 1) return run<QUANT, 1, 1, GEMM1>(p, grid, s);
            if (CT == 2) return run<QUANT, 1, 2, GEMM1>(p, grid, s);
            if (!GEMM1 && CT == 4) return run<QUANT, 1, 4, GEMM1>(p, grid, s);
        } else if (RT == 2) {
            if (CT == 1) return run<QUANT, 2, 1, GEMM1>(p, grid, s);
            if (CT == 2) return run<QUANT, 2, 2, GEMM1>(p, grid, s);
            if (!GEMM1 && CT == 4) return run<QUANT, 2, 4, GEMM1>(p, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

template <bool GEMM1>
hipError_t dispatch(const StreamParams &p, int quant, int RT, int CT, dim3 grid, hipStream_t s) {
    if (quant == 0) return dispatch_rt_ct<GEMM1, 0>(p, RT, CT, grid, s);
    if (quant == 1) return dispatch_rt_ct<GEMM1, 1>(p, RT, CT, grid, s);
    if (quant == 3) return dispatch_rt_ct<GEMM1, 3>(p, RT, CT, grid, s);
    return dispatch_rt_ct<GEMM1, 2>(p, RT, CT, grid, s);
}

}  // namespace

// Supported shapes: K (d for GEMM1, f for GEMM2) in whole 128-byte steps;
// GEMM1's h columns in whole workgroups (64 per column tile of each wave);
// one expert's weights below 2 GiB (buffer offsets).
static bool expert_slice_fits(const GemmShape &sh, size_t rows, size_t K) {
    const size_t elems = rows * K;
    const size_t bytes = sh.quant == 0 ? 2 * elems : (sh.quant == 3 ? elems / 2 : elems);
    return bytes < ((size_t)1 << 31);
}

// MXFP4 activation scales (a_rows x K/32 bytes) are read through a buffer
// resource as well
static bool mx_scales_fit(const GemmShape &sh, size_t a_rows, size_t K) {
    return sh.quant != 3 || a_rows * (K / 32) < ((size_t)1 << 31);
}

bool stream_gemm1_supported(const GemmShape &sh) {
    const int kstep = sh.quant == 3 ? 256 : 128;
    return (sh.B == 16 || sh.B == 32) && sh.f % 128 == 0 && sh.d % kstep == 0 &&
           expert_slice_fits(sh, 2 * (size_t)sh.f, sh.d) && mx_scales_fit(sh, sh.T, sh.d);
}

bool stream_gemm2_supported(const GemmShape &sh) {
    const int kstep = sh.quant == 3 ? 256 : 128;
    return (sh.B == 16 || sh.B == 32) && sh.f % kstep == 0 && sh.d % 128 == 0 &&
           expert_slice_fits(sh, sh.d, sh.f) &&
           mx_scales_fit(sh, (size_t)sh.T * sh.k + (size_t)sh.E * sh.B - sh.k, sh.f);
}

hipError_t launch_stream_gemm1(const Gemm1Args &g, int CT, hipStream_t s) {
    const GemmShape &sh = g.sh;
    StreamParams p{};
    p.a = static_cast<const uint8_t *>(g.a);
    p.a_scale = g.a_scale;
    p.w = static_cast<const uint8_t *>(g.w13);
    p.w_scale = g.w13_scale;
    p.sorted_ids = g.sorted_ids;
    p.seid = g.sorted_expert_ids;
    p.out = g.h;
    p.out_scale = g.h_scale;
    p.T = sh.T; p.d = sh.d; p.f = sh.f; p.k = sh.k; p.B = sh.B;
    p.kchunk = sh.d;
    p.rotate = MOE_STREAM_ROTATE & 1;
    p.zero = g.zero;
    p.zero_n = g.zero_n;
    p.a_mx = g.a_mx;
    p.a_rows = sh.T;
    p.w_mx = g.w13_mx;
    p.out_mx = g.h_mx;
    p.gu_out = g.gu_out;
    // quant 2: one 128-column quant block per workgroup; quant 3: one
    // 32-column MXFP4 block per wave
    if (sh.quant == 2 || sh.quant == 3) CT = 2;
    const int RT = sh.B / 16;
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + sh.B - 1) / sh.B;
    // K split (bf16): parts of whole 128-byte steps, raw sums to gu_part
    int parts = 1;
    if (sh.quant == 0 && g.gu_part && g.ksplit > 1) {
        const int steps = sh.d / Elem<0>::kstep;
        const int steps_per = (steps + g.ksplit - 1) / g.ksplit;
        p.kchunk = steps_per * Elem<0>::kstep;
        p.gu_part = g.gu_part;
        parts = (steps + steps_per - 1) / steps_per;
    }
    const dim3 grid(sh.f / (64 * CT), parts, NB);
    return dispatch<true>(p, sh.quant, RT, CT, grid, s);
}

// Parts of the bf16 GEMM1 K split actually launched for a requested split
// (each part whole 128-byte steps).
int stream_gemm1_parts(int d, int ksplit) {
    const int steps = d / Elem<0>::kstep;
    if (ksplit < 1) ksplit = 1;
    if (ksplit > steps) ksplit = steps;
    const int steps_per = (steps + ksplit - 1) / ksplit;
    return (steps + steps_per - 1) / steps_per;
}

// Backward of the down projection and SwiGLU (bf16): v = Wd^T dy per slot,
// then dg, du and the routing-weight gradient (see StreamParams). B = 16 or 32.
hipError_t launch_stream_bwd_dh(const GemmShape &sh, const uint16_t *dy, const uint16_t *w2t,
                                const int32_t *sorted_ids, const float *sorted_w,
                                const int32_t *sorted_expert_ids, const float *gu,
                                const uint16_t *h, uint16_t *dgu, uint16_t *dgu_lo, float *dtw,
                                hipStream_t s) {
    StreamParams p{};
    p.a = reinterpret_cast<const uint8_t *>(dy);
    p.w = reinterpret_cast<const uint8_t *>(w2t);
    p.sorted_ids = sorted_ids;
    p.sorted_w = sorted_w;
    p.seid = sorted_expert_ids;
    p.T = sh.T; p.d = sh.d; p.f = sh.f / 2; p.k = sh.k; p.B = sh.B;
    p.kchunk = sh.d;
    p.rotate = MOE_STREAM_ROTATE & 1;
    p.bwd = 1;
    p.bwd_f = sh.f;
    p.bwd_gu = gu;
    p.bwd_h = h;
    p.bwd_dgu = dgu;
    p.bwd_dgu_lo = dgu_lo;
    p.bwd_dtw = dtw;
    const int CT = 1, RT = sh.B / 16;
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + sh.B - 1) / sh.B;
    const dim3 grid(p.f / (64 * CT), 1, NB);
    return dispatch<true>(p, 0, RT, CT, grid, s);
}

hipError_t launch_stream_gemm2(const Gemm2Args &g, int CT, int ksplit, hipStream_t s) {
    const GemmShape &sh = g.sh;
    StreamParams p{};
    p.a = static_cast<const uint8_t *>(g.h);
    p.a_scale = g.h_scale;
    p.w = static_cast<const uint8_t *>(g.w2);
    p.w_scale = g.w2_scale;
    p.sorted_ids = g.sorted_ids;
    p.sorted_w = g.sorted_w;
    p.seid = g.sorted_expert_ids;
    p.out = g.acc;
    p.a_mx = g.h_mx;
    p.a_rows = sh.T * sh.k + sh.E * sh.B - sh.k;
    p.w_mx = g.w2_mx;
    p.T = sh.T; p.d = sh.d; p.f = sh.f; p.k = sh.k; p.B = sh.B;
    const int KS = sh.quant == 0 ? 64 : (sh.quant == 3 ? 256 : 128);
    const int steps = sh.f / KS;
    if (ksplit < 1) ksplit = 1;
    if (ksplit > steps) ksplit = steps;
    const int steps_per = (steps + ksplit - 1) / ksplit;
    p.kchunk = steps_per * KS;
    p.rotate = MOE_STREAM_ROTATE & 2;
    ksplit = (steps + steps_per - 1) / steps_per;
    const int RT = sh.B / 16;
    const int P = sh.T * sh.k + sh.E * sh.B - sh.k;
    const int NB = (P + sh.B - 1) / sh.B;
    while (CT > 1 && sh.d % (64 * CT) != 0) CT >>= 1;
    const dim3 grid(sh.d / (64 * CT), ksplit, NB);
    return dispatch<false>(p, sh.quant, RT, CT, grid, s);
}

}  // namespace moe
