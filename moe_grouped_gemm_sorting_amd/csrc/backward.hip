// backward.hip -- kernels of the bf16 layer's backward pass that the forward
// GEMMs do not cover: per-expert transposes of the weights (so that the
// backward GEMMs again reduce over a contiguous dimension), the SwiGLU
// backward of the tiled path, the gather of the weight gradients' operands
// into slot order, and the weight gradients, which reduce over the rows of
// each expert's segment of the sorted assignment list.
//
// The backward is the training step the pages name as the next milestone
// (rocketrecap.com/entries/19116, 10:07; rocketrecap.com/entries/19188,
// custom VJP); its arithmetic is the chain rule of the forward layer.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// out[e] [C, R] = in[e] [R, C]^T, bf16, one 64 x 64 tile per workgroup
// through LDS (rows padded by one element against bank conflicts).
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t *__restrict__ in, int R, int C,
                                                         uint16_t *__restrict__ out) {
    __shared__ uint16_t tile[64][65];
    const size_t e = blockIdx.z;
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const uint16_t *src = in + e * (size_t)R * C;
    uint16_t *dst = out + e * (size_t)R * C;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) tile[r][tx] = src[(size_t)(r0 + r) * C + c0 + tx];
    __syncthreads();
    for (int c = ty; c < 64; c += 4) dst[(size_t)(c0 + c) * R + r0 + tx] = tile[tx][c];
}

// SwiGLU backward for the tiled path, from the recomputed gate / up sums
// gu [P, 2f] and v = Wd^T dy [P, f] (fp32, slot order) of a real slot with
// routing weight w: h = bf16(silu(g) u) (the forward's h), dh = w v,
// dg = dh u silu'(g), du = dh silu(g), each stored as two bf16 parts
// (dgu = bf16(x), dgu_lo = bf16(x - dgu), [P, 2f]), and the routing-weight
// gradient dtw[a] += sum over the row of v h (one atomic per workgroup).
// Workgroup: 2048 columns of one slot, 8 per thread. Padding slots get
// zero rows of h, dgu and dgu_lo: the DMA weight-gradient kernel sums whole
// 32-row chunks of each expert's segment, padding rows included, and
// depends on those rows being zero.
__global__ __launch_bounds__(256) void k_bwd_swiglu(const float *__restrict__ gu, const float *__restrict__ v,
                                                    const int32_t *__restrict__ sorted_ids,
                                                    const float *__restrict__ sorted_w, int T, int k, int f,
                                                    uint16_t *__restrict__ h, uint16_t *__restrict__ dgu,
                                                    uint16_t *__restrict__ dgu_lo, float *__restrict__ dtw) {
    __shared__ float red[4];
    const int slot = blockIdx.x;
    const int a = sorted_ids[slot];
    const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (a >= T * k) {   // padding slot: zero rows (the weight gradients read them)
        if (c < f) {
            const size_t o = (size_t)slot * 2 * f + c;
            const uint4 z = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(h + (size_t)slot * f + c) = z;
            *reinterpret_cast<uint4 *>(dgu + o) = z;
            *reinterpret_cast<uint4 *>(dgu + o + f) = z;
            *reinterpret_cast<uint4 *>(dgu_lo + o) = z;
            *reinterpret_cast<uint4 *>(dgu_lo + o + f) = z;
        }
        return;
    }
    const float w = sorted_w[slot];
    float part = 0.0f;
    if (c < f) {
        const size_t f2 = 2 * (size_t)f;
        const float *gp = gu + (size_t)slot * f2 + c;
        const float *vp = v + (size_t)slot * f + c;
        float g[8], u[8], vv[8];
#pragma unroll
        for (int j = 0; j < 8; j += 4) {
            const float4 g4 = *reinterpret_cast<const float4 *>(gp + j);
            const float4 u4 = *reinterpret_cast<const float4 *>(gp + f + j);
            const float4 v4 = *reinterpret_cast<const float4 *>(vp + j);
            g[j] = g4.x; g[j + 1] = g4.y; g[j + 2] = g4.z; g[j + 3] = g4.w;
            u[j] = u4.x; u[j + 1] = u4.y; u[j + 2] = u4.z; u[j + 3] = u4.w;
            vv[j] = v4.x; vv[j + 1] = v4.y; vv[j + 2] = v4.z; vv[j + 3] = v4.w;
        }
        uint32_t hw[4], gh[4], gl[4], uh[4], ul[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            uint32_t hb[2], dgh[2], dgl[2], duh[2], dul[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float gg = g[j + i], uu = u[j + i], vi = vv[j + i];
                const uint16_t hbits = f32_to_bf16_bits(silu(gg) * uu);
                part += vi * bf16_bits_to_f32(hbits);
                const float dh = w * vi;
                const float dg = dh * uu * silu_grad(gg), du = dh * silu(gg);
                const uint16_t dgb = f32_to_bf16_bits(dg), dub = f32_to_bf16_bits(du);
                hb[i] = hbits;
                dgh[i] = dgb;
                dgl[i] = f32_to_bf16_bits(dg - bf16_bits_to_f32(dgb));
                duh[i] = dub;
                dul[i] = f32_to_bf16_bits(du - bf16_bits_to_f32(dub));
            }
            hw[j / 2] = hb[0] | (hb[1] << 16);
            gh[j / 2] = dgh[0] | (dgh[1] << 16);
            gl[j / 2] = dgl[0] | (dgl[1] << 16);
            uh[j / 2] = duh[0] | (duh[1] << 16);
            ul[j / 2] = dul[0] | (dul[1] << 16);
        }
        const size_t o = (size_t)slot * f2 + c;
        *reinterpret_cast<uint4 *>(h + (size_t)slot * f + c) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4 *>(dgu + o) = make_uint4(gh[0], gh[1], gh[2], gh[3]);
        *reinterpret_cast<uint4 *>(dgu + o + f) = make_uint4(uh[0], uh[1], uh[2], uh[3]);
        *reinterpret_cast<uint4 *>(dgu_lo + o) = make_uint4(gl[0], gl[1], gl[2], gl[3]);
        *reinterpret_cast<uint4 *>(dgu_lo + o + f) = make_uint4(ul[0], ul[1], ul[2], ul[3]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) atomic_add_f32(dtw + a, red[0] + red[1] + red[2] + red[3]);
}

// The weight gradients' operands in slot order: xs[slot] = x[t] and the
// fp32 value w[slot] dy[t] as two bf16 parts, dz_hi = bf16(z) and dz_lo =
// bf16(z - dz_hi), for the assignment a = t k + j in the slot; zeros for
// padding slots. One thread per (slot, 8 columns).
__global__ __launch_bounds__(256) void k_gather_bwd(const int32_t *__restrict__ sorted_ids,
                                                    const float *__restrict__ sorted_w, int P, int T,
                                                    int k, int d, const uint16_t *__restrict__ x,
                                                    const uint16_t *__restrict__ dy,
                                                    uint16_t *__restrict__ xs, uint16_t *__restrict__ dz_hi,
                                                    uint16_t *__restrict__ dz_lo) {
    const int g8 = d / 8;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)P * g8) return;
    const int slot = (int)(i / g8), c = (int)(i % g8) * 8;
    const int a = sorted_ids[slot];
    uint4 xv = make_uint4(0, 0, 0, 0);
    uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
    if (a < T * k) {
        const size_t src = (size_t)(a / k) * d + c;
        xv = *reinterpret_cast<const uint4 *>(x + src);
        const uint4 dv = *reinterpret_cast<const uint4 *>(dy + src);
        const float w = sorted_w[slot];
        const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float z0 = w * bf16_bits_to_f32(dw[j] & 0xffffu);
            const float z1 = w * bf16_bits_to_f32(dw[j] >> 16);
            const uint16_t h0 = f32_to_bf16_bits(z0), h1 = f32_to_bf16_bits(z1);
            hi[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[j] = (uint32_t)f32_to_bf16_bits(z0 - bf16_bits_to_f32(h0)) |
                    ((uint32_t)f32_to_bf16_bits(z1 - bf16_bits_to_f32(h1)) << 16);
        }
    }
    const size_t o = (size_t)slot * d + c;
    *reinterpret_cast<uint4 *>(xs + o) = xv;
    *reinterpret_cast<uint4 *>(dz_hi + o) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4 *>(dz_lo + o) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// C[e] [M, N] = sum over the slots of expert e's segment of P[slot]^T Q[slot]
// (P = P_hi + P_lo and Q bf16, [slots, M] and [slots, N], in slot order;
// rows past the expert's count are padding and contribute zeros).
// Workgroup: a 128 x 256 tile of C, 4 waves of 64 x 128 (2 x 4 accumulators
// of v_mfma_f32_32x32x16_bf16). The segment is walked 32 rows at a time.
// Thread t loads rows 4 (t % 8) .. + 3 of a chunk, P columns 4 (t / 8) ..
// + 3 and Q columns 8 (t / 8) .. + 7 (8- and 16-byte row pieces), and stores
// them transposed into LDS, [column][row] with 4 rows per 8-byte store, so
// that an MFMA operand (8 consecutive K = rows of one column) is one 16-byte
// LDS read. LDS rows are 80 bytes apart: the 16-byte operand reads of 16
// lanes then cover all 64 banks once, and the 8-byte P stores of 32 lanes
// (row offset fastest) are conflict-free (Q stores: 2-way). Slot-ordered
// operands make every load address affine in the row, so with NST = 2 LDS
// stages the loads run a chunk ahead in registers and a chunk's store
// overlaps the previous chunk's MFMAs. NST = 1 (half the LDS, for short
// segments) loads, stores and multiplies one chunk at a time.
// P is an fp32 value (a routing weight times dy, or dg / du), which its
// producer stores as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi); it
// enters as two MFMAs: about 16 mantissa bits, against 8 for a plain bf16
// operand (split once there rather than once per column tile of C here). Q
// (x or h) is exactly bf16.

// Workgroup barrier for LDS hand-over only: this wave's LDS operations
// complete, then s_barrier. A __syncthreads() also waits for every
// outstanding global load (its release fence), which would drain the
// register prefetch ring at every chunk.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int WG_ROWS = 32;
constexpr int WG_PITCH = WG_ROWS + 8;   // bf16 per LDS row: 80 bytes
#ifndef MOE_WG_QCOLS
#define MOE_WG_QCOLS 256
#endif
// Q columns (C columns) per workgroup: 256, or 128 (measured 1.75x slower at
// the prefill shape: more LDS fragment reads and global loads per MFMA)
constexpr int WG_QC = MOE_WG_QCOLS;
constexpr int WG_QW = WG_QC / 32;       // ... per loading thread
constexpr int WG_NB = WG_QC / 64;       // 32-column accumulator tiles per wave
constexpr int WG_RD = WG_QC == 128 ? 3 : 2;   // chunks in flight in registers

struct WgChunk {
    uint32_t p[2][4][2];          // [P_hi, P_lo][row][column pair]
    uint32_t q[4][WG_QW / 2];     // [row][column pair]
    int nreal;                    // real rows among the thread's 4 (a prefix)
};

template <int NST>
__global__ __launch_bounds__(256) void k_wgrad(const uint16_t *__restrict__ p_hi,
                                               const uint16_t *__restrict__ p_lo,
                                               const uint16_t *__restrict__ q, int M, int N,
                                               const int32_t *__restrict__ offsets,
                                               const int32_t *__restrict__ counts,
                                               float *__restrict__ C) {
    __shared__ __attribute__((aligned(16))) uint16_t lp[NST][2][128][WG_PITCH];   // [stage][hi, lo]
    __shared__ __attribute__((aligned(16))) uint16_t lq[NST][WG_QC][WG_PITCH];
    const int e = blockIdx.z;
    const int m0 = blockIdx.y * 128, n0 = blockIdx.x * WG_QC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int beg = offsets[e];
    const int real_end = beg + counts[e];
    // chunks over the real rows (an empty expert has none)
    const int nch = (real_end - beg + WG_ROWS - 1) / WG_ROWS;
    // loader: rows lr0 .. lr0 + 3 of a chunk, P columns lc0 .. lc0 + 3 and
    // Q columns lq0 .. lq0 + WG_QW - 1 of the tile
    const int lr0 = 4 * (tid & 7), lc0 = 4 * (tid >> 3), lq0 = WG_QW * (tid >> 3);
    const bool pm_ok = m0 + lc0 < M, qn_ok = n0 + lq0 < N;   // M, N multiples of 4 / WG_QW

    f32x16 acc[2][WG_NB];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < WG_NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    // Every load is issued (no divergent branch, whose join would make the
    // compiler wait for it at once): rows past real_end read the last real
    // row and columns past M / N read column 0; the store zeroes them.
    const size_t pcol = pm_ok ? (size_t)(m0 + lc0) : 0, qcol = qn_ok ? (size_t)(n0 + lq0) : 0;
    auto load = [&](WgChunk &ch, int c) {
        const int r0 = beg + c * WG_ROWS + lr0;
        ch.nreal = max(0, min(4, real_end - r0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t r = (size_t)min(r0 + i, real_end - 1);
            const uint2 h = *reinterpret_cast<const uint2 *>(p_hi + r * M + pcol);
            const uint2 l = *reinterpret_cast<const uint2 *>(p_lo + r * M + pcol);
            ch.p[0][i][0] = h.x; ch.p[0][i][1] = h.y;
            ch.p[1][i][0] = l.x; ch.p[1][i][1] = l.y;
            if constexpr (WG_QW == 4) {
                const uint2 u = *reinterpret_cast<const uint2 *>(q + r * N + qcol);
                ch.q[i][0] = u.x; ch.q[i][1] = u.y;
            } else {
                const uint4 u = *reinterpret_cast<const uint4 *>(q + r * N + qcol);
                ch.q[i][0] = u.x; ch.q[i][1] = u.y; ch.q[i][2] = u.z; ch.q[i][3] = u.w;
            }
        }
    };
    // column j of the thread's: rows lr0 .. lr0 + 3 as one 8-byte store
    // per operand (v_perm picks 16-bit halves; selector bytes 0-3 index the
    // second operand)
    auto store = [&](const WgChunk &ch, int st) {
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            uint32_t vv[4][WG_QW / 2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int w = 0; w < 2; ++w) vv[i][w] = (pm_ok && i < ch.nreal) ? ch.p[o][i][w] : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t r01 = __builtin_amdgcn_perm(vv[1][j >> 1], vv[0][j >> 1], sel);
                const uint32_t r23 = __builtin_amdgcn_perm(vv[3][j >> 1], vv[2][j >> 1], sel);
                *reinterpret_cast<uint2 *>(&lp[st][o][lc0 + j][lr0]) = make_uint2(r01, r23);
            }
        }
        uint32_t vq[4][WG_QW / 2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int w = 0; w < WG_QW / 2; ++w) vq[i][w] = (qn_ok && i < ch.nreal) ? ch.q[i][w] : 0u;
#pragma unroll
        for (int j = 0; j < WG_QW; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t r01 = __builtin_amdgcn_perm(vq[1][j >> 1], vq[0][j >> 1], sel);
            const uint32_t r23 = __builtin_amdgcn_perm(vq[3][j >> 1], vq[2][j >> 1], sel);
            *reinterpret_cast<uint2 *>(&lq[st][lq0 + j][lr0]) = make_uint2(r01, r23);
        }
    };
    // two K = 16 sub-steps over the chunk's 32 rows; lane half lane / 32
    // takes rows 8 (lane / 32) .. of each
    auto compute = [&](int st) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kr = 16 * sub + 8 * (lane >> 5);
            u32x4 ah[2], al[2], bq[WG_NB];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int col = 64 * wm + 32 * a + (lane & 31);
                ah[a] = *reinterpret_cast<const u32x4 *>(&lp[st][0][col][kr]);
                al[a] = *reinterpret_cast<const u32x4 *>(&lp[st][1][col][kr]);
            }
#pragma unroll
            for (int b = 0; b < WG_NB; ++b)
                bq[b] = *reinterpret_cast<const u32x4 *>(&lq[st][(WG_QC / 2) * wn + 32 * b + (lane & 31)][kr]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < WG_NB; ++b) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah[a]),
                                                                        __builtin_bit_cast(bf16x8, bq[b]),
                                                                        acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al[a]),
                                                                        __builtin_bit_cast(bf16x8, bq[b]),
                                                                        acc[a][b], 0, 0, 0);
                }
        }
    };
    if (nch > 0) {
        // chunk c lives in ring[c % RD]; the loop is unrolled by RD so the
        // ring index is a constant, and runs over a multiple of RD chunks so
        // that it is straight-line code (the compiler's wait counts then stay
        // exact). Chunks past the last real one have no real rows: they load
        // the last real row, store zeros and add nothing.
        constexpr int RD = NST == 2 ? WG_RD : 1;
        const int nch_pad = (nch + RD - 1) / RD * RD;
        WgChunk ring[RD];
#pragma unroll
        for (int i = 0; i < RD; ++i) load(ring[i], i);
        store(ring[0], 0);
        lds_barrier();
        for (int c0 = 0; c0 < nch_pad; c0 += RD) {
            static_for<RD>([&](auto ic) {
                constexpr int r = decltype(ic)::value;
                const int c = c0 + r;
                if constexpr (NST == 2) {
                    compute(c & 1);
                    store(ring[(r + 1) % RD], (c + 1) & 1);   // stage last read at chunk c - 1
                    load(ring[r], c + RD);                     // ring[r] (chunk c) is in LDS
                    lds_barrier();
                } else {
                    compute(0);
                    load(ring[0], c + 1);
                    lds_barrier();                             // every wave is done with the stage
                    store(ring[0], 0);
                    lds_barrier();
                }
            });
        }
    }
    // 32x32 accumulator: lane holds column (lane & 31), rows 8 (v / 4) + 4 (lane / 32) + (v & 3)
    float *dst = C + (size_t)e * M * N;
#pragma unroll
    for (int b = 0; b < WG_NB; ++b) {
        const int n = n0 + (WG_QC / 2) * wn + 32 * b + (lane & 31);
        if (n >= N) continue;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + 64 * wm + 32 * a + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M) dst[(size_t)m * N + n] = acc[a][b][v];
            }
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t *in, int E, int R, int C, uint16_t *out, hipStream_t s) {
    if (E == 0 || R % 64 || C % 64) return E == 0 ? hipSuccess : hipErrorInvalidValue;
    k_transpose_bf16<<<dim3(C / 64, R / 64, E), 256, 0, s>>>(in, R, C, out);
    return hipGetLastError();
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void wg_dma16(const void *base, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wg_wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t wg_lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)p;
}
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// The weight gradients for long segments of whole 32-row chunks whose
// padding rows are zero (the tiled path's producers zero them): the same sum
// as k_wgrad, with the slot rows moved into LDS by DMA as they lie in memory
// (no VGPR round trip, no transposing stores) and the MFMA operands read
// with the transposing LDS read ds_read_tr16_b64. Within a 16-lane group,
// lane i of that read receives element i % 4 of the 8-byte chunks that lanes
// 4j + i / 4 address (j = 0..3): with lane 4j + q pointing at row k0 + j and
// columns c0 + 4q .. + 3, lane i gets rows k0 .. k0 + 3 of column c0 + i, and
// two such reads give the 8 consecutive K values of a v_mfma_f32_16x16x32_bf16
// operand. Tile TM x 256 (TM = 128 or 256) with TM / 32 waves of 64 x 128 as
// 4 x 8 accumulators; three stages of P_hi, P_lo [32][TM] and Q [32][256]
// bf16 (32 KB for TM = 128, 48 KB for TM = 256), the 16-byte chunk c of row r
// stored at position c ^ 2 (r % 4), so that a transposing read's 16 lanes
// (4 rows x 2 chunks) meet 8 distinct chunk positions and no bank twice. The
// DMA wait counts are written out as in the tiled GEMMs. The 256-row tile
// moves a quarter fewer operand bytes per MFMA and puts two waves on each
// SIMD, so one wave's fragment reads overlap the other's MFMAs.
constexpr int WD_NBUF = 3;
constexpr int WD_QB = 32 * 512;           // bytes of the Q plane per stage
template <int TM>
struct WdShape {
    static constexpr int WAVES = TM / 32;
    static constexpr int PB = 32 * TM * 2;            // bytes of one P plane per stage
    static constexpr int STAGE = 2 * PB + WD_QB;
    static constexpr int NP = PB / 1024;              // DMA instructions per P plane
    static constexpr int NI = STAGE / 1024 / WAVES;   // ... per wave per stage
    static_assert(STAGE % (1024 * WAVES) == 0, "whole DMA instructions per wave");
    static_assert(WD_NBUF * STAGE <= 160 * 1024, "LDS");
};

template <int TM>
__global__ __launch_bounds__(64 * (TM / 32)) void k_wgrad_dma(const uint16_t *__restrict__ p_hi,
                                                              const uint16_t *__restrict__ p_lo,
                                                              const uint16_t *__restrict__ q, int M, int N,
                                                              const int32_t *__restrict__ offsets,
                                                              float *__restrict__ C) {
    using S = WdShape<TM>;
    constexpr int NI = S::NI, NP = S::NP, PB = S::PB, STAGE = S::STAGE, WAVES = S::WAVES;
    __shared__ __attribute__((aligned(16))) uint8_t lds[WD_NBUF * STAGE];
    const int e = blockIdx.z;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * 256;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int beg = offsets[e];
    const int nch = (offsets[e + 1] - beg) / 32;   // segments are whole 64-row blocks
    // DMA: instruction i fills 1 KB (64 chunks) of the stage: the P planes
    // NP KB each (instructions 0 .. NP - 1 hi, NP .. 2 NP - 1 lo), then Q
    // 16 KB; wave w issues instructions w, w + WAVES, ... (NI per wave)
    uint32_t goff[NI];
    const uint16_t *gbase[NI];
#pragma unroll
    for (int t = 0; t < NI; ++t) {
        const int ins = wave + WAVES * t;
        int plane, L;
        if (ins < 2 * NP) { plane = ins < NP ? 0 : 1; L = (ins % NP) * 64 + lane; }
        else { plane = 2; L = (ins - 2 * NP) * 64 + lane; }
        const int cpr = plane < 2 ? TM / 8 : 32;   // 16-byte chunks per row
        const int r = L / cpr, pos = L % cpr;
        const int c = pos ^ ((r & 3) << 1);
        if (plane < 2) {
            gbase[t] = plane == 0 ? p_hi : p_lo;
            goff[t] = (uint32_t)(r * M * 2 + m0 * 2 + c * 16);
        } else {
            gbase[t] = q;
            goff[t] = (uint32_t)(r * N * 2 + n0 * 2 + c * 16);
        }
    }
    const uint32_t lds0 = wg_lds_addr(lds);
    auto issue = [&](int buf, int ch) {
        ch = min(ch, nch - 1);
        const size_t row0 = (size_t)beg + (size_t)ch * 32;
#pragma unroll
        for (int t = 0; t < NI; ++t) {
            const int ins = wave + WAVES * t;
            const size_t rowbytes = ins < 2 * NP ? (size_t)M * 2 : (size_t)N * 2;
            const uint8_t *b = reinterpret_cast<const uint8_t *>(gbase[t]) + row0 * rowbytes;
            wg_dma16(b, goff[t], lds0 + (uint32_t)(buf * STAGE + ins * 1024));
        }
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // transposing read of 8 consecutive K rows (k = 8 g .. 8 g + 7, g = lane / 16) of column
    // c0 + lane % 16 of a plane with rows of rb bytes
    const int li = lane & 15, g = lane >> 4;
    const int tj = li >> 2, tq = li & 3;
    auto frag = [&](uint32_t plane_base, int rb, int c0) -> u32x4 {
        u32x4 out;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int r = 8 * g + 4 * hh + tj;
            const int col = c0 + 4 * tq;
            const int chunk = (col >> 3) ^ ((r & 3) << 1);
            const uint32_t addr = plane_base + (uint32_t)(r * rb + chunk * 16 + (col & 7) * 2);
            const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(uintptr_t)addr);
            out[2 * hh] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
            out[2 * hh + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
        }
        return out;
    };
    auto compute = [&](int buf) {
        const uint32_t sb = lds0 + (uint32_t)(buf * STAGE);
        u32x4 bq[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) bq[b] = frag(sb + 2 * PB, 512, 128 * wn + 16 * b);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const u32x4 ah = frag(sb, 2 * TM, 64 * wm + 16 * a);
            const u32x4 al = frag(sb + PB, 2 * TM, 64 * wm + 16 * a);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah),
                                                                    __builtin_bit_cast(bf16x8, bq[b]),
                                                                    acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al),
                                                                    __builtin_bit_cast(bf16x8, bq[b]),
                                                                    acc[a][b], 0, 0, 0);
            }
        }
    };
    if (nch > 0) {
#pragma unroll
        for (int b = 0; b < WD_NBUF - 1; ++b) issue(b, b);
        wg_wait_vmem<NI * (WD_NBUF - 2)>();
        __builtin_amdgcn_s_barrier();
        for (int c0 = 0; c0 < nch; c0 += WD_NBUF) {
            static_for<WD_NBUF>([&](auto ic) {
                constexpr int r = decltype(ic)::value;
                const int c = c0 + r;
                if (c < nch) {
                    issue((r + WD_NBUF - 1) % WD_NBUF, c + WD_NBUF - 1);
                    compute(r);
                    wg_wait_vmem<NI * (WD_NBUF - 2)>();
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                }
            });
        }
        wg_wait_vmem<0>();
    }
    // 16x16 accumulator: lane holds column lane % 16, rows 4 (lane / 16) + v
    float *dst = C + (size_t)e * M * N;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int n = n0 + 128 * wn + 16 * b + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 64 * wm + 16 * a + 4 * g + v;
                if (m < M && n < N) dst[(size_t)m * N + n] = acc[a][b][v];
            }
        }
}

hipError_t launch_wgrad_dma(const uint16_t *p_hi, const uint16_t *p_lo, const uint16_t *q, int M, int N, int E,
                            const int32_t *offsets, float *C, hipStream_t s) {
    if (E == 0) return hipSuccess;
    if (M % 128 || N % 256) return hipErrorInvalidValue;
    // 256-row tiles where M allows; MOE_WGRAD_TM=128 keeps the 128-row tile
    static const int tm_env = [] {
        const char *v = getenv("MOE_WGRAD_TM");
        return v ? atoi(v) : 0;
    }();
    if (M % 256 == 0 && tm_env != 128)
        k_wgrad_dma<256><<<dim3(N / 256, M / 256, E), 512, 0, s>>>(p_hi, p_lo, q, M, N, offsets, C);
    else
        k_wgrad_dma<128><<<dim3(N / 256, M / 128, E), 256, 0, s>>>(p_hi, p_lo, q, M, N, offsets, C);
    return hipGetLastError();
}

hipError_t launch_bwd_swiglu(const float *gu, const float *v, const int32_t *sorted_ids,
                             const float *sorted_w, int P, int T, int k, int f, uint16_t *h, uint16_t *dgu,
                             uint16_t *dgu_lo, float *dtw, hipStream_t s) {
    if (P == 0) return hipSuccess;
    if (f % 8) return hipErrorInvalidValue;
    k_bwd_swiglu<<<dim3(P, (f + 2047) / 2048), 256, 0, s>>>(gu, v, sorted_ids, sorted_w, T, k, f, h, dgu,
                                                             dgu_lo, dtw);
    return hipGetLastError();
}

hipError_t launch_gather_bwd(const int32_t *sorted_ids, const float *sorted_w, int P, int T, int k,
                             int d, const uint16_t *x, const uint16_t *dy, uint16_t *xs, uint16_t *dz_hi,
                             uint16_t *dz_lo, hipStream_t s) {
    if (P == 0) return hipSuccess;
    if (d % 8) return hipErrorInvalidValue;
    const size_t n = (size_t)P * (d / 8);
    k_gather_bwd<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(sorted_ids, sorted_w, P, T, k, d, x, dy, xs,
                                                              dz_hi, dz_lo);
    return hipGetLastError();
}

hipError_t launch_wgrad(const uint16_t *p_hi, const uint16_t *p_lo, const uint16_t *q, int M, int N, int E,
                        const int32_t *offsets, const int32_t *counts, bool short_segments, float *C,
                        hipStream_t s) {
    if (E == 0) return hipSuccess;
    if (M % 4 || N % WG_QW) return hipErrorInvalidValue;
    const dim3 grid((N + WG_QC - 1) / WG_QC, (M + 127) / 128, E);
    if (short_segments)
        k_wgrad<1><<<grid, 256, 0, s>>>(p_hi, p_lo, q, M, N, offsets, counts, C);
    else
        k_wgrad<2><<<grid, 256, 0, s>>>(p_hi, p_lo, q, M, N, offsets, counts, C);
    return hipGetLastError();
}

}  // namespace moe
