// backward.hip -- kernels of the bf16 layer's backward pass that the forward
// GEMMs do not cover: per-expert transposes of the weights (so that the
// backward GEMMs again reduce over a contiguous dimension) and the weight
// gradients, which reduce over the rows of each expert's segment of the
// sorted assignment list.
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

// C[e] [M, N] = sum over slots of the expert's segment of P[slot]^T Q[slot].
// Workgroup: a 64 x 64 tile of C; 4 waves of 32 x 32 (one 32x32x16 bf16 MFMA
// accumulator each). The segment is walked 32 rows at a time: each thread
// loads 8 values of one row of P and of Q and stores them transposed into
// LDS ([column][row], rows contiguous), so that an MFMA operand (8
// consecutive K = rows of one column) is one 16-byte LDS read. P is an fp32
// value in general (a routing weight times dy, or the fp32 dg / du), so it
// enters as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi), and two MFMAs:
// about 16 mantissa bits, against 8 for a plain bf16 operand. Q (x or h) is
// exactly bf16.
constexpr int WG_ROWS = 32;
constexpr int LDSW = WG_ROWS + 8;   // padded row of the transposed tiles (bf16)

__global__ __launch_bounds__(256) void k_wgrad(WgradOperand P, WgradOperand Q, int M, int N, int T,
                                               int k, const int32_t *__restrict__ sorted_ids,
                                               const float *__restrict__ sorted_w,
                                               const int32_t *__restrict__ offsets,
                                               float *__restrict__ C) {
    __shared__ __attribute__((aligned(16))) uint16_t pt[64][LDSW];
    __shared__ __attribute__((aligned(16))) uint16_t pl[64][LDSW];
    __shared__ __attribute__((aligned(16))) uint16_t qt[64][LDSW];
    const int e = blockIdx.z;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int sentinel = T * k;
    const int beg = offsets[e], end = offsets[e + 1];

    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

    // loader: thread -> row lr (0..31) of the chunk and 8 columns cs
    const int lr = tid >> 3, cs = (tid & 7) * 8;
    auto row_of = [&](const WgradOperand &o, int slot, int a) -> long {
        return o.by_token ? (long)(a / k) : (long)slot;
    };
    for (int r0 = beg; r0 < end; r0 += WG_ROWS) {
        const int slot = r0 + lr;
        const int a = slot < end ? sorted_ids[slot] : sentinel;
        const bool ok = a < sentinel;
        const float w = ok ? sorted_w[slot] : 0.0f;
        float pvals[8];
        uint4 qv = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) pvals[i] = 0.0f;
        if (ok) {
            const long pr = row_of(P, slot, a) * M + m0 + cs;
            if (P.base32) {
                const float4 u0 = *reinterpret_cast<const float4 *>(P.base32 + pr);
                const float4 u1 = *reinterpret_cast<const float4 *>(P.base32 + pr + 4);
                pvals[0] = u0.x; pvals[1] = u0.y; pvals[2] = u0.z; pvals[3] = u0.w;
                pvals[4] = u1.x; pvals[5] = u1.y; pvals[6] = u1.z; pvals[7] = u1.w;
            } else {
                const uint4 pv = *reinterpret_cast<const uint4 *>(P.base + pr);
                const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pvals[2 * i] = bf16_bits_to_f32(pw[i] & 0xffffu);
                    pvals[2 * i + 1] = bf16_bits_to_f32(pw[i] >> 16);
                }
            }
            if (P.scale_by_w)
#pragma unroll
                for (int i = 0; i < 8; ++i) pvals[i] *= w;
            qv = *reinterpret_cast<const uint4 *>(Q.base + row_of(Q, slot, a) * N + n0 + cs);
        }
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t hi = f32_to_bf16_bits(pvals[i]);
            pt[cs + i][lr] = hi;
            pl[cs + i][lr] = f32_to_bf16_bits(pvals[i] - bf16_bits_to_f32(hi));
            qt[cs + i][lr] = (uint16_t)((i & 1) ? qw[i >> 1] >> 16 : qw[i >> 1] & 0xffffu);
        }
        __syncthreads();
        // two K = 16 sub-steps over the 32 rows; lane half takes rows 8 (lane / 32) ..
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kr = 16 * sub + 8 * (lane >> 5);
            const u32x4 av = *reinterpret_cast<const u32x4 *>(&pt[32 * wm + (lane & 31)][kr]);
            const u32x4 al = *reinterpret_cast<const u32x4 *>(&pl[32 * wm + (lane & 31)][kr]);
            const u32x4 bv = *reinterpret_cast<const u32x4 *>(&qt[32 * wn + (lane & 31)][kr]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // 32x32 accumulator: lane holds column (lane & 31), rows 8 (v / 4) + 4 (lane / 32) + (v & 3)
    float *dst = C + (size_t)e * M * N;
    const int n = n0 + 32 * wn + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = m0 + 32 * wm + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        dst[(size_t)m * N + n] = acc[v];
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t *in, int E, int R, int C, uint16_t *out, hipStream_t s) {
    if (E == 0 || R % 64 || C % 64) return E == 0 ? hipSuccess : hipErrorInvalidValue;
    k_transpose_bf16<<<dim3(C / 64, R / 64, E), 256, 0, s>>>(in, R, C, out);
    return hipGetLastError();
}

hipError_t launch_wgrad(WgradOperand P, WgradOperand Q, int M, int N, int T, int k, int E,
                        const int32_t *sorted_ids, const float *sorted_w, const int32_t *offsets,
                        float *C, hipStream_t s) {
    if (E == 0) return hipSuccess;
    if (M % 64 || N % 64) return hipErrorInvalidValue;
    k_wgrad<<<dim3(N / 64, M / 64, E), 256, 0, s>>>(P, Q, M, N, T, k, sorted_ids, sorted_w, offsets, C);
    return hipGetLastError();
}

}  // namespace moe
