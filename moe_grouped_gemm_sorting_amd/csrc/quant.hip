// quant.hip -- dynamic e4m3 quantisation of activations and of the
// intermediate h, plus the accumulator fill and the final fp32 -> bf16 pass.
//
// The quantisation rules and the per-row and per-block bodies are in
// quant_body.h (shared with the routing launches that carry the activation
// quantisation).
#include <algorithm>

#include "quant_body.h"

namespace moe {

// One workgroup of NT threads per row (quant_row). With num_valid (rows of h
// by sort slot), rows at or past num_valid and rows of padding slots
// (sorted_ids[r] == sentinel) are skipped. zero[0, zero_n), when given, is
// cleared on the way (the row amax that the e4m3 GEMM1 which follows takes
// with atomics). The rows of h (amax given, 14336 columns in the Mixtral
// shape) take 512 threads: 14.6 against 20.7 us for 1024 rows at 256
// threads; the activation rows, whose amax the workgroup finds itself, gain
// nothing.
template <bool GROUP_ROW, int NT = 256>
__global__ __launch_bounds__(NT) void k_quant_rows(const uint16_t *__restrict__ x,
                                                    const float *__restrict__ row_amax,
                                                    const int32_t *__restrict__ num_valid,
                                                    const int32_t *__restrict__ sorted_ids,
                                                    int sentinel, int cols,
                                                    uint8_t *__restrict__ codes,
                                                    float *__restrict__ scales,
                                                    float *__restrict__ zero, int zero_n) {
    for (int i = blockIdx.x * NT + threadIdx.x; i < zero_n; i += gridDim.x * NT) zero[i] = 0.0f;
    const int r = blockIdx.x;
    if (num_valid && r >= *num_valid) return;
    if (sorted_ids && sorted_ids[r] >= sentinel) return;
    quant_row<GROUP_ROW, NT>(x, row_amax, r, cols, codes, scales);
}

// MXFP4 (per_1x32) quantisation: one thread per 32-element block of a row.
__global__ __launch_bounds__(256) void k_quant_mx(const uint16_t *__restrict__ x, int rows, int cols,
                                                  uint8_t *__restrict__ codes,
                                                  uint8_t *__restrict__ scales) {
    const size_t b = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= (size_t)rows * (cols / 32)) return;
    quant_mx_block(x, b, codes, scales);
}

hipError_t launch_quant_mx(const uint16_t *x, int rows, int cols, uint8_t *codes, uint8_t *scales,
                           hipStream_t s) {
    const size_t n = (size_t)rows * (cols / 32);
    if (n == 0) return hipSuccess;
    k_quant_mx<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, rows, cols, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t *x, int rows, int cols, int group, uint8_t *codes,
                            float *scales, hipStream_t s, float *zero, int zero_n) {
    if (rows == 0) return zero_n > 0 ? launch_fill_f32(zero, (size_t)zero_n, 0.0f, s) : hipSuccess;
    if (group == cols)
        k_quant_rows<true><<<rows, 256, 0, s>>>(x, nullptr, nullptr, nullptr, 0, cols, codes, scales,
                                                zero, zero_n);
    else
        k_quant_rows<false><<<rows, 256, 0, s>>>(x, nullptr, nullptr, nullptr, 0, cols, codes, scales,
                                                 zero, zero_n);
    return hipGetLastError();
}

hipError_t launch_quant_h_rows(const uint16_t *h, const float *amax, int rows, int cols,
                               const int32_t *num_valid, const int32_t *sorted_ids,
                               int sentinel, uint8_t *codes, float *scales, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    k_quant_rows<true, 512><<<rows, 512, 0, s>>>(h, amax, num_valid, sorted_ids, sentinel, cols, codes,
                                                 scales, nullptr, 0);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill(float *__restrict__ p, size_t n, float v) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t n4 = n / 4;
    float4 *p4 = reinterpret_cast<float4 *>(p);
    for (; i < n4; i += stride) p4[i] = make_float4(v, v, v, v);
    for (size_t j = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; j < n; j += stride) p[j] = v;
}

hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n / 4 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks == 0) blocks = 1;
    k_fill<<<(unsigned)blocks, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_finalize(const float *__restrict__ acc,
                                                  uint16_t *__restrict__ out, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t n4 = n / 4;
    const float4 *a4 = reinterpret_cast<const float4 *>(acc);
    uint2 *o4 = reinterpret_cast<uint2 *>(out);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const float4 v = a4[i];
        o4[i] = make_uint2(f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16),
                           f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16));
    }
    for (size_t j = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; j < n; j += stride)
        out[j] = f32_to_bf16_bits(acc[j]);
}

hipError_t launch_finalize(const float *acc, uint16_t *out, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n / 4 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks == 0) blocks = 1;
    k_finalize<<<(unsigned)blocks, 256, 0, s>>>(acc, out, n);
    return hipGetLastError();
}

// The combine over stored rows: each token's k weighted expert rows, which
// GEMM2 wrote at the token's assignments t*k + j, summed in fp32 in
// ascending j and rounded once to bf16. d is a multiple of 4.
// rows: `parts` slabs of [T*k, d] (one per part of a split reduction); a
// token's sum takes its rows in ascending j and, within a row, the parts in
// ascending order. written (optional, [T*k]): nonzero for the assignments
// the sort placed; rows of the others were never written and count as zero
// (NULL: every assignment was placed).
__global__ __launch_bounds__(256) void k_combine_rows(const float *__restrict__ rows, int T, int k,
                                                      int parts, int d,
                                                      const int32_t *__restrict__ written,
                                                      uint16_t *__restrict__ out) {
    const int d4 = d / 4;
    const size_t n4 = (size_t)T * d4;
    const size_t slab4 = (size_t)T * k * d4;
    const size_t stride = (size_t)gridDim.x * 256;
    const float4 *r4 = reinterpret_cast<const float4 *>(rows);
    uint2 *o4 = reinterpret_cast<uint2 *>(out);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const size_t t = i / d4, c = i - t * d4;
        const float4 *src = r4 + t * k * d4 + c;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        bool first = true;
        for (int j = 0; j < k; ++j) {
            if (written && !written[t * k + j]) continue;
            for (int q = 0; q < parts; ++q) {
                const float4 u = src[(size_t)q * slab4 + (size_t)j * d4];
                if (first) {
                    v = u;
                    first = false;
                    continue;
                }
                v.x += u.x;
                v.y += u.y;
                v.z += u.z;
                v.w += u.w;
            }
        }
        o4[i] = make_uint2(f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16),
                           f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16));
    }
}

hipError_t launch_combine_rows(const float *rows, int T, int k, int parts, int d,
                               const int32_t *written, uint16_t *out, hipStream_t s) {
    const size_t n4 = (size_t)T * (d / 4);
    if (n4 == 0) return hipSuccess;
    size_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    k_combine_rows<<<(unsigned)blocks, 256, 0, s>>>(rows, T, k, parts, d, written, out);
    return hipGetLastError();
}

// written[a] = 1 for every assignment a in sorted_ids[0, num_valid) (the
// array is cleared first by the caller).
__global__ __launch_bounds__(256) void k_mark_written(const int32_t *__restrict__ sorted_ids,
                                                      const int32_t *__restrict__ num_valid, int n_asg,
                                                      int32_t *__restrict__ written) {
    const int nv = *num_valid;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < nv; i += gridDim.x * 256) {
        const int a = sorted_ids[i];
        if (a >= 0 && a < n_asg) written[a] = 1;
    }
}

__global__ __launch_bounds__(256) void k_clear_i32(int32_t *__restrict__ p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

hipError_t launch_mark_written(const int32_t *sorted_ids, const int32_t *num_valid, int P, int n_asg,
                               int32_t *written, hipStream_t s) {
    if (n_asg == 0) return hipSuccess;
    const unsigned bc = (unsigned)std::min(1024, (n_asg + 255) / 256);
    k_clear_i32<<<bc, 256, 0, s>>>(written, n_asg);
    const unsigned bm = (unsigned)std::min(1024, (P + 255) / 256);
    k_mark_written<<<bm, 256, 0, s>>>(sorted_ids, num_valid, n_asg, written);
    return hipGetLastError();
}

// The end of the bf16 GEMM1 split over K: for each real slot, the parts'
// gate and up sums added in ascending part order (a fixed order, so the
// result does not depend on scheduling), then h = bf16(silu(g) u), the same
// epilogue as the unsplit kernel. One workgroup: 2048 columns of one slot.
__global__ __launch_bounds__(256) void k_swiglu_parts(const float *__restrict__ gu_part, int parts, int n_asg,
                                                      int f, const int32_t *__restrict__ sorted_ids,
                                                      const int32_t *__restrict__ num_valid,
                                                      uint16_t *__restrict__ h) {
    const int slot = blockIdx.x;
    if (slot >= *num_valid) return;
    const int a = sorted_ids[slot];
    if (a >= n_asg) return;
    const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (c >= f) return;
    const size_t f2 = 2 * (size_t)f, slab = (size_t)n_asg * f2;
    const float *src = gu_part + (size_t)a * f2 + c;
    float g[8], u[8];
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
        const float4 gv = *reinterpret_cast<const float4 *>(src + i);
        const float4 uv = *reinterpret_cast<const float4 *>(src + f + i);
        g[i] = gv.x; g[i + 1] = gv.y; g[i + 2] = gv.z; g[i + 3] = gv.w;
        u[i] = uv.x; u[i + 1] = uv.y; u[i + 2] = uv.z; u[i + 3] = uv.w;
    }
    for (int q = 1; q < parts; ++q) {
        const float *sq = src + (size_t)q * slab;
#pragma unroll
        for (int i = 0; i < 8; i += 4) {
            const float4 gv = *reinterpret_cast<const float4 *>(sq + i);
            const float4 uv = *reinterpret_cast<const float4 *>(sq + f + i);
            g[i] += gv.x; g[i + 1] += gv.y; g[i + 2] += gv.z; g[i + 3] += gv.w;
            u[i] += uv.x; u[i + 1] += uv.y; u[i + 2] += uv.z; u[i + 3] += uv.w;
        }
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = f32_to_bf16_bits(silu(g[2 * i]) * u[2 * i]) |
               ((uint32_t)f32_to_bf16_bits(silu(g[2 * i + 1]) * u[2 * i + 1]) << 16);
    *reinterpret_cast<uint4 *>(h + (size_t)slot * f + c) = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t launch_swiglu_parts(const float *gu_part, int parts, int n_asg, int f, const int32_t *sorted_ids,
                               const int32_t *num_valid, int P, uint16_t *h, hipStream_t s) {
    if (P == 0 || n_asg == 0) return hipSuccess;
    const dim3 grid((unsigned)P, (unsigned)((f / 8 + 255) / 256));
    k_swiglu_parts<<<grid, 256, 0, s>>>(gu_part, parts, n_asg, f, sorted_ids, num_valid, h);
    return hipGetLastError();
}

}  // namespace moe
