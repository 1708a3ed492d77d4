// quant_body.h -- the dynamic quantisation of activation rows as device
// functions, shared by the standalone quantisation kernels and by the routing
// launches that carry an activation quantisation on extra workgroups.
//
// Quantisation rule (the per_Token and per_1x128 quant types of the AITER
// walk-through, itsolotime.com/th/archives/32381, sections 1.1 and 3.2):
// s = amax / 448 over the group (s = 1 when amax = 0), q = e4m3(v / s) with
// round-to-nearest-even and saturation; both divisions are IEEE correctly
// rounded. MXFP4 (per_1x32): the E8M0 block exponent of mx_block_exp and
// round-to-nearest-even E2M1 codes of v / 2^E.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {

// Row r of x (bf16 [rows, cols]) as e4m3 codes, by the whole workgroup of NT
// threads (every thread calls it). Thread t owns the 8-element chunks t,
// t + NT, ... (16-byte loads, four in flight). GROUP_ROW: one scale for the
// row, from row_amax[r] when given, else found here; otherwise one scale per
// 128 columns (16 consecutive chunks = 16 lanes, all in the same pass since
// NT is a multiple of 16).
template <bool GROUP_ROW, int NT>
__device__ __forceinline__ void quant_row(const uint16_t *__restrict__ x, const float *__restrict__ row_amax,
                                          int r, int cols, uint8_t *__restrict__ codes,
                                          float *__restrict__ scales) {
    const int tid = threadIdx.x;
    const int nchunk = cols / 8;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)r * cols);
    uint2 *dst = reinterpret_cast<uint2 *>(codes + (size_t)r * cols);
    __shared__ float red[NT / 64];

    float s_row = 1.0f;
    if (GROUP_ROW) {
        float amax;
        if (row_amax) {
            amax = row_amax[r];
        } else {
            float m = 0.0f;
            for (int c = tid; c < nchunk; c += NT) {
                const uint4 q = src[c];
                const uint32_t wds[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(wds[i] & 0xffffu)));
                    m = fmaxf(m, fabsf(bf16_bits_to_f32(wds[i] >> 16)));
                }
            }
            m = wave_max(m);
            if ((tid & 63) == 0) red[tid >> 6] = m;
            __syncthreads();
            amax = 0.0f;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
            __syncthreads();   // red is free for the workgroup's next row
        }
        s_row = amax == 0.0f ? 1.0f : amax / 448.0f;
        if (tid == 0) scales[r] = s_row;
    }
    // chunk loop, QU chunks per thread per pass with their loads issued
    // first; for the 1x128 grouping all 16 lanes of a group are in the same
    // pass because NT is a multiple of 16.
    constexpr int QU = 4;
    for (int c0 = 0; c0 < nchunk; c0 += QU * NT) {
        uint4 q[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int c = c0 + u * NT + tid;
            q[u] = c < nchunk ? src[c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int c = c0 + u * NT + tid;
            const bool live = c < nchunk;
            float v[8];
            const uint32_t wds[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_bits_to_f32(wds[i] & 0xffffu);
                v[2 * i + 1] = bf16_bits_to_f32(wds[i] >> 16);
            }
            float s = s_row;
            if (!GROUP_ROW) {
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                s = m == 0.0f ? 1.0f : m / 448.0f;
                if (live && (c & 15) == 0) scales[(size_t)r * (cols / 128) + c / 16] = s;
            }
            if (live) {
                uint32_t lo = f32x2_to_e4m3x2(v[0] / s, v[1] / s) |
                              (f32x2_to_e4m3x2(v[2] / s, v[3] / s) << 16);
                uint32_t hi = f32x2_to_e4m3x2(v[4] / s, v[5] / s) |
                              (f32x2_to_e4m3x2(v[6] / s, v[7] / s) << 16);
                dst[c] = make_uint2(lo, hi);
            }
        }
    }
}

// MXFP4 block b (32 consecutive elements of x, blocks of a row adjacent):
// its E8M0 scale byte and 16 bytes of codes, two per byte (even column in
// the low nibble).
__device__ __forceinline__ void quant_mx_block(const uint16_t *__restrict__ x, size_t b,
                                               uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const uint4 *src = reinterpret_cast<const uint4 *>(x + b * 32);
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 q = src[c];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * c + 2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
            v[8 * c + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            amax = fmaxf(amax, fmaxf(fabsf(v[8 * c + 2 * i]), fabsf(v[8 * c + 2 * i + 1])));
        }
    }
    const int E = mx_block_exp(amax);
    const float inv = mx_inv_scale(E);
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = v[8 * j + i] * inv;
        out[j] = e2m1_pack8(sv);
    }
    *reinterpret_cast<uint4 *>(codes + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    scales[b] = (uint8_t)(E + 127);
}

// Workgroups an activation quantisation takes at NT threads each: one per
// row (e4m3), or one thread per MXFP4 block.
__host__ __device__ inline int act_quant_groups(const ActQuant &q, int nt) {
    if (q.kind == ACT_QUANT_NONE || q.rows <= 0) return 0;
    if (q.kind == ACT_QUANT_MX) return (int)(((size_t)q.rows * (q.cols / 32) + nt - 1) / nt);
    return q.rows;
}

// Workgroup `part` of the `nparts` that carry the quantisation q: a share of
// q.zero cleared, then its rows or blocks.
template <int NT>
__device__ __forceinline__ void act_quant_part(const ActQuant &q, int part, int nparts) {
    for (int i = part * NT + (int)threadIdx.x; i < q.zero_n; i += nparts * NT) q.zero[i] = 0.0f;
    if (q.kind == ACT_QUANT_MX) {
        const size_t nb = (size_t)q.rows * (q.cols / 32);
        for (size_t b = (size_t)part * NT + threadIdx.x; b < nb; b += (size_t)nparts * NT)
            quant_mx_block(q.x, b, q.codes, q.mx_scales);
        return;
    }
    for (int r = part; r < q.rows; r += nparts) {
        if (q.kind == ACT_QUANT_ROW)
            quant_row<true, NT>(q.x, nullptr, r, q.cols, q.codes, q.scales);
        else
            quant_row<false, NT>(q.x, nullptr, r, q.cols, q.codes, q.scales);
    }
}

}  // namespace moe
