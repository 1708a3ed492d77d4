// launch.h -- host-side launchers of libmoe's kernels (internal to the library).
// Every launcher only enqueues work on `s` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// An activation quantisation that a routing launch carries on workgroups of
// its own after the routing ones (the two are independent, so it runs while
// the routing does). x bf16 [rows, cols]; ACT_QUANT_ROW: e4m3 codes
// [rows, cols] with one fp32 scale per row; ACT_QUANT_BLOCK: one per 1x128;
// ACT_QUANT_MX: E2M1 codes two per byte [rows, cols / 2] and E8M0 scales
// [rows, cols / 32]. zero[0, zero_n), when given, is cleared on the way.
enum { ACT_QUANT_NONE = 0, ACT_QUANT_ROW = 1, ACT_QUANT_BLOCK = 2, ACT_QUANT_MX = 3 };
struct ActQuant {
    const uint16_t *x;
    int rows, cols, kind;
    uint8_t *codes;
    float *scales;        // e4m3 kinds
    uint8_t *mx_scales;   // ACT_QUANT_MX
    float *zero;
    int zero_n;
};

hipError_t launch_topk(const float *logits, int T, int E, int k, int score, int renorm,
                       int32_t *ids, float *w, hipStream_t s, const ActQuant *aq = nullptr);

hipError_t launch_sort(const int32_t *ids, const float *w, int T, int k, int E, int B,
                       int32_t *sorted_ids, float *sorted_w, int32_t *sorted_expert_ids,
                       int32_t *counts, int32_t *offsets, int32_t *num_valid, hipStream_t s);

// routing + sort in one launch (ids / w are written as scratch)
hipError_t launch_route_sort(const float *logits, int T, int k, int E, int B, int score,
                             int renorm, int32_t *ids, float *w, int32_t *sorted_ids,
                             float *sorted_w, int32_t *sorted_expert_ids, int32_t *counts,
                             int32_t *offsets, int32_t *num_valid, hipStream_t s,
                             float *zero = nullptr, int zero_n = 0, const ActQuant *aq = nullptr);

// MXFP4: codes [rows, cols / 2] (two per byte), E8M0 scales [rows, cols / 32]
hipError_t launch_quant_mx(const uint16_t *x, int rows, int cols, uint8_t *codes, uint8_t *scales,
                           hipStream_t s);

// codes [rows, cols], scales [rows, cols / group]; zero[0, zero_n), when
// given, is cleared in the same launch
hipError_t launch_quant_act(const uint16_t *x, int rows, int cols, int group, uint8_t *codes,
                            float *scales, hipStream_t s, float *zero = nullptr, int zero_n = 0);

// h rows: bf16 [rows, cols] with row amax [rows] -> e4m3 codes + scale [rows]
hipError_t launch_quant_h_rows(const uint16_t *h, const float *amax, int rows, int cols,
                               const int32_t *num_valid, const int32_t *sorted_ids,
                               int sentinel, uint8_t *codes, float *scales, hipStream_t s);

hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t s);

// acc fp32 [n] -> bf16 [n]
hipError_t launch_finalize(const float *acc, uint16_t *out, size_t n, hipStream_t s);

// out[t, :] = bf16(sum over j < k of rows[t*k + j, :]) (j ascending), rows fp32
// [parts][T*k, d]; written (optional, [T*k]) marks the rows GEMM2 stored: an
// unmarked row counts as zero
hipError_t launch_combine_rows(const float *rows, int T, int k, int parts, int d,
                               const int32_t *written, uint16_t *out, hipStream_t s);
// written[a] = 1 for the assignments in sorted_ids[0, num_valid), 0 for the
// others (the ones the sort dropped); n_asg = T*k
hipError_t launch_mark_written(const int32_t *sorted_ids, const int32_t *num_valid, int P, int n_asg,
                               int32_t *written, hipStream_t s);

struct GemmShape {
    int T, d, f, E, k, B, quant;
};

struct Gemm1Args {
    GemmShape sh;
    const void *a;          // x bf16 [T, d] (quant 0) or e4m3 codes [T, d]
    const float *a_scale;   // fp8: [T] or [T, d/128]
    const void *w13;
    const float *w13_scale;
    const int32_t *sorted_ids, *sorted_expert_ids, *num_valid;
    void *h;                // quant 0/1: bf16 [P, f]; quant 2: e4m3 [P, f]
    float *h_scale;         // quant 1: row amax [P] (zeroed by the caller); quant 2: [P, f/128]
    float *zero;            // optional: fp32 buffer [zero_n] the kernel clears on the way
    size_t zero_n;
    // quant 3 (MXFP4): a / w13 / h are E2M1 codes two per byte, with E8M0
    // scales a_mx [T, d/32], w13_mx [E, 2f, d/32], h_mx [P, f/32] (out)
    const uint8_t *a_mx, *w13_mx;
    uint8_t *h_mx;
    float *gu_out;          // optional (bf16): raw gate / up sums [P, 2f] fp32; the streaming
                            // kernel also writes h, the tiled kernel writes only these
    // streaming kernel, bf16: split K = d into ksplit parts whose raw gate /
    // up sums go to gu_part [parts][T*k, 2f] fp32 (by assignment); h is then
    // written by launch_swiglu_parts
    int ksplit;
    float *gu_part;
    // tiled kernel, bf16: w13 is stored [K][N] = [d][2f] (N contiguous; the
    // gate columns 0..f-1, the up columns f..2f-1) instead of [2f][d]
    bool w_kn;
};

// Parts the streaming bf16 GEMM1 launches for a requested K split.
int stream_gemm1_parts(int d, int ksplit);
// h[slot] = bf16(silu(sum_q g_q) * sum_q u_q) for the real slots (the parts
// q ascending; g, u from gu_part [parts][n_asg, 2f] at the slot's
// assignment); padding slots and slots past num_valid are left untouched.
hipError_t launch_swiglu_parts(const float *gu_part, int parts, int n_asg, int f, const int32_t *sorted_ids,
                               const int32_t *num_valid, int P, uint16_t *h, hipStream_t s);

struct Gemm2Args {
    GemmShape sh;
    int ksplit;
    const void *h;
    const float *h_scale;
    const void *w2;
    const float *w2_scale;
    const int32_t *sorted_ids;
    const float *sorted_w;
    const int32_t *sorted_expert_ids, *num_valid;
    float *acc;             // fp32 [T, d], zeroed by the caller
    float *yrows;           // tiled kernel: rows [parts][T*k, d] by K part and assignment instead of acc
                            // (sorted_w NULL: unit weights, streaming kernel)
    const uint8_t *h_mx, *w2_mx;   // quant 3: E8M0 scales [P, f/32] and [E, d, f/32]
    bool w_kn;              // tiled kernel, bf16: w2 stored [K][N] = [f][d] instead of [d][f]
};

// ---- backward of the bf16 layer (streaming kernel, B = 16 or 32)
hipError_t launch_stream_bwd_dh(const GemmShape &sh, const uint16_t *dy, const uint16_t *w2t,
                                const int32_t *sorted_ids, const float *sorted_w,
                                const int32_t *sorted_expert_ids, const float *gu,
                                const uint16_t *h, uint16_t *dgu, uint16_t *dgu_lo, float *dtw,
                                hipStream_t s);
// out[e] = in[e]^T for E matrices [R, C] bf16 (R, C multiples of 64)
hipError_t launch_transpose_bf16(const uint16_t *in, int E, int R, int C, uint16_t *out, hipStream_t s);
// Backward, tiled path: from the recomputed sums gu [P, 2f] and v = Wd^T dy
// [P, f] (fp32, slot order): h [P, f], dg / du as two bf16 parts (dgu,
// dgu_lo [P, 2f]) and dtw[a] += <v, h> (dtw zeroed by the caller).
hipError_t launch_bwd_swiglu(const float *gu, const float *v, const int32_t *sorted_ids,
                             const float *sorted_w, int P, int T, int k, int f, uint16_t *h, uint16_t *dgu,
                             uint16_t *dgu_lo, float *dtw, hipStream_t s);
// Weight gradient per expert as launch_wgrad below, for segments of whole
// 32-row chunks (the tiled path): operands by LDS DMA and transposing LDS
// reads. M a multiple of 128, N of 256. Precondition: every padding row of
// p_hi, p_lo and q inside an expert's padded segment [offsets[e],
// offsets[e+1]) is zero (k_bwd_swiglu and k_gather_bwd write those zeros),
// because whole chunks are summed, padding rows included.
hipError_t launch_wgrad_dma(const uint16_t *p_hi, const uint16_t *p_lo, const uint16_t *q, int M, int N, int E,
                            const int32_t *offsets, float *C, hipStream_t s);
// Backward: xs[slot] = x[t] and w[slot] dy[t] as two bf16 parts dz_hi + dz_lo
// (zeros for padding slots; P slots).
hipError_t launch_gather_bwd(const int32_t *sorted_ids, const float *sorted_w, int P, int T, int k,
                             int d, const uint16_t *x, const uint16_t *dy, uint16_t *xs, uint16_t *dz_hi,
                             uint16_t *dz_lo, hipStream_t s);
// Weight gradient per expert: C[e] [M, N] fp32 = sum over expert e's slots
// of (P_hi + P_lo)[slot]^T Q[slot] (bf16 rows in slot order; rows past the
// expert's count add nothing). M, N multiples of 4. short_segments: a variant with one LDS stage, for
// segments of a few chunks.
hipError_t launch_wgrad(const uint16_t *p_hi, const uint16_t *p_lo, const uint16_t *q, int M, int N, int E,
                        const int32_t *offsets, const int32_t *counts, bool short_segments, float *C,
                        hipStream_t s);

bool onestage_supported(const GemmShape &sh);
hipError_t launch_moe_1stage(const GemmShape &sh, const void *x, const void *w13, const void *w2,
                             const int32_t *sorted_ids, const float *sorted_w,
                             const int32_t *sorted_expert_ids, float *acc, hipStream_t s);

}  // namespace moe
