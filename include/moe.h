/*
 * moe.h -- C ABI of libmoe.so, a fused Mixture-of-Experts layer for AMD
 * Instinct MI355X (gfx950 / CDNA4).
 *
 * The layer (rocketrecap.com/entries/19116, talk summary at 5:58: grouped
 * GEMMs replace masked dense GEMMs for MoE; AITER walk-through at
 * itsolotime.com/th/archives/32381, section 1.2 data flow and section 3
 * "Fused MoE"):
 *
 *   logits --moe_topk--> topk_ids, topk_w
 *          --moe_sort--> expert-contiguous, block-padded assignment list
 *          --moe_gemm1_swiglu--> h = silu(x Wg) * (x Wu), one row per slot
 *          --moe_gemm2_combine--> out[t] = sum_j w[t,j] * (h Wd)[slot(t,j)]
 *
 * fused_moe runs the whole chain.
 *
 * Notation: T tokens, d hidden size, f expert FFN size, E experts, k experts
 * per token, B sort block size. The flat assignment index is a = t*k + j.
 * P = T*k + E*B - k is the padded slot count, and NB = ceil(P / B) the
 * block count (AITER walk-through, section 3.1, max_num_tokens_padded and
 * max_num_m_blocks).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers, allocated and owned by the caller. The
 *    library keeps none of them after the call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *    enqueue work on it: they never synchronise the host and never allocate.
 *    Scratch memory comes from the caller's `ws` of at least the size the
 *    matching *_workspace_bytes query returns (any alignment is accepted;
 *    256-byte alignment is best).
 *  - Arguments are validated on the host before any HIP call. Device-side
 *    preconditions (not checked): expert ids in [0, E) where the caller
 *    supplies them, and finite inputs. Ids outside [0, E) are skipped by the
 *    sort: they reach no out-of-bounds address, and the assignments that
 *    carry them add nothing to the layer's output.
 *  - Return value: MOE_OK, or an error code. Nothing aborts and nothing is
 *    thrown. moe_last_error() gives this thread's last error text.
 *  - Calls on one stream are ordered. Calls that share output or workspace
 *    buffers on different streams race.
 *
 * Formats:
 *  - bf16: IEEE bfloat16 (uint16 bit patterns). fp8: OCP E4M3FN codes
 *    (bias 7, max 448, no infinities).
 *  - quant = MOE_QUANT_BF16: bf16 activations and weights.
 *    quant = MOE_QUANT_FP8_TOKEN ("per_Token"): e4m3 weights with one fp32
 *    scale per output channel, and activations quantised per row at run time.
 *    quant = MOE_QUANT_FP8_BLOCK ("per_1x128"): e4m3 weights with one fp32
 *    scale per 128x128 block, and activations quantised per 1x128 block at
 *    run time. These quant-type names come from the AITER walk-through,
 *    sections 1.1 and 3.2. Dynamic quantisation uses s = amax / 448 (s = 1
 *    when amax = 0) and q = round-to-nearest-even of v / s, saturated to
 *    +-448.
 *    quant = MOE_QUANT_MXFP4 ("per_1x32", the MXFP4 quant type of the same
 *    sections): E2M1 weights and activations (values 0, 0.5, 1, 1.5, 2, 3,
 *    4, 6 and negatives), two codes per byte with the even element in the
 *    low nibble, and one E8M0 scale byte (2^(c - 127)) per 32 consecutive
 *    elements along the reduction dimension. Activations and h are
 *    quantised at run time as moe_quant_act_mx describes. d and f must be
 *    multiples of 256; sort blocks of 16 or 32 rows run on the
 *    weight-streaming kernels, blocks of 64, 128 or 256 rows on the
 *    LDS-tiled kernels, which need d and f multiples of 512.
 *  - Weights are laid out with the reduction dimension contiguous:
 *      w13 [E, 2f, d]: rows 0..f-1 are the gate projection, rows f..2f-1
 *                      the up projection;
 *      w2  [E, d, f];
 *      scales: per-channel w13_scale [E, 2f], w2_scale [E, d] (fp32);
 *              per-block   w13_scale [E, 2f/128, d/128],
 *                          w2_scale  [E, d/128, f/128] (fp32);
 *              MXFP4: w13 codes [E, 2f, d/2] with w13_scale [E, 2f, d/32],
 *                     w2 codes [E, d, f/2] with w2_scale [E, d, f/32]
 *                     (uint8 E8M0).
 *    Scale pointers are typed void: fp32 arrays for the e4m3 types, uint8
 *    arrays for MXFP4.
 *  - d and f must be multiples of 128.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum value       */
    MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. d % 128 != 0) */
    MOE_ERR_WORKSPACE = 3,   /* ws_bytes below the size the query returns    */
    MOE_ERR_HIP = 4          /* a HIP runtime call failed (see moe_last_error) */
};

enum moe_quant {
    MOE_QUANT_BF16 = 0,
    MOE_QUANT_FP8_TOKEN = 1,
    MOE_QUANT_FP8_BLOCK = 2,
    MOE_QUANT_MXFP4 = 3
};
enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };

/* Limits checked by every call. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/* Sizes of the sort buffers (AITER walk-through, section 3.1):
 * P = T*k + E*B - k and NB = ceil(P / B). Return -1 on invalid arguments
 * (T < 0, k < 1, k > E, B < 1). */
int64_t moe_sort_max_padded(int T, int k, int E, int B);
int64_t moe_sort_max_blocks(int T, int k, int E, int B);

/* Top-k routing: the gating stage at the head of the fused MoE pipeline
 * (AITER walk-through, section 3). For each token t the k experts with the
 * largest logit are chosen, ordered by (logit descending, expert ascending);
 * selection uses the raw logit. Their scores (score = MOE_SCORE_SOFTMAX:
 * softmax over all E logits; MOE_SCORE_SIGMOID: 1 / (1 + exp(-logit))) are
 * divided by their sum when renorm != 0.
 *   logits   [T, E] fp32 row-major (in)
 *   topk_ids [T, k] int32 (out), topk_w [T, k] fp32 (out)
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS. */
int moe_topk(const float *logits, int T, int E, int k, int score, int renorm,
             int32_t *topk_ids, float *topk_w, void *stream);

/* Token sort into expert-contiguous, block-padded groups (AITER
 * walk-through, section 3.1: tokens of one expert are made contiguous so
 * that its GEMM is dense, and every expert segment is padded to a multiple
 * of B so that tiled GEMMs need no tail handling). A stable counting sort of
 * the assignments a = t*k + j by expert:
 *   expert_counts[e]      = number of assignments to e             [E]
 *   expert_offsets[e]     = sum over e' < e of ceil(cnt[e']/B)*B   [E+1]
 *   num_valid[0]          = expert_offsets[E]                      [1]
 *   sorted_ids[i]         = a, in ascending a inside each expert's
 *                           segment; T*k in padding and in [num_valid, P) [P]
 *   sorted_w[i]           = topk_w.flat[a], 0.0f where sorted_ids = T*k [P]
 *   sorted_expert_ids[b]  = expert owning slots [b*B, b*B + B); -1 for
 *                           b >= num_valid / B                    [NB]
 * Every output element is written (whole buffers are deterministic).
 *   topk_ids [T, k] int32, topk_w [T, k] fp32 (in).
 * Requires T >= 0, 1 <= k <= E <= MOE_MAX_EXPERTS, 1 <= B <= 1024,
 * T*k <= 2^24. */
int moe_sort(const int32_t *topk_ids, const float *topk_w, int T, int k, int E, int B,
             int32_t *sorted_ids, float *sorted_w, int32_t *sorted_expert_ids,
             int32_t *expert_counts, int32_t *expert_offsets, int32_t *num_valid,
             void *stream);

/* Dynamic e4m3 quantisation of a bf16 matrix x [rows, cols], one scale per
 * `group` consecutive columns of a row (group = cols: per_Token;
 * group = 128: per_1x128; AITER walk-through, section 3.2 quant types).
 *   codes [rows, cols] uint8 (out), scales [rows, cols / group] fp32 (out).
 * Requires cols % group == 0 and group % 128 == 0 (or group == cols with
 * cols % 128 == 0). */
int moe_quant_act(const void *x, int rows, int cols, int group, uint8_t *codes, float *scales,
                  void *stream);

/* Dynamic MXFP4 quantisation (quant type per_1x32, AITER walk-through
 * sections 1.1 and 3.2) of a bf16 matrix x [rows, cols], cols % 32 == 0: for
 * each block of 32 consecutive columns, shared exponent
 * E = floor(log2(amax)) - 2 (-127 for an all-zero block), E2M1 codes of
 * x / 2^E rounded to nearest (ties to the even code) and saturated at +-6.
 *   codes [rows, cols / 2] uint8 (out): two codes per byte, the even column
 *   in the low nibble; scales [rows, cols / 32] uint8 (out): E8M0, E + 127. */
int moe_quant_act_mx(const void *x, int rows, int cols, uint8_t *codes, uint8_t *scales,
                     void *stream);

/* Grouped GEMM 1 with fused SwiGLU: stage 1 of the two-stage MoE (AITER
 * walk-through, section 3.2: gate + up projections and the activation). For
 * every used block b (expert e = sorted_expert_ids[b]) and slot
 * i in [b*B, b*B + B) with a = sorted_ids[i]:
 *   A_i = x[a / k] (zero when a = T*k),
 *   h[i, n] = bf16( silu(A_i . Wg_e[n]) * (A_i . Wu_e[n]) ),  n < f,
 * with fp32 accumulation. Blocks at or past num_valid / B are skipped (their
 * h rows are left untouched); the h (and h_scale) rows of padding slots
 * (sorted_ids[i] == T*k) are unspecified, and moe_gemm2_combine ignores them.
 *   x [T, d] bf16; w13 / w13_scale as in the header comment;
 *   sorted_ids [P], sorted_expert_ids [NB], num_valid [1] from moe_sort.
 *   quant BF16:       h [P, f] bf16, h_scale unused (may be NULL).
 *   quant FP8_TOKEN:  h [P, f] e4m3 codes of the bf16 h quantised per row,
 *                     h_scale [P].
 *   quant FP8_BLOCK:  h [P, f] e4m3 codes per 1x128 block, h_scale [P, f/128].
 *   quant MXFP4:      h [P, f/2] E2M1 codes of the bf16 h per 1x32 block,
 *                     h_scale [P, f/32] uint8 E8M0.
 *   For fp8 and MXFP4, x is quantised inside (into ws) with the matching group.
 * B must be 16, 32, 64, 128 or 256. */
size_t moe_gemm1_workspace_bytes(int T, int d, int f, int E, int k, int B, int quant);
int moe_gemm1_swiglu(int T, int d, int f, int E, int k, int B, int quant,
                     const void *x, const void *w13, const void *w13_scale,
                     const int32_t *sorted_ids, const int32_t *sorted_expert_ids,
                     const int32_t *num_valid, void *h, void *h_scale,
                     void *ws, size_t ws_bytes, void *stream);

/* Grouped GEMM 2 with the routing-weighted combine: stage 2 of the two-stage
 * MoE (down projection, AITER walk-through, section 3.2) followed by the
 * weighted combine that ends the pipeline (section 3). For every used slot i
 * with a = sorted_ids[i] != T*k:
 *   out[a / k, :] += sorted_w[i] * (h_i . Wd_e)
 * accumulated in fp32 in ws, then rounded once to bf16 into out [T, d]
 * (fully overwritten; a token with no assignment gets zeros). The reduction
 * over f may be split into `ksplit` parts whose partial sums are added into
 * the same accumulator (K-split, section 3.4); ksplit <= 0 lets the library
 * choose. The order of the fp32 additions is not specified.
 *   h / h_scale in the format moe_gemm1_swiglu writes for the same quant. */
size_t moe_gemm2_workspace_bytes(int T, int d, int f, int E, int k, int B, int quant);
int moe_gemm2_combine(int T, int d, int f, int E, int k, int B, int quant, int ksplit,
                      const void *h, const void *h_scale, const void *w2, const void *w2_scale,
                      const int32_t *sorted_ids, const float *sorted_w,
                      const int32_t *sorted_expert_ids, const int32_t *num_valid,
                      void *out, void *ws, size_t ws_bytes, void *stream);

/* The whole layer (AITER walk-through, section 1.2 data flow and section 3):
 * routing (skipped when logits is NULL: topk_ids / topk_w are then inputs),
 * sort, dynamic activation quantisation (fp8), then either the two-stage
 * path (stage = 2) or the one-stage kernel that runs gate/up, SwiGLU and the
 * down projection per (block, f-chunk) with the weighted scatter-add
 * (stage = 1). B = 0, stage = 0 and ksplit <= 0 let the library choose from
 * (T, d, f, E, k, quant) and the device's CU count. out [T, d] bf16 is fully
 * overwritten.
 *   The workspace query takes the same B / stage (0 = the library's choice). */
size_t fused_moe_workspace_bytes(int T, int d, int f, int E, int k, int quant, int B, int stage);
int fused_moe(int T, int d, int f, int E, int k, int quant, int score, int renorm,
              const float *logits, const int32_t *topk_ids, const float *topk_w,
              const void *x, const void *w13, const void *w13_scale,
              const void *w2, const void *w2_scale,
              int B, int stage, int ksplit, void *out, void *ws, size_t ws_bytes, void *stream);

/* fused_moe without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace is a static array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's device code, one per GPU,
 * present from the library's first use on that GPU until the process ends;
 * the call allocates nothing. Layers whose fused_moe workspace (the query
 * fused_moe_workspace_bytes) exceeds that size are refused with
 * MOE_ERR_UNSUPPORTED before any device work. Every call on one GPU uses the
 * same array (the previous call's contents are overwritten; nothing in it
 * needs to start at zero), so calls that overlap on one GPU, on different
 * streams or host threads, race: order them on one stream. Arguments,
 * results and errors are otherwise those of fused_moe. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int fused_moe_noalloc(int T, int d, int f, int E, int k, int quant, int score, int renorm,
                      const float *logits, const int32_t *topk_ids, const float *topk_w,
                      const void *x, const void *w13, const void *w13_scale,
                      const void *w2, const void *w2_scale,
                      int B, int stage, int ksplit, void *out, void *stream);

/* The library's choice of block size B, stage and K-split for a shape
 * (AITER walk-through, sections 3.2 to 3.4 describe the choices; the rule
 * here is this library's own, from measurement on MI355X). cu_count <= 0
 * uses the current device's. Host-only: touches no device memory. */
int moe_select_config(int T, int d, int f, int E, int k, int quant, int cu_count,
                      int *B, int *stage, int *ksplit);

/* Backward of the bf16 layer (the training step named as the next milestone:
 * rocketrecap.com/entries/19116, talk summary at 10:07; entries/19188, the
 * custom VJP of the JAX bridge). For a given routing (topk_ids / topk_w, as
 * the forward used them) and the output gradient dy, computes
 *   dx [T, d] bf16, dw13 [E, 2f, d] fp32, dw2 [E, d, f] fp32 (all experts;
 *   zero for experts no token selects) and dtopk_w [T, k] fp32 (the gradient
 *   of each assignment's routing weight: <dy[t], Wd h>),
 * from the chain rule of the forward: dz = w dy, dh = Wd^T dz,
 * dg = dh u silu'(g), du = dh silu(g), dx = Wg^T dg + Wu^T du,
 * dWd = sum dz h^T, dWg = sum dg x^T, dWu = sum du x^T. h is the forward's
 * bf16 h; its rounding passes the gradient unchanged. The gate / up sums are
 * recomputed (a second GEMM1), the weights are transposed into the workspace
 * per call, and the weight gradients reduce over each expert's rows of the
 * sorted assignment list. bf16 only. B = 16 or 32 runs the GEMMs on the
 * streaming kernels; B = 64, 128 or 256 on the tiled kernels (d and f
 * multiples of 256, else MOE_ERR_UNSUPPORTED); B = 0 lets the library choose
 * (tiled from 2 assignments per expert on average where d and f allow).
 * Layouts and ownership as in fused_moe; every output is overwritten. */
size_t moe_backward_workspace_bytes(int T, int d, int f, int E, int k, int B);
int moe_backward(int T, int d, int f, int E, int k, int B, const void *x,
                 const int32_t *topk_ids, const float *topk_w, const void *w13,
                 const void *w2, const void *dy, void *dx, float *dw13, float *dw2,
                 float *dtopk_w, void *ws, size_t ws_bytes, void *stream);

/* Tuned configurations (AITER walk-through, section 4.1: a table of tuned
 * configurations measured offline and keyed by shape, looked up with a fuzzy
 * match on the token count). Loads a CSV of rows
 *     cu,T,d,f,E,k,quant,B,stage,ksplit[,more columns ignored]
 * (quant: bf16, fp8_token, fp8_block, mxfp4 or 0..3; lines starting with '#'
 * and a header line are skipped) and replaces the process-wide table.
 * While a table is loaded, moe_select_config and every B = 0 / stage = 0 /
 * ksplit <= 0 choice take the row with the same (cu, d, f, E, k, quant)
 * whose T is the smallest at or above the call's T (else the largest T);
 * shapes without such a row keep the built-in rule. A K-split from the table
 * is used only with the row's own B.
 *   path: a host string; NULL clears the table. rows (may be NULL): the
 * number of rows loaded. Returns MOE_ERR_INVALID_ARG for an unreadable file
 * or a malformed row and MOE_ERR_UNSUPPORTED for a row no kernel can run
 * (moe_last_error names the line); the table in use is then left unchanged.
 * Host-only; thread-safe against concurrent lookups. */
int moe_load_config_table(const char *path, int *rows);

const char *moe_status_string(int status);
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
