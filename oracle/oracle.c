/*
 * oracle.c — plain CPU oracle of the fused Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The GPU library never
 * links, includes or calls it, and this file shares no code, header, table or
 * helper with it.
 *
 * What it computes, and where the pages define it:
 *  - oracle_route: top-k gating, the first stage of the fused MoE pipeline
 *    (AITER article, itsolotime.com/th/archives/32381, section 3 "Fused MoE",
 *    pipeline gating -> token re-sort -> expert GEMMs -> weighted combine).
 *    The scoring (softmax or sigmoid, renormalised over the selected k) is the
 *    plain reading of "top-k of softmax(router logits) renormalised".
 *  - oracle_sort: the token sort of section 3.1 of the same article. Buffer
 *    sizes follow its max_num_tokens_padded / max_num_m_blocks formulas.
 *    Inside an expert, assignments keep ascending flat order (stable sort);
 *    padding and tail slots hold the sentinel T*k with weight 0; blocks past
 *    the last used one get expert id -1.
 *  - oracle_moe: the MoE FFN written as a per-token loop over the selected
 *    experts in fp32 (one accumulator per dot product, ascending index, no
 *    contraction into FMA). SwiGLU is silu(x Wg) * (x Wu) followed by Wd
 *    (rocketrecap.com/entries/19116 talk summary, glossary "SwiGLU"; MoE GEMMs
 *    at 5:58). The intermediate h is rounded to bf16; fp8 layers then
 *    re-quantise that bf16 h (per row, or per 1x128 block) before the down
 *    projection, and quantise the input row the same way.
 *    The sum order of an fp32 dot product is not fixed by the pages, so an
 *    h whose fp32 value lies within rounding noise of the midpoint between
 *    two bfloat16 values may round either way; where the other rounding
 *    would change its quantisation group's scale (the largest magnitude, or
 *    the MXFP4 shared exponent), every code of the group moves, and where it
 *    would change the element's own code, that code moves. oracle_moe
 *    reports such elements (tie_band > 0) and can round listed elements to
 *    the other neighbour (h_flip), so that a test can bound what these
 *    readings allow.
 *  - oracle_e4m3_encode / _decode / oracle_quant_group: the OCP FP8 E4M3FN
 *    format (bias 7, 3 mantissa bits, max 448, no infinities, S.1111.111 is
 *    NaN) and the scale rule s = amax / 448 (s = 1 when amax = 0),
 *    q = round-to-nearest-even, saturating encode of v / s.
 *  - oracle_fp4_encode / _decode / oracle_mx_quant_group: MXFP4, the
 *    microscaling 4-bit float that the pages name as quant type per_1x32
 *    (AITER article, sections 1.1, 3.2 and the gfx950 FP4 build flag of 2.2;
 *    rocketrecap.com/entries/19188 glossary "MXFP4"). The pages give no
 *    numerics; this follows the published OCP MX format: E2M1 elements
 *    (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), 32 consecutive
 *    elements share one E8M0 scale 2^(c - 127), the shared exponent is
 *    floor(log2(amax)) - 2 (2 = exponent of the largest E2M1 value; -127
 *    for an all-zero block), elements are round-to-nearest-even of v / 2^E,
 *    saturating at +-6.
 *  - oracle_moe_backward: the gradients of the bf16 layer (the training
 *    step the pages name as the next milestone: rocketrecap.com/entries/
 *    19116, 10:07; entries/19188, custom VJP). Written from the chain rule of
 *    the forward above, one token at a time in fp32: dz = w dy,
 *    dh = Wd^T dz, dg = dh * u * silu'(g), du = dh * silu(g),
 *    dx = Wg^T dg + Wu^T du, dWd += dz h^T, dWg += dg x^T, dWu += du x^T,
 *    dw = <dy, Wd h>. The bf16 rounding of h passes the gradient unchanged
 *    (a cast's derivative is taken as 1, as automatic differentiation of a
 *    dtype conversion does).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no BLAS, no
 * fast-math). Every exported function returns 0 on success and a negative
 * value on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* scalar formats                                                      */
/* ------------------------------------------------------------------ */

static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE round-to-nearest-even of an fp32 value to bfloat16 (1-8-7). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN stays a quiet NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

static float round_to_bf16(float f) { return bf16_bits_to_f32(oracle_f32_to_bf16(f)); }

/* The bfloat16 value adjacent to r (a finite bfloat16 value) on the side
 * of v: one step of the 7-bit mantissa up or down. */
static float bf16_neighbour(float r, float v)
{
    uint32_t u;
    memcpy(&u, &r, sizeof u);
    uint16_t b = (uint16_t)(u >> 16);
    const int up = v > r;
    if (r == 0.0f)
        b = up ? 0x0001u : 0x8001u;
    else if ((r > 0.0f) == up)
        b = (uint16_t)(b + 1u); /* away from zero */
    else
        b = (uint16_t)(b - 1u); /* toward zero */
    return bf16_bits_to_f32(b);
}

/* OCP E4M3FN decode: value = (-1)^s * 2^(e-7) * (1 + m/8) for e > 0,
 * (-1)^s * 2^-6 * (m/8) for e = 0, NaN for e = 15, m = 7. */
float oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

/* OCP E4M3FN encode, round to nearest, ties to even, saturating at +-448. */
uint8_t oracle_e4m3_encode(float v)
{
    if (isnan(v))
        return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7e);
    if (a == 0.0)
        return sign;
    /* spacing of representable values around a: 2^(binade-3), with the
     * binade clamped at -6 (subnormals are spaced 2^-9). */
    int ex;
    frexp(a, &ex);
    int binade = ex - 1;
    if (binade < -6)
        binade = -6;
    double quantum = ldexp(1.0, binade - 3);
    double r = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
    if (r == 0.0)
        return sign;
    frexp(r, &ex);
    binade = ex - 1;
    if (binade < -6) /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    int mant = (int)(r / ldexp(1.0, binade) * 8.0) - 8;
    return (uint8_t)(sign | ((binade + 7) << 3) | mant);
}

/* MXFP4 E2M1 decode: bit 3 sign, bits 2..1 exponent e (bias 1), bit 0
 * mantissa m: value = 2^(e-1) * (1 + m/2) for e > 0, m/2 for e = 0. */
float oracle_fp4_decode(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -v : v);
}

/* E2M1 encode: round to nearest, ties to the even code (mantissa 0),
 * saturating at +-6. The format has no NaN; NaN encodes as +-6. */
uint8_t oracle_fp4_encode(float v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (isnan(v) || a >= 6.0)
        return (uint8_t)(sign | 7);
    /* spacing of representable values: 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; the even
     * multiples of the spacing are exactly the codes with mantissa 0 */
    double q = (a < 2.0) ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
    double r = nearbyint(a / q) * q; /* default mode: ties to even */
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (int c = 0; c < 8; ++c)
        if (r == mag[c])
            return (uint8_t)(sign | c);
    return (uint8_t)(sign | 7); /* not reached */
}

/* One MXFP4 block of n values (n = 32 in the layer): shared exponent
 * E = floor(log2(amax)) - 2, clamped to [-127, 127], and -127 when amax is 0;
 * q_i = encode(v_i / 2^E). Writes the codes to q (one per byte, if not NULL)
 * and the dequantised values decode(q_i) * 2^E to deq (if not NULL); returns
 * the E8M0 scale code E + 127. */
uint8_t oracle_mx_quant_group(const float *v, int n, uint8_t *q, float *deq)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    int E = -127;
    if (amax > 0.0f) {
        int ex;
        frexp((double)amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) */
        E = (ex - 1) - 2;
        if (E < -127)
            E = -127;
        if (E > 127)
            E = 127;
    }
    for (int i = 0; i < n; ++i) {
        uint8_t c = oracle_fp4_encode((float)ldexp((double)v[i], -E));
        if (q)
            q[i] = c;
        if (deq)
            deq[i] = (float)ldexp((double)oracle_fp4_decode(c), E);
    }
    return (uint8_t)(E + 127);
}

/* Quantise n values that share one scale. s = amax / 448 in fp32 (s = 1 if
 * amax is 0), q_i = encode(v_i / s). Writes the codes to q (if not NULL),
 * the dequantised values fp32(decode(q_i)) * s to deq (if not NULL) and
 * returns s. */
float oracle_quant_group(const float *v, int n, uint8_t *q, float *deq)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    for (int i = 0; i < n; ++i) {
        uint8_t c = oracle_e4m3_encode(v[i] / s);
        if (q)
            q[i] = c;
        if (deq)
            deq[i] = oracle_e4m3_decode(c) * s;
    }
    return s;
}

/* ------------------------------------------------------------------ */
/* routing                                                             */
/* ------------------------------------------------------------------ */

/* score: 0 = softmax over all E logits, 1 = sigmoid of each logit.
 * renorm: 1 = divide the k selected scores by their sum.
 * Selection is on the raw logit, ordered by (logit descending, expert
 * ascending); topk_ids[t, j] lists the selected experts in that order. */
int oracle_route(const float *logits, int T, int E, int k, int score, int renorm,
                 int32_t *topk_ids, float *topk_w)
{
    if (!logits || !topk_ids || !topk_w || T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    if (score != 0 && score != 1)
        return -1;
    char *taken = (char *)malloc((size_t)E);
    float *p = (float *)malloc(sizeof(float) * (size_t)E);
    if (!taken || !p) {
        free(taken);
        free(p);
        return -2;
    }
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            topk_ids[(size_t)t * k + j] = best;
        }
        if (score == 0) {
            float m = l[0];
            for (int e = 1; e < E; ++e)
                if (l[e] > m)
                    m = l[e];
            float den = 0.0f;
            for (int e = 0; e < E; ++e)
                den += expf(l[e] - m);
            for (int e = 0; e < E; ++e)
                p[e] = expf(l[e] - m) / den;
        } else {
            for (int e = 0; e < E; ++e)
                p[e] = 1.0f / (1.0f + expf(-l[e]));
        }
        float sum = 0.0f;
        for (int j = 0; j < k; ++j)
            sum += p[topk_ids[(size_t)t * k + j]];
        for (int j = 0; j < k; ++j) {
            float pj = p[topk_ids[(size_t)t * k + j]];
            topk_w[(size_t)t * k + j] = renorm ? pj / sum : pj;
        }
    }
    free(taken);
    free(p);
    return 0;
}

/* ------------------------------------------------------------------ */
/* token sort                                                          */
/* ------------------------------------------------------------------ */

int64_t oracle_max_padded(int T, int k, int E, int B)
{
    return (int64_t)T * k + (int64_t)E * B - k;
}

int64_t oracle_max_blocks(int T, int k, int E, int B)
{
    int64_t P = oracle_max_padded(T, k, E, B);
    return (P + B - 1) / B;
}

/* Stable counting sort of the T*k assignments a = t*k + j by expert, each
 * expert's segment padded up to a multiple of B. Outputs:
 *   sorted_ids [P], sorted_w [P], sorted_expert_ids [NB],
 *   expert_counts [E], expert_offsets [E+1] (padded), num_valid [1]. */
int oracle_sort(const int32_t *topk_ids, const float *topk_w, int T, int k, int E, int B,
                int32_t *sorted_ids, float *sorted_w, int32_t *sorted_expert_ids,
                int32_t *expert_counts, int32_t *expert_offsets, int32_t *num_valid)
{
    if (!topk_ids || !topk_w || !sorted_ids || !sorted_w || !sorted_expert_ids ||
        !expert_counts || !expert_offsets || !num_valid)
        return -1;
    if (T < 0 || k < 1 || E < k || B < 1)
        return -1;
    const int64_t N = (int64_t)T * k;
    const int64_t P = oracle_max_padded(T, k, E, B);
    const int64_t NB = oracle_max_blocks(T, k, E, B);
    for (int64_t a = 0; a < N; ++a)
        if (topk_ids[a] < 0 || topk_ids[a] >= E)
            return -1;

    for (int e = 0; e < E; ++e)
        expert_counts[e] = 0;
    for (int64_t a = 0; a < N; ++a)
        expert_counts[topk_ids[a]] += 1;

    expert_offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int32_t padded = (expert_counts[e] + B - 1) / B * B;
        expert_offsets[e + 1] = expert_offsets[e] + padded;
    }
    *num_valid = expert_offsets[E];
    if (*num_valid > P)
        return -3; /* cannot happen when k <= E */

    for (int64_t i = 0; i < P; ++i) {
        sorted_ids[i] = (int32_t)N;
        sorted_w[i] = 0.0f;
    }
    for (int64_t b = 0; b < NB; ++b)
        sorted_expert_ids[b] = -1;

    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor)
        return -2;
    for (int e = 0; e < E; ++e)
        cursor[e] = expert_offsets[e];
    for (int64_t a = 0; a < N; ++a) {
        int e = topk_ids[a];
        sorted_ids[cursor[e]] = (int32_t)a;
        sorted_w[cursor[e]] = topk_w[a];
        cursor[e] += 1;
    }
    free(cursor);

    for (int e = 0; e < E; ++e)
        for (int32_t b = expert_offsets[e] / B; b < expert_offsets[e + 1] / B; ++b)
            sorted_expert_ids[b] = e;
    return 0;
}

/* ------------------------------------------------------------------ */
/* the MoE FFN, one token at a time                                     */
/* ------------------------------------------------------------------ */

/* quant: 0 = bf16 operands; 1 = e4m3 weights with one fp32 scale per output
 * channel and e4m3 activations with one scale per row; 2 = e4m3 weights with
 * one scale per 128x128 block and activations with one scale per 1x128 block;
 * 3 = MXFP4 weights and activations (E2M1 codes, one E8M0 scale per 32
 * consecutive elements along the reduction dimension).
 * Weights are given per expert (entries of unused experts may be NULL):
 *   w13[e]: [2f, d] (rows 0..f-1 gate, f..2f-1 up), d contiguous,
 *           scales fp32 [2f] (quant 1) or [2f/128, d/128] (quant 2);
 *           quant 3: codes packed two per byte [2f, d/2] (even column in the
 *           low nibble), E8M0 scales uint8 [2f, d/32];
 *   w2[e]:  [d, f], f contiguous, scales [d] or [d/128, f/128]; quant 3:
 *           codes [d, f/2], scales [d, f/32].
 * h_exact = 1 skips the rounding of h (pinning use only). */
typedef struct {
    int d, f, quant;
    const void *w13, *w2;
    const void *s13, *s2;
} expert_view;

/* element (row, col) of an MXFP4 matrix with `cols` columns */
static float mx_elem(const void *codes, const void *scales, int cols, int row, int col)
{
    uint8_t byte = ((const uint8_t *)codes)[(size_t)row * (cols / 2) + col / 2];
    uint8_t c = (col & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    int e = (int)((const uint8_t *)scales)[(size_t)row * (cols / 32) + col / 32] - 127;
    return (float)ldexp((double)oracle_fp4_decode(c), e);
}

static float weight13(const expert_view *v, int row, int col)
{
    size_t idx = (size_t)row * v->d + col;
    if (v->quant == 0)
        return bf16_bits_to_f32(((const uint16_t *)v->w13)[idx]);
    if (v->quant == 3)
        return mx_elem(v->w13, v->s13, v->d, row, col);
    const float *sc = (const float *)v->s13;
    float code = oracle_e4m3_decode(((const uint8_t *)v->w13)[idx]);
    float s = (v->quant == 1) ? sc[row] : sc[(size_t)(row / 128) * (v->d / 128) + col / 128];
    return code * s;
}

static float weight2(const expert_view *v, int row, int col)
{
    size_t idx = (size_t)row * v->f + col;
    if (v->quant == 0)
        return bf16_bits_to_f32(((const uint16_t *)v->w2)[idx]);
    if (v->quant == 3)
        return mx_elem(v->w2, v->s2, v->f, row, col);
    const float *sc = (const float *)v->s2;
    float code = oracle_e4m3_decode(((const uint8_t *)v->w2)[idx]);
    float s = (v->quant == 1) ? sc[row] : sc[(size_t)(row / 128) * (v->f / 128) + col / 128];
    return code * s;
}

/* Row `row` of an expert matrix with `cols` columns as fp32 operand values:
 * the same value weight13 / weight2 give for each element (bf16 converted
 * exactly; e4m3 code value times its fp32 scale; E2M1 code value times
 * 2^(c - 127)), taken once per row so that a dot product reads a plain
 * array. e4m3_tab / fp4_tab hold oracle_e4m3_decode / oracle_fp4_decode of
 * every code. For an MXFP4
 * block with c in [0, 254] the product of the code value and the fp32 2^e
 * is exact (at most 3 significant bits, no underflow below 2^-149) or
 * overflows to infinity, as the double-precision ldexp of mx_elem does once
 * converted to fp32; the E8M0 NaN code 255 goes through mx_elem itself. */
static void weight_row(const void *w, const void *s, int quant, int cols, int row,
                       const float *e4m3_tab, const float *fp4_tab, float *out)
{
    const size_t base = (size_t)row * cols;
    if (quant == 0) {
        for (int c = 0; c < cols; ++c)
            out[c] = bf16_bits_to_f32(((const uint16_t *)w)[base + c]);
    } else if (quant == 3) {
        const uint8_t *sc = (const uint8_t *)s + (size_t)row * (cols / 32);
        for (int b = 0; b < cols / 32; ++b) {
            const int e = (int)sc[b] - 127;
            if (e > 127) {
                for (int c = 32 * b; c < 32 * b + 32; ++c)
                    out[c] = mx_elem(w, s, cols, row, c);
                continue;
            }
            const float p2 = (float)ldexp(1.0, e);
            const uint8_t *bytes = (const uint8_t *)w + base / 2 + 16 * (size_t)b;
            for (int i = 0; i < 16; ++i) {   /* even column in the low nibble */
                out[32 * b + 2 * i] = fp4_tab[bytes[i] & 15] * p2;
                out[32 * b + 2 * i + 1] = fp4_tab[bytes[i] >> 4] * p2;
            }
        }
    } else {
        const float *sc = (const float *)s;
        const uint8_t *q = (const uint8_t *)w + base;
        for (int c = 0; c < cols; ++c) {
            const float scale = (quant == 1) ? sc[row] : sc[(size_t)(row / 128) * (cols / 128) + c / 128];
            out[c] = e4m3_tab[q[c]] * scale;
        }
    }
}

/* Replace v[0..n) by its quantise-dequantise image: one group (quant 1),
 * groups of 128 (quant 2) or MXFP4 blocks of 32 (quant 3). */
static void fake_quant(float *v, int n, int quant)
{
    if (quant == 3) {
        for (int i = 0; i < n; i += 32)
            oracle_mx_quant_group(v + i, 32, NULL, v + i);
        return;
    }
    int g = (quant == 1) ? n : 128;
    for (int i = 0; i < n; i += g)
        oracle_quant_group(v + i, g, NULL, v + i);
}

static float silu(float z) { return z / (1.0f + expf(-z)); }

/* What fixes a quantisation group's scale, from its largest magnitude a:
 * a itself for the e4m3 formats (s = a / 448), the shared exponent of
 * oracle_mx_quant_group for MXFP4. */
static double group_scale_key(int quant, float a)
{
    if (quant != 3)
        return a;
    if (a == 0.0f)
        return -127.0;
    int ex;
    frexp((double)a, &ex);
    int E = (ex - 1) - 2;
    return E < -127 ? -127.0 : (E > 127 ? 127.0 : (double)E);
}

/* Is key in the ascending list a[0..n)? */
static int listed(const int64_t *a, int64_t n, int64_t key)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < key)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo < n && a[lo] == key;
}

/* Elements of one assignment's h (f values, bf16-rounded in h, fp32 before
 * rounding in hpre) whose fp32 value lies within band * |value| of the
 * midpoint between its bf16 rounding and the adjacent bf16 value, and whose
 * rounding to that other value would change the scale of its group (f
 * values for quant 1, 128 for quant 2, 32 for quant 3) or, under the same
 * scale, its own code. Appends base + n for each; *n_ties counts them all,
 * ties[] keeps the first max_ties. */
static void find_ties(const float *h, const float *hpre, int f, int quant, float band, int64_t base,
                      int64_t *ties, int64_t max_ties, int64_t *n_ties)
{
    const int g = (quant == 1) ? f : (quant == 2 ? 128 : 32);
    for (int g0 = 0; g0 < f; g0 += g) {
        float a1 = 0.0f, a2 = 0.0f; /* largest and second largest magnitude */
        int i1 = -1;
        for (int n = g0; n < g0 + g; ++n) {
            const float a = fabsf(h[n]);
            if (a > a1) {
                a2 = a1;
                a1 = a;
                i1 = n;
            } else if (a > a2) {
                a2 = a;
            }
        }
        const double key = group_scale_key(quant, a1);
        /* the group's scale: a1 / 448 (e4m3), 2^key (MXFP4) */
        const float s = (quant == 3) ? 1.0f : (a1 == 0.0f ? 1.0f : a1 / 448.0f);
        for (int n = g0; n < g0 + g; ++n) {
            const float r = h[n], v = hpre[n];
            if (v == r)
                continue;
            const float o = bf16_neighbour(r, v);
            const float mid = 0.5f * (r + o); /* exact: r and o are adjacent bf16 values */
            if (fabsf(v - mid) > band * fabsf(v))
                continue;
            const float others = (n == i1) ? a2 : a1;
            int moves = group_scale_key(quant, fmaxf(others, fabsf(o))) != key;
            if (!moves && quant == 3)
                moves = oracle_fp4_encode((float)ldexp((double)r, -(int)key)) !=
                        oracle_fp4_encode((float)ldexp((double)o, -(int)key));
            else if (!moves)
                moves = oracle_e4m3_encode(r / s) != oracle_e4m3_encode(o / s);
            if (!moves)
                continue;
            int64_t at;
#ifdef _OPENMP
#pragma omp atomic capture
#endif
            at = (*n_ties)++;
            if (at < max_ties)
                ties[at] = base + n;
        }
    }
}

/* The layer output for the rows tokens[0..n_tokens): y fp32 [n_tokens, d]
 * and its bf16 rounding out. h_exact = 1 keeps h in fp32 and unquantised.
 * Element n of the h of assignment (tokens[i], j) has the flat index
 * (i * k + j) * f + n. h_flip (ascending, n_flip entries) lists elements
 * rounded to the other of their two nearest bf16 values; tie_band > 0
 * writes the elements find_ties reports to ties (at most max_ties) and
 * their count to *n_ties. */
int oracle_moe(int T, int d, int f, int E, int k, int quant, int h_exact,
               const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
               const void *const *w13, const void *const *w13_scale,
               const void *const *w2, const void *const *w2_scale,
               const int32_t *tokens, int n_tokens, float *y, uint16_t *out, int nthreads,
               const int64_t *h_flip, int64_t n_flip, float tie_band, int64_t *ties,
               int64_t max_ties, int64_t *n_ties)
{
    if (!x || !topk_ids || !topk_w || !w13 || !w2 || !tokens || !y || !out)
        return -1;
    if (n_flip < 0 || (n_flip > 0 && !h_flip) || !(tie_band >= 0.0f))
        return -1;
    if (tie_band > 0.0f && (!ties || !n_ties || max_ties < 0))
        return -1;
    if (n_ties)
        *n_ties = 0;
    if (T < 0 || d < 1 || f < 1 || E < 1 || k < 1 || k > E || n_tokens < 0)
        return -1;
    if (quant < 0 || quant > 3)
        return -1;
    if (quant != 0 && (!w13_scale || !w2_scale))
        return -1;
    if (quant == 2 && (d % 128 || f % 128))
        return -1;
    if (quant == 3 && (d % 32 || f % 32))
        return -1;
    for (int i = 0; i < n_tokens; ++i) {
        int t = tokens[i];
        if (t < 0 || t >= T)
            return -1;
        for (int j = 0; j < k; ++j) {
            int e = topk_ids[(size_t)t * k + j];
            if (e < 0 || e >= E || !w13[e] || !w2[e] || (quant && (!w13_scale[e] || !w2_scale[e])))
                return -1;
        }
    }
    float e4m3_tab[256], fp4_tab[16];
    for (int c = 0; c < 256; ++c)
        e4m3_tab[c] = oracle_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 16; ++c)
        fp4_tab[c] = oracle_fp4_decode((uint8_t)c);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int i = 0; i < n_tokens; ++i) {
        const int t = tokens[i];
        float *xt = (float *)malloc(sizeof(float) * (size_t)d);
        float *h = (float *)malloc(sizeof(float) * (size_t)f);
        float *hpre = (float *)malloc(sizeof(float) * (size_t)f); /* h before its bf16 rounding */
        /* one weight row at a time: gate row, up row (d each), down row (f) */
        float *wrow = (float *)malloc(sizeof(float) * (size_t)(2 * d + f));
        float *yt = y + (size_t)i * d;
        if (!xt || !h || !hpre || !wrow) {
            free(xt);
            free(h);
            free(hpre);
            free(wrow);
            bad |= 1;
            continue;
        }
        for (int c = 0; c < d; ++c)
            xt[c] = bf16_bits_to_f32(x[(size_t)t * d + c]);
        if (quant)
            fake_quant(xt, d, quant);
        for (int m = 0; m < d; ++m)
            yt[m] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int e = topk_ids[(size_t)t * k + j];
            const float w = topk_w[(size_t)t * k + j];
            const void *s13 = quant ? w13_scale[e] : NULL, *s2 = quant ? w2_scale[e] : NULL;
            float *wg = wrow, *wu = wrow + d, *wd = wrow + 2 * d;
            for (int n = 0; n < f; ++n) {
                weight_row(w13[e], s13, quant, d, n, e4m3_tab, fp4_tab, wg);
                weight_row(w13[e], s13, quant, d, f + n, e4m3_tab, fp4_tab, wu);
                float g = 0.0f, u = 0.0f;
                for (int c = 0; c < d; ++c) {
                    g += xt[c] * wg[c];
                    u += xt[c] * wu[c];
                }
                const float hn = silu(g) * u;
                float r = round_to_bf16(hn);
                /* listed elements take the other of the two nearest bf16 values */
                if (n_flip && r != hn && listed(h_flip, n_flip, ((int64_t)i * k + j) * f + n))
                    r = bf16_neighbour(r, hn);
                hpre[n] = hn;
                h[n] = h_exact ? hn : r;
            }
            if (quant && !h_exact && tie_band > 0.0f)
                find_ties(h, hpre, f, quant, tie_band, ((int64_t)i * k + j) * f, ties, max_ties, n_ties);
            if (quant && !h_exact)
                fake_quant(h, f, quant);
            for (int m = 0; m < d; ++m) {
                weight_row(w2[e], s2, quant, f, m, e4m3_tab, fp4_tab, wd);
                float z = 0.0f;
                for (int n = 0; n < f; ++n)
                    z += h[n] * wd[n];
                yt[m] += w * z;
            }
        }
        for (int m = 0; m < d; ++m)
            out[(size_t)i * d + m] = oracle_f32_to_bf16(yt[m]);
        free(xt);
        free(h);
        free(hpre);
        free(wrow);
    }
    return bad ? -2 : 0;
}

static float silu_grad(float z)
{
    const float sg = 1.0f / (1.0f + expf(-z));
    return sg * (1.0f + z * (1.0f - sg));
}

/* Backward of the bf16 layer (quant 0) for every token.
 * In: x [T, d] bf16, topk_ids / topk_w [T, k], weights per expert as in
 * oracle_moe (bf16 bits; unused experts may be NULL), dy [T, d] bf16 bits,
 * h_exact as in oracle_moe.
 * Out (overwritten): dx [T, d] fp32; dw13[e] [2f, d] and dw2[e] [d, f] fp32
 * for every expert whose pointer is non-NULL (zero for experts no token
 * selects); dtopk_w [T, k] fp32.
 * Per-token work runs in parallel; the weight gradients are then summed per
 * expert over tokens in ascending order, so the result does not depend on
 * the thread count. */
int oracle_moe_backward(int T, int d, int f, int E, int k, int h_exact, const uint16_t *x,
                        const int32_t *topk_ids, const float *topk_w,
                        const void *const *w13, const void *const *w2, const uint16_t *dy,
                        float *dx, float *const *dw13, float *const *dw2, float *dtopk_w,
                        int nthreads)
{
    if (!x || !topk_ids || !topk_w || !w13 || !w2 || !dy || !dx || !dw13 || !dw2 || !dtopk_w)
        return -1;
    if (T < 0 || d < 1 || f < 1 || E < 1 || k < 1 || k > E)
        return -1;
    for (size_t a = 0; a < (size_t)T * k; ++a) {
        int e = topk_ids[a];
        if (e < 0 || e >= E || !w13[e] || !w2[e])
            return -1;
    }
    const size_t n_asg = (size_t)T * k;
    /* per assignment: dz [d], h [f], dg [f], du [f] */
    float *dz = (float *)malloc(sizeof(float) * (n_asg * d + 3 * n_asg * f + 1));
    if (!dz)
        return -2;
    float *hh = dz + n_asg * d, *dg = hh + n_asg * f, *du = dg + n_asg * f;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int t = 0; t < T; ++t) {
        float *xt = (float *)malloc(sizeof(float) * (size_t)(2 * d + 3 * f));
        if (!xt) {
            bad |= 1;
            continue;
        }
        float *dyt = xt + d, *g = dyt + d, *u = g + f, *dh = u + f;
        for (int c = 0; c < d; ++c) {
            xt[c] = bf16_bits_to_f32(x[(size_t)t * d + c]);
            dyt[c] = bf16_bits_to_f32(dy[(size_t)t * d + c]);
            dx[(size_t)t * d + c] = 0.0f;
        }
        for (int j = 0; j < k; ++j) {
            const size_t a = (size_t)t * k + j;
            const int e = topk_ids[a];
            const float w = topk_w[a];
            expert_view v = {d, f, 0, w13[e], w2[e], NULL, NULL};
            float *h = hh + a * f, *dga = dg + a * f, *dua = du + a * f, *dza = dz + a * d;
            for (int n = 0; n < f; ++n) {
                float gs = 0.0f, us = 0.0f;
                for (int c = 0; c < d; ++c) {
                    gs += xt[c] * weight13(&v, n, c);
                    us += xt[c] * weight13(&v, f + n, c);
                }
                g[n] = gs;
                u[n] = us;
                const float hn = silu(gs) * us;
                h[n] = h_exact ? hn : round_to_bf16(hn);
            }
            /* dw = <dy, Wd h>; dz = w dy; dh = Wd^T dz */
            float dw = 0.0f;
            for (int m = 0; m < d; ++m) {
                float z = 0.0f;
                for (int n = 0; n < f; ++n)
                    z += h[n] * weight2(&v, m, n);
                dw += dyt[m] * z;
                dza[m] = w * dyt[m];
            }
            dtopk_w[a] = dw;
            for (int n = 0; n < f; ++n) {
                float s = 0.0f;
                for (int m = 0; m < d; ++m)
                    s += dza[m] * weight2(&v, m, n);
                dh[n] = s;
            }
            for (int n = 0; n < f; ++n) {
                dga[n] = dh[n] * u[n] * silu_grad(g[n]);
                dua[n] = dh[n] * silu(g[n]);
            }
            for (int c = 0; c < d; ++c) {
                float s = 0.0f;
                for (int n = 0; n < f; ++n)
                    s += dga[n] * weight13(&v, n, c) + dua[n] * weight13(&v, f + n, c);
                dx[(size_t)t * d + c] += s;
            }
        }
        free(xt);
    }
    if (bad) {
        free(dz);
        return -2;
    }
    /* weight gradients: per expert, tokens in ascending order */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int e = 0; e < E; ++e) {
        if (dw2[e])
            memset(dw2[e], 0, sizeof(float) * (size_t)d * f);
        if (dw13[e])
            memset(dw13[e], 0, sizeof(float) * (size_t)2 * f * d);
        for (size_t a = 0; a < n_asg; ++a) {
            if (topk_ids[a] != e)
                continue;
            const size_t t = a / k;
            const float *h = hh + a * f, *dga = dg + a * f, *dua = du + a * f, *dza = dz + a * d;
            if (dw2[e])
                for (int m = 0; m < d; ++m)
                    for (int n = 0; n < f; ++n)
                        dw2[e][(size_t)m * f + n] += dza[m] * h[n];
            if (dw13[e])
                for (int n = 0; n < f; ++n)
                    for (int c = 0; c < d; ++c) {
                        const float xc = bf16_bits_to_f32(x[t * d + c]);
                        dw13[e][(size_t)n * d + c] += dga[n] * xc;
                        dw13[e][(size_t)(f + n) * d + c] += dua[n] * xc;
                    }
        }
    }
    free(dz);
    return 0;
}

/* Dynamic MXFP4 quantisation of a bf16 matrix [rows, cols] (cols % 32 == 0):
 * codes packed two per byte [rows, cols / 2] (even column in the low nibble),
 * E8M0 scales [rows, cols / 32]. */
int oracle_mx_quant_rows(const uint16_t *x, int rows, int cols, uint8_t *codes, uint8_t *scales)
{
    if (!x || !codes || !scales || rows < 0 || cols < 32 || cols % 32)
        return -1;
    float buf[32];
    uint8_t q[32];
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; c += 32) {
            for (int i = 0; i < 32; ++i)
                buf[i] = bf16_bits_to_f32(x[(size_t)r * cols + c + i]);
            scales[(size_t)r * (cols / 32) + c / 32] = oracle_mx_quant_group(buf, 32, q, NULL);
            for (int i = 0; i < 32; i += 2)
                codes[(size_t)r * (cols / 2) + (c + i) / 2] = (uint8_t)(q[i] | (q[i + 1] << 4));
        }
    return 0;
}

/* Dynamic activation quantisation of a bf16 matrix [rows, cols]: one scale
 * per row (group = cols) or per 1x128 block (group = 128). codes [rows, cols],
 * scales [rows, cols / group]. */
int oracle_quant_rows(const uint16_t *x, int rows, int cols, int group, uint8_t *codes, float *scales)
{
    if (!x || !codes || !scales || rows < 0 || cols < 1 || group < 1 || cols % group)
        return -1;
    float *buf = (float *)malloc(sizeof(float) * (size_t)cols);
    if (!buf)
        return -2;
    for (int r = 0; r < rows; ++r) {
        for (int c = 0; c < cols; ++c)
            buf[c] = bf16_bits_to_f32(x[(size_t)r * cols + c]);
        for (int c = 0; c < cols; c += group)
            scales[(size_t)r * (cols / group) + c / group] =
                oracle_quant_group(buf + c, group, codes + (size_t)r * cols + c, NULL);
    }
    free(buf);
    return 0;
}
