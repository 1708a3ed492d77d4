// api.cpp -- the C ABI of libmoe (declared in include/moe.h): argument
// validation, workspace carving, the block-size / stage / K-split choice and
// launch sequencing. No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "moe.h"
#include "launch.h"

#ifndef MOE_G1_CT
#define MOE_G1_CT 1
#endif
#ifndef MOE_G2_CT
#define MOE_G2_CT 4
#endif
// tiled-kernel tile shape: rows and weight rows (0: the library's choice)
// routing runs inside the sort's single workgroup while T * E is at most this
#ifndef MOE_FUSE_ROUTE_MAX
#define MOE_FUSE_ROUTE_MAX 512
#endif
#ifndef MOE_G1_BM
#define MOE_G1_BM 0
#endif
#ifndef MOE_G2_BM
#define MOE_G2_BM 0
#endif
#ifndef MOE_G1_TN
#define MOE_G1_TN 0
#endif
#ifndef MOE_G2_TN
#define MOE_G2_TN 0
#endif

namespace moe {
// implemented in gemm_stream.hip / gemm_tiled.hip / moe_1stage.hip
bool stream_gemm1_supported(const GemmShape &sh);
bool stream_gemm2_supported(const GemmShape &sh);
hipError_t launch_stream_gemm1(const Gemm1Args &g, int CT, hipStream_t s);
hipError_t launch_stream_gemm2(const Gemm2Args &g, int CT, int ksplit, hipStream_t s);
bool tiled_gemm_supported(const GemmShape &sh);
int tiled_tile_cols(int B, int quant, bool gemm1, int bm, int tn);
int tiled_tile_rows(int B, int quant, bool gemm1, int bm, int tn);
hipError_t launch_tiled_gemm1(const Gemm1Args &g, int bm, int tn, hipStream_t s);
hipError_t launch_tiled_gemm2(const Gemm2Args &g, int bm, int tn, int ksplit, hipStream_t s);
int tiled_gemm2_parts(int f, int quant, int ksplit);
}  // namespace moe

using namespace moe;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                          \
    do {                                             \
        hipError_t _e = (expr);                      \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

// Carves 256-byte aligned sub-buffers out of a workspace. With base == NULL
// it only measures, so size queries and launches share one layout.
struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    template <class T>
    T *take(size_t count) {
        size_t start = (off + 255) & ~size_t(255);
        off = start + count * sizeof(T);
        return base ? reinterpret_cast<T *>(base + start) : nullptr;
    }
    size_t bytes() const { return (off + 255) & ~size_t(255); }
};

int cu_count_cached() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cu <= 0)
            cu = 256;
        cached[dev] = cu;
    }
    return cached[dev];
}

bool valid_B(int B) { return B == 16 || B == 32 || B == 64 || B == 128 || B == 256; }

int check_shape(int T, int d, int f, int E, int k, int B, int quant) {
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
        return fail(MOE_ERR_INVALID_ARG, "bad shape T=%d E=%d k=%d (need T>=0, 1<=k<=E<=%d, k<=%d)",
                    T, E, k, MOE_MAX_EXPERTS, MOE_MAX_TOPK);
    if (d < 1 || f < 1) return fail(MOE_ERR_INVALID_ARG, "bad sizes d=%d f=%d", d, f);
    if (d % 128 || f % 128)
        return fail(MOE_ERR_UNSUPPORTED, "d=%d and f=%d must be multiples of 128", d, f);
    if (quant < 0 || quant > 3) return fail(MOE_ERR_INVALID_ARG, "bad quant %d", quant);
    if (quant == MOE_QUANT_MXFP4 && (d % 256 || f % 256))
        return fail(MOE_ERR_UNSUPPORTED, "MXFP4 needs d=%d and f=%d multiples of 256", d, f);
    if (!valid_B(B)) return fail(MOE_ERR_INVALID_ARG, "B=%d must be 16, 32, 64, 128 or 256", B);
    if ((int64_t)T * k > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "T*k=%lld above 2^24", (long long)T * k);
    if ((int64_t)T * d >= (int64_t(1) << 31) || ((int64_t)T * k + (int64_t)E * B) * f >= (int64_t(1) << 31))
        return fail(MOE_ERR_UNSUPPORTED, "activation buffers above 2^31 elements");
    if ((int64_t)2 * f * d * 2 >= (int64_t(1) << 32))
        return fail(MOE_ERR_UNSUPPORTED, "one expert's weights above 4 GiB");
    return MOE_OK;
}

int64_t max_padded(int T, int k, int E, int B) { return (int64_t)T * k + (int64_t)E * B - k; }
int64_t max_blocks(int T, int k, int E, int B) { return (max_padded(T, k, E, B) + B - 1) / B; }

// ----------------------------------------------------------- config choice
struct Config {
    int B, stage, ksplit;
};

bool use_tiled(int B) { return B >= 64; }

int auto_ksplit(int T, int d, int f, int E, int k, int B, int quant, int cu) {
    // the streaming kernel: about two workgroups per CU in the down projection
    // (measured best on the Mixtral decode shape: 4 splits of K = 14336)
    const int64_t rows = (int64_t)T * k;
    const int64_t blocks = std::min<int64_t>(max_blocks(T, k, E, B), std::min<int64_t>(E, rows) + rows / B);
    int64_t ntiles;
    if (use_tiled(B)) {
        ntiles = (int64_t)(d / tiled_tile_cols(B, quant, false, MOE_G2_BM, MOE_G2_TN)) *
                 (B / tiled_tile_rows(B, quant, false, MOE_G2_BM, MOE_G2_TN));
    } else {
        const int CT = (d % 256 == 0) ? 4 : 2;
        ntiles = d / (64 * CT);
    }
    const int64_t base = std::max<int64_t>(1, ntiles * blocks);
    const int KS = quant == 0 ? 64 : (quant == MOE_QUANT_MXFP4 ? 256 : 128);   // K per 128-byte step
    // the tiled kernel holds one workgroup per CU: split when there are fewer
    // tiles than CUs; bf16 (MFMA-bound) also splits in two under four rounds
    // of tiles, which halves the idle tail of the last round (Mixtral
    // prefill, 560 tiles of 256 x 256: 1110 -> 1015 us). e4m3 at one full
    // round of tiles got slower (121 -> 130 us), and so did MXFP4 at the
    // Mixtral prefill shape (362 -> 384 us).
    if (use_tiled(B) && base >= cu)
        return (quant == 0 && base < 4 * (int64_t)cu && f / KS >= 8) ? 2 : 1;
    const int64_t target = use_tiled(B) ? cu : 2 * (int64_t)cu;
    int ks = (int)std::min<int64_t>((target + base - 1) / base, f / KS / 4);
    return std::max(1, ks);
}

// Block size (measured on MI355X at the Mixtral shape with the sweep that
// writes the tuned-config table; the table overrides this rule where it has
// rows). 64/128/256-row blocks go to the LDS-tiled kernels.
// - bf16 takes 256-row blocks from 512 rows per expert on: their 256 x 256
//   tiles need a third fewer operand bytes per MFMA than 128 x 256 (Mixtral
//   prefill: GEMM1 -8 %; GEMM2 -9 % with the two-part split of K). From
//   about 12 rows per expert a 64-row tiled block beats the streaming kernel
//   (T = 128: 530 against 816 us), which re-reads an expert's weights for
//   each of its blocks once random routing gives it more than 32 rows.
// - e4m3 per-token takes the tiled kernel at every size where it runs: at a
//   few rows per expert its 64 x 256 tiles stream the weights as full
//   128-byte lines and beat the streaming kernel by about a quarter
//   (T = 32: 275 against 376 us); 256-row blocks from about 100 rows per
//   expert read each expert's weights once.
// - MXFP4 goes to the tiled kernels like bf16 from about 24 rows per expert
//   when d and f are multiples of 512 (its K pairs), else it stays on the
//   streaming kernel; e4m3 1x128 runs on the streaming kernel only.
int choose_B(int T, int d, int f, int E, int k, int quant) {
    const double rows = (double)T * k / E;
    // shapes the tiled kernels take (d a multiple of 256; MXFP4 whole K pairs)
    const bool bf16_tiled = quant == 0 && d % 256 == 0;
    const bool mx_tiled = quant == MOE_QUANT_MXFP4 && d % 512 == 0 && f % 512 == 0;
    const bool fp8_tiled = quant == 1 && d % 256 == 0;
    if ((bf16_tiled || mx_tiled) && rows >= 512) return 256;
    if (fp8_tiled && rows >= 96) return 256;
    if ((bf16_tiled || mx_tiled) && rows >= 96) return 128;
    if (fp8_tiled) return 64;
    if (bf16_tiled && rows >= 12) return 64;
    if (mx_tiled && rows >= 24) return 64;
    if (rows <= 4) return 16;
    return 32;
}

// ------------------------------------------------------ tuned-config table
// Rows measured offline (cu, T, d, f, E, k, quant) -> (B, stage, ksplit), in
// the spirit of the tuned-configuration CSV of the AITER walk-through
// (section 4.1), whose lookup matches the token count fuzzily (padded M).
// Here: among rows with the call's (cu, d, f, E, k, quant), the one with the
// smallest T at or above the call's T, else the one with the largest T.
struct TableRow {
    int cu, T, d, f, E, k, quant, B, stage, ksplit;
};
std::mutex g_table_mu;
std::vector<TableRow> g_table;

bool table_lookup(int T, int d, int f, int E, int k, int quant, int cu, Config *out) {
    std::lock_guard<std::mutex> lock(g_table_mu);
    const TableRow *best = nullptr;
    for (const TableRow &r : g_table) {
        if (r.cu != cu || r.d != d || r.f != f || r.E != E || r.k != k || r.quant != quant) continue;
        if (!best) {
            best = &r;
            continue;
        }
        const bool r_up = r.T >= T, b_up = best->T >= T;
        if ((r_up && (!b_up || r.T < best->T)) || (!r_up && !b_up && r.T > best->T)) best = &r;
    }
    if (!best) return false;
    out->B = best->B;
    out->stage = best->stage;
    out->ksplit = best->ksplit;
    return true;
}

Config choose(int T, int d, int f, int E, int k, int quant, int cu) {
    Config c;
    if (table_lookup(T, d, f, E, k, quant, cu, &c)) return c;
    c.B = choose_B(T, d, f, E, k, quant);
    c.stage = 2;
    c.ksplit = auto_ksplit(T, d, f, E, k, c.B, quant, cu);
    return c;
}

// K-split when the caller leaves it to the library: the table's, if its row
// has the block size in use, else the rule above
int pick_ksplit(int T, int d, int f, int E, int k, int B, int quant, int cu) {
    Config c;
    if (table_lookup(T, d, f, E, k, quant, cu, &c) && c.B == B) return c.ksplit;
    return auto_ksplit(T, d, f, E, k, B, quant, cu);
}

// -------------------------------------------------------------- stage 1/2
// Split of GEMM1's reduction (K = d) for few assignments (the AITER
// walk-through, section 3.4, splits K when token * topk <= expert and the
// tiles do not fill the CUs). bf16 on the streaming kernel: with
// T * k <= E at most T * k sort blocks hold rows, which is too few
// workgroups to keep enough weight bytes in flight; the parts' raw gate / up
// sums are added in a fixed order by a second kernel that applies SwiGLU.
// Aimed at about MOE_G1_WG_PER_CU workgroups per CU, at most 8 parts.
#ifndef MOE_G1_WG_PER_CU
#define MOE_G1_WG_PER_CU 8
#endif
int gemm1_ksplit(int T, int d, int f, int E, int k, int B, int quant, int cu) {
    if (quant != 0 || use_tiled(B) || (int64_t)T * k > E) return 1;
    const int64_t blocks = std::min<int64_t>(max_blocks(T, k, E, B), (int64_t)T * k);
    const int64_t wgs = std::max<int64_t>(1, (int64_t)(f / (64 * MOE_G1_CT)) * blocks);
    const int64_t want = ((int64_t)MOE_G1_WG_PER_CU * cu + wgs - 1) / wgs;
    const int ks = (int)std::max<int64_t>(1, std::min<int64_t>(8, want));
    return ks > 1 ? stream_gemm1_parts(d, ks) : 1;
}

struct Gemm1Ws {
    uint8_t *qx = nullptr;
    float *sx = nullptr;
    uint8_t *sxm = nullptr;   // MXFP4: E8M0 scales of x [T, d/32]
    uint16_t *hb = nullptr;
    float *amax = nullptr;
    int ksplit = 1;           // GEMM1 parts (bf16 streaming kernel, few assignments)
    float *gu_part = nullptr; // their raw sums [ksplit][T*k, 2f]
};

Gemm1Ws carve_gemm1(Carver &c, int T, int d, int f, int E, int k, int B, int quant) {
    Gemm1Ws w;
    const size_t P = (size_t)max_padded(T, k, E, B);
    w.ksplit = gemm1_ksplit(T, d, f, E, k, B, quant, cu_count_cached());
    if (w.ksplit > 1) w.gu_part = c.take<float>((size_t)w.ksplit * T * k * 2 * f);
    if (quant == MOE_QUANT_MXFP4) {
        w.qx = c.take<uint8_t>((size_t)T * d / 2);
        w.sxm = c.take<uint8_t>((size_t)T * (d / 32));
    } else if (quant != 0) {
        w.qx = c.take<uint8_t>((size_t)T * d);
        w.sx = c.take<float>(quant == 1 ? (size_t)T : (size_t)T * (d / 128));
    }
    if (quant == 1) {
        w.hb = c.take<uint16_t>(P * f);
        w.amax = c.take<float>(P);
    }
    return w;
}

// x_ready: the activation codes are already in w (quantised by the routing
// launch, which also cleared the per-token row amax of h), so no
// quantisation launch here.
int run_gemm1(int T, int d, int f, int E, int k, int B, int quant, const void *x, const void *w13,
              const void *w13_scale_v, const int32_t *sorted_ids, const int32_t *seid,
              const int32_t *num_valid, void *h, void *h_scale_v, const Gemm1Ws &w, hipStream_t s,
              float *zero = nullptr, size_t zero_n = 0, bool x_ready = false) {
    // fp32 scales (e4m3) or E8M0 bytes (MXFP4)
    const float *w13_scale = quant == MOE_QUANT_MXFP4 ? nullptr : static_cast<const float *>(w13_scale_v);
    float *h_scale = quant == MOE_QUANT_MXFP4 ? nullptr : static_cast<float *>(h_scale_v);
    Gemm1Args g{};
    g.zero = zero;
    g.zero_n = zero_n;
    g.sh = GemmShape{T, d, f, E, k, B, quant};
    g.w13 = w13;
    g.w13_scale = w13_scale;
    g.sorted_ids = sorted_ids;
    g.sorted_expert_ids = seid;
    g.num_valid = num_valid;
    const size_t P = (size_t)max_padded(T, k, E, B);
    if (quant == 0) {
        g.a = x;
        g.h = h;
    } else if (quant == MOE_QUANT_MXFP4) {
        if (!x_ready)
            HIP_TRY(launch_quant_mx(static_cast<const uint16_t *>(x), T, d, w.qx, w.sxm, s),
                    "activation quantisation launch");
        g.a = w.qx;
        g.a_mx = w.sxm;
        g.w13_mx = static_cast<const uint8_t *>(w13_scale_v);
        g.h = h;
        g.h_mx = static_cast<uint8_t *>(h_scale_v);
    } else {
        // (per-token e4m3: the same launch clears the row amax of h, which
        // GEMM1 takes with atomics)
        if (!x_ready)
            HIP_TRY(launch_quant_act(static_cast<const uint16_t *>(x), T, d, quant == 1 ? d : 128, w.qx,
                                     w.sx, s, quant == 1 ? w.amax : nullptr, quant == 1 ? (int)P : 0),
                    "activation quantisation launch");
        g.a = w.qx;
        g.a_scale = w.sx;
        if (quant == 1) {
            g.h = w.hb;
            g.h_scale = w.amax;
        } else {
            g.h = h;
            g.h_scale = h_scale;
        }
    }
    if (use_tiled(B)) {
        if (!tiled_gemm_supported(g.sh))
            return fail(MOE_ERR_UNSUPPORTED, "no tiled GEMM1 kernel for B=%d quant=%d d=%d", B, quant, d);
        HIP_TRY(launch_tiled_gemm1(g, MOE_G1_BM, MOE_G1_TN, s), "GEMM1 launch");
    } else {
        if (!stream_gemm1_supported(g.sh))
            return fail(MOE_ERR_UNSUPPORTED, "no GEMM1 kernel for B=%d", B);
        if (w.ksplit > 1) {
            g.ksplit = w.ksplit;
            g.gu_part = w.gu_part;
        }
        HIP_TRY(launch_stream_gemm1(g, MOE_G1_CT, s), "GEMM1 launch");
        if (w.ksplit > 1)
            HIP_TRY(launch_swiglu_parts(w.gu_part, w.ksplit, T * k, f, sorted_ids, num_valid, (int)P,
                                        static_cast<uint16_t *>(h), s),
                    "SwiGLU launch");
    }
    if (quant == 1)
        HIP_TRY(launch_quant_h_rows(w.hb, w.amax, (int)P, f, num_valid, sorted_ids, T * k,
                                    static_cast<uint8_t *>(h), h_scale, s),
                "h quantisation launch");
    return MOE_OK;
}

// K parts of the tiled down projection whose weighted rows are stored
constexpr int STORED_SPLITS = 2;

// GEMM2's fp32 buffer: the token accumulator [T, d], or, for the tiled
// kernel, the weighted rows by K part and assignment [STORED_SPLITS][T*k, d]
// (the larger of the two, so that one layout serves both), then, for the
// tiled kernel, the marks of the assignments the sort placed [T*k].
struct Gemm2Ws {
    float *acc = nullptr;
    int32_t *written = nullptr;
};

Gemm2Ws carve_gemm2(Carver &c, int T, int d, int k, int B) {
    Gemm2Ws w;
    w.acc = c.take<float>((size_t)T * d * (use_tiled(B) ? (size_t)k * STORED_SPLITS : 1));
    if (use_tiled(B)) w.written = c.take<int32_t>((size_t)T * k);
    return w;
}

// The tiled down projection split into at most STORED_SPLITS parts of K
// stores each part's weighted rows, and a combine kernel sums each token's
// k x parts rows: no atomics, no accumulator clearing, and a fixed
// summation order.
bool stored_rows(int B, int ksplit) { return use_tiled(B) && ksplit <= STORED_SPLITS; }

// ids_valid: every assignment is in sorted_ids (routing ran inside the
// library); otherwise the stored-row combine first marks the assignments the
// sort placed, so that dropped ones (ids outside [0, E)) add nothing.
int run_gemm2(int T, int d, int f, int E, int k, int B, int quant, int ksplit, const void *h,
              const void *h_scale_v, const void *w2, const void *w2_scale_v,
              const int32_t *sorted_ids, const float *sorted_w, const int32_t *seid,
              const int32_t *num_valid, void *out, const Gemm2Ws &ws2, bool ids_valid, hipStream_t s,
              bool acc_zeroed = false) {
    float *acc = ws2.acc;
    Gemm2Args g{};
    g.sh = GemmShape{T, d, f, E, k, B, quant};
    g.h = h;
    g.w2 = w2;
    if (quant == MOE_QUANT_MXFP4) {
        g.h_mx = static_cast<const uint8_t *>(h_scale_v);
        g.w2_mx = static_cast<const uint8_t *>(w2_scale_v);
    } else {
        g.h_scale = static_cast<const float *>(h_scale_v);
        g.w2_scale = static_cast<const float *>(w2_scale_v);
    }
    g.sorted_ids = sorted_ids;
    g.sorted_w = sorted_w;
    g.sorted_expert_ids = seid;
    g.num_valid = num_valid;
    g.acc = acc;
    if (ksplit <= 0) ksplit = pick_ksplit(T, d, f, E, k, B, quant, cu_count_cached());
    g.ksplit = ksplit;
    const bool tiled = use_tiled(B);
    if (tiled ? !tiled_gemm_supported(g.sh) : !stream_gemm2_supported(g.sh))
        return fail(MOE_ERR_UNSUPPORTED, "no GEMM2 kernel for B=%d quant=%d d=%d", B, quant, d);
    if (stored_rows(B, ksplit)) {
        g.acc = nullptr;
        g.yrows = acc;
        if (!ids_valid)
            HIP_TRY(launch_mark_written(sorted_ids, num_valid, (int)max_padded(T, k, E, B), T * k,
                                        ws2.written, s),
                    "mark launch");
        HIP_TRY(launch_tiled_gemm2(g, MOE_G2_BM, MOE_G2_TN, ksplit, s), "GEMM2 launch");
        HIP_TRY(launch_combine_rows(acc, T, k, tiled_gemm2_parts(f, quant, ksplit), d,
                                    ids_valid ? nullptr : ws2.written, static_cast<uint16_t *>(out), s),
                "combine launch");
        return MOE_OK;
    }
    if (!acc_zeroed) HIP_TRY(launch_fill_f32(acc, (size_t)T * d, 0.0f, s), "fill launch");
    if (tiled)
        HIP_TRY(launch_tiled_gemm2(g, MOE_G2_BM, MOE_G2_TN, ksplit, s), "GEMM2 launch");
    else
        HIP_TRY(launch_stream_gemm2(g, MOE_G2_CT, ksplit, s), "GEMM2 launch");
    HIP_TRY(launch_finalize(acc, static_cast<uint16_t *>(out), (size_t)T * d, s), "finalize launch");
    return MOE_OK;
}

struct FusedWs {
    int32_t *topk_ids = nullptr;
    float *topk_w = nullptr;
    int32_t *sorted_ids = nullptr, *seid = nullptr, *counts = nullptr, *offsets = nullptr,
            *num_valid = nullptr;
    float *sorted_w = nullptr;
    void *h = nullptr;
    void *h_scale = nullptr;   // fp32 (e4m3) or E8M0 bytes (MXFP4)
    Gemm1Ws g1;
    Gemm2Ws g2;
};

FusedWs carve_fused(Carver &c, int T, int d, int f, int E, int k, int quant, int B, bool route) {
    FusedWs w;
    const size_t P = (size_t)max_padded(T, k, E, B), NB = (size_t)max_blocks(T, k, E, B);
    if (route) {
        w.topk_ids = c.take<int32_t>((size_t)T * k);
        w.topk_w = c.take<float>((size_t)T * k);
    }
    w.sorted_ids = c.take<int32_t>(P);
    w.sorted_w = c.take<float>(P);
    w.seid = c.take<int32_t>(NB);
    w.counts = c.take<int32_t>(E);
    w.offsets = c.take<int32_t>(E + 1);
    w.num_valid = c.take<int32_t>(1);
    w.h = c.take<uint8_t>(quant == MOE_QUANT_MXFP4 ? P * f / 2 : P * f * (quant == 0 ? 2 : 1));
    if (quant == 1) w.h_scale = c.take<float>(P);
    if (quant == 2) w.h_scale = c.take<float>(P * (f / 128));
    if (quant == MOE_QUANT_MXFP4) w.h_scale = c.take<uint8_t>(P * (f / 32));
    w.g1 = carve_gemm1(c, T, d, f, E, k, B, quant);
    w.g2 = carve_gemm2(c, T, d, k, B);
    return w;
}

}  // namespace

// ====================================================================== ABI
extern "C" {

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *moe_last_error(void) { return g_err; }

int64_t moe_sort_max_padded(int T, int k, int E, int B) {
    if (T < 0 || k < 1 || k > E || B < 1) return -1;
    return max_padded(T, k, E, B);
}

int64_t moe_sort_max_blocks(int T, int k, int E, int B) {
    if (T < 0 || k < 1 || k > E || B < 1) return -1;
    return max_blocks(T, k, E, B);
}

int moe_topk(const float *logits, int T, int E, int k, int score, int renorm, int32_t *topk_ids,
             float *topk_w, void *stream) {
    g_err[0] = 0;
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
        return fail(MOE_ERR_INVALID_ARG, "bad routing shape T=%d E=%d k=%d", T, E, k);
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARG, "bad score %d", score);
    if (T > 0 && (!logits || !topk_ids || !topk_w)) return fail(MOE_ERR_INVALID_ARG, "null pointer");
    HIP_TRY(launch_topk(logits, T, E, k, score, renorm, topk_ids, topk_w, (hipStream_t)stream),
            "topk launch");
    return MOE_OK;
}

int moe_sort(const int32_t *topk_ids, const float *topk_w, int T, int k, int E, int B,
             int32_t *sorted_ids, float *sorted_w, int32_t *sorted_expert_ids,
             int32_t *expert_counts, int32_t *expert_offsets, int32_t *num_valid, void *stream) {
    g_err[0] = 0;
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || B < 1 || B > 1024)
        return fail(MOE_ERR_INVALID_ARG, "bad sort shape T=%d k=%d E=%d B=%d", T, k, E, B);
    if ((int64_t)T * k > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "T*k above 2^24");
    if ((T > 0 && (!topk_ids || !topk_w)) || !sorted_ids || !sorted_w || !sorted_expert_ids ||
        !expert_counts || !expert_offsets || !num_valid)
        return fail(MOE_ERR_INVALID_ARG, "null pointer");
    HIP_TRY(launch_sort(topk_ids, topk_w, T, k, E, B, sorted_ids, sorted_w, sorted_expert_ids,
                        expert_counts, expert_offsets, num_valid, (hipStream_t)stream),
            "sort launch");
    return MOE_OK;
}

int moe_quant_act_mx(const void *x, int rows, int cols, uint8_t *codes, uint8_t *scales,
                     void *stream) {
    g_err[0] = 0;
    if (rows < 0 || cols < 32 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "bad MXFP4 shape rows=%d cols=%d", rows, cols);
    if (rows > 0 && (!x || !codes || !scales)) return fail(MOE_ERR_INVALID_ARG, "null pointer");
    HIP_TRY(launch_quant_mx(static_cast<const uint16_t *>(x), rows, cols, codes, scales,
                            (hipStream_t)stream),
            "quant launch");
    return MOE_OK;
}

int moe_quant_act(const void *x, int rows, int cols, int group, uint8_t *codes, float *scales,
                  void *stream) {
    g_err[0] = 0;
    if (rows < 0 || cols < 1 || group < 1) return fail(MOE_ERR_INVALID_ARG, "bad quant shape");
    if (cols % 128 || !(group == cols || group == 128))
        return fail(MOE_ERR_UNSUPPORTED, "cols=%d group=%d: need cols %% 128 == 0 and group in {128, cols}",
                    cols, group);
    if (rows > 0 && (!x || !codes || !scales)) return fail(MOE_ERR_INVALID_ARG, "null pointer");
    HIP_TRY(launch_quant_act(static_cast<const uint16_t *>(x), rows, cols, group, codes, scales,
                             (hipStream_t)stream),
            "quant launch");
    return MOE_OK;
}

size_t moe_gemm1_workspace_bytes(int T, int d, int f, int E, int k, int B, int quant) {
    if (check_shape(T, d, f, E, k, B, quant) != MOE_OK) return 0;
    Carver c(nullptr);
    carve_gemm1(c, T, d, f, E, k, B, quant);
    return c.bytes();
}

int moe_gemm1_swiglu(int T, int d, int f, int E, int k, int B, int quant, const void *x,
                     const void *w13, const void *w13_scale, const int32_t *sorted_ids,
                     const int32_t *sorted_expert_ids, const int32_t *num_valid, void *h,
                     void *h_scale, void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    int rc = check_shape(T, d, f, E, k, B, quant);
    if (rc) return rc;
    if (!w13 || !sorted_ids || !sorted_expert_ids || !num_valid || !h || (T > 0 && !x))
        return fail(MOE_ERR_INVALID_ARG, "null pointer");
    if (quant != 0 && (!w13_scale || !h_scale))
        return fail(MOE_ERR_INVALID_ARG, "fp8 and MXFP4 need w13_scale and h_scale");
    Carver c(nullptr);
    carve_gemm1(c, T, d, f, E, k, B, quant);
    if (ws_bytes < c.bytes() || (c.bytes() > 0 && !ws))
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, c.bytes());
    if (T == 0) return MOE_OK;
    Carver cw(ws);
    Gemm1Ws w = carve_gemm1(cw, T, d, f, E, k, B, quant);
    return run_gemm1(T, d, f, E, k, B, quant, x, w13, w13_scale, sorted_ids, sorted_expert_ids,
                     num_valid, h, h_scale, w, (hipStream_t)stream);
}

size_t moe_gemm2_workspace_bytes(int T, int d, int f, int E, int k, int B, int quant) {
    if (check_shape(T, d, f, E, k, B, quant) != MOE_OK) return 0;
    Carver c(nullptr);
    carve_gemm2(c, T, d, k, B);
    return c.bytes();
}

int moe_gemm2_combine(int T, int d, int f, int E, int k, int B, int quant, int ksplit,
                      const void *h, const void *h_scale, const void *w2, const void *w2_scale,
                      const int32_t *sorted_ids, const float *sorted_w,
                      const int32_t *sorted_expert_ids, const int32_t *num_valid, void *out,
                      void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    int rc = check_shape(T, d, f, E, k, B, quant);
    if (rc) return rc;
    if (!h || !w2 || !sorted_ids || !sorted_w || !sorted_expert_ids || !num_valid ||
        (T > 0 && !out))
        return fail(MOE_ERR_INVALID_ARG, "null pointer");
    if (quant != 0 && (!w2_scale || !h_scale))
        return fail(MOE_ERR_INVALID_ARG, "fp8 and MXFP4 need w2_scale and h_scale");
    Carver c(nullptr);
    carve_gemm2(c, T, d, k, B);
    if (ws_bytes < c.bytes() || (c.bytes() > 0 && !ws))
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, c.bytes());
    if (T == 0) return MOE_OK;
    Carver cw(ws);
    const Gemm2Ws w2s = carve_gemm2(cw, T, d, k, B);
    return run_gemm2(T, d, f, E, k, B, quant, ksplit, h, h_scale, w2, w2_scale, sorted_ids,
                     sorted_w, sorted_expert_ids, num_valid, out, w2s, false, (hipStream_t)stream);
}

// ------------------------------------------------------------- backward
namespace {
struct BwdWs {
    int32_t *sorted_ids = nullptr, *seid = nullptr, *counts = nullptr, *offsets = nullptr,
            *num_valid = nullptr;
    float *sorted_w = nullptr, *gu = nullptr, *acc = nullptr;
    uint16_t *w13t = nullptr, *w2t = nullptr, *h = nullptr, *dgu = nullptr;
    uint16_t *dgu_lo = nullptr;   // low bf16 parts of dg / du [P, 2f]
    uint16_t *xs = nullptr;       // x in slot order [P, d]
    uint16_t *dz_hi = nullptr, *dz_lo = nullptr;   // w dy in slot order, two bf16 parts [P, d]
    float *v = nullptr;           // tiled path: Wd^T dy per slot [P, f]
};

BwdWs carve_backward(Carver &c, int T, int d, int f, int E, int k, int B) {
    BwdWs w;
    const size_t P = (size_t)max_padded(T, k, E, B), NB = (size_t)max_blocks(T, k, E, B);
    w.sorted_ids = c.take<int32_t>(P);
    w.sorted_w = c.take<float>(P);
    w.seid = c.take<int32_t>(NB);
    w.counts = c.take<int32_t>(E);
    w.offsets = c.take<int32_t>((size_t)E + 1);
    w.num_valid = c.take<int32_t>(1);
    if (B < 64) {   // the streaming kernels read transposed copies of the weights
        w.w13t = c.take<uint16_t>((size_t)E * 2 * f * d);
        w.w2t = c.take<uint16_t>((size_t)E * f * d);
    }
    w.gu = c.take<float>(P * 2 * f);
    w.h = c.take<uint16_t>(P * f);
    w.dgu = c.take<uint16_t>(P * 2 * f);
    w.dgu_lo = c.take<uint16_t>(P * 2 * f);
    w.acc = c.take<float>((size_t)T * d);
    w.xs = c.take<uint16_t>(P * d);
    w.dz_hi = c.take<uint16_t>(P * d);
    w.dz_lo = c.take<uint16_t>(P * d);
    if (B >= 64) w.v = c.take<float>(P * f);
    return w;
}

// The backward's GEMMs on the tiled kernels (sort blocks of 64, 128 or 256
// rows): the forward sums, v = Wd^T dy with Wd^T [E, f, d] taken as two
// halves of f/2 rows, and dx with K = 2f.
bool backward_tiled_ok(int T, int d, int f, int E, int k, int B) {
    return f % 256 == 0 && tiled_gemm_supported(GemmShape{T, d, f, E, k, B, 0}) &&
           tiled_gemm_supported(GemmShape{T, d, f / 2, E, k, B, 0}) &&
           tiled_gemm_supported(GemmShape{T, d, 2 * f, E, k, B, 0});
}

// The tiled path wherever it runs (d, f multiples of 256) from 2 rows per
// expert on: measured faster than the streaming path on Mixtral-shaped
// layers from T = 16 (4 rows per expert) to 4096, blocks of 64 rows below
// 48 rows per expert, 128 below 192 and 256 above. Otherwise the streaming
// kernels, with 16-row blocks up to 4 rows per expert and 32 above.
int backward_B(int T, int d, int f, int E, int k) {
    const double rows = (double)T * k / E;
    if (rows >= 2) {
        const int B = rows >= 192 ? 256 : (rows >= 48 ? 128 : 64);
        if (backward_tiled_ok(T, d, f, E, k, B)) return B;
    }
    return rows <= 4 ? 16 : 32;
}

int check_backward(int T, int d, int f, int E, int k, int B) {
    int rc = check_shape(T, d, f, E, k, B == 0 ? 32 : B, 0);
    if (rc) return rc;
    if (B != 0 && B != 16 && B != 32 && B != 64 && B != 128 && B != 256)
        return fail(MOE_ERR_UNSUPPORTED, "the backward runs sort blocks of 16, 32, 64, 128 or 256 rows (got B=%d)", B);
    if (B >= 64 && !backward_tiled_ok(T, d, f, E, k, B))
        return fail(MOE_ERR_UNSUPPORTED, "the backward's tiled GEMMs need d %% 256 == 0 and f %% 256 == 0 (B=%d)", B);
    if ((int64_t)E * 2 * f * d >= (int64_t(1) << 31))
        return fail(MOE_ERR_UNSUPPORTED, "the backward's weight copies need E*2f*d below 2^31");
    return MOE_OK;
}
}  // namespace

size_t moe_backward_workspace_bytes(int T, int d, int f, int E, int k, int B) {
    if (check_backward(T, d, f, E, k, B) != MOE_OK) return 0;
    if (B == 0) B = backward_B(T, d, f, E, k);
    Carver c(nullptr);
    carve_backward(c, T, d, f, E, k, B);
    return c.bytes();
}

int moe_backward(int T, int d, int f, int E, int k, int B, const void *x, const int32_t *topk_ids,
                 const float *topk_w, const void *w13, const void *w2, const void *dy, void *dx,
                 float *dw13, float *dw2, float *dtopk_w, void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    int rc = check_backward(T, d, f, E, k, B);
    if (rc) return rc;
    if (B == 0) B = backward_B(T, d, f, E, k);
    if (!w13 || !w2 || !dw13 || !dw2 || (T > 0 && (!x || !topk_ids || !topk_w || !dy || !dx || !dtopk_w)))
        return fail(MOE_ERR_INVALID_ARG, "null pointer");
    Carver c(nullptr);
    carve_backward(c, T, d, f, E, k, B);
    if (ws_bytes < c.bytes() || !ws)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, c.bytes());
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {   // no assignment: zero weight gradients
        HIP_TRY(launch_fill_f32(dw13, (size_t)E * 2 * f * d, 0.0f, s), "fill launch");
        HIP_TRY(launch_fill_f32(dw2, (size_t)E * d * f, 0.0f, s), "fill launch");
        return MOE_OK;
    }
    Carver cw(ws);
    BwdWs w = carve_backward(cw, T, d, f, E, k, B);
    const GemmShape sh{T, d, f, E, k, B, 0};
    HIP_TRY(launch_sort(topk_ids, topk_w, T, k, E, B, w.sorted_ids, w.sorted_w, w.seid, w.counts,
                        w.offsets, w.num_valid, s),
            "sort launch");
    if (B < 64) {
        HIP_TRY(launch_transpose_bf16(static_cast<const uint16_t *>(w13), E, 2 * f, d, w.w13t, s),
                "transpose launch");
        HIP_TRY(launch_transpose_bf16(static_cast<const uint16_t *>(w2), E, d, f, w.w2t, s),
                "transpose launch");
    }
    HIP_TRY(launch_fill_f32(dtopk_w, (size_t)T * k, 0.0f, s), "fill launch");
    HIP_TRY(launch_fill_f32(w.acc, (size_t)T * d, 0.0f, s), "fill launch");
    // forward GEMM1 again, keeping the gate / up sums
    Gemm1Args g{};
    g.sh = sh;
    g.a = x;
    g.w13 = w13;
    g.sorted_ids = w.sorted_ids;
    g.sorted_expert_ids = w.seid;
    g.num_valid = w.num_valid;
    g.h = w.h;
    g.gu_out = w.gu;
    // dx = Wg^T dg + Wu^T du summed over each token's assignments (unit weights)
    Gemm2Args g2{};
    g2.sh = GemmShape{T, d, 2 * f, E, k, B, 0};
    g2.h = w.dgu;
    g2.w2 = w.w13t;   // the tiled path reads w13 in place (below)
    g2.sorted_ids = w.sorted_ids;
    g2.sorted_w = nullptr;
    g2.sorted_expert_ids = w.seid;
    g2.num_valid = w.num_valid;
    g2.acc = w.acc;
    if (B >= 64) {
        HIP_TRY(launch_tiled_gemm1(g, 0, 0, s), "GEMM1 launch");
        // v = Wd^T dy per slot: Wd [E, d, f] read in place as [K][N] weights of f/2 gate
        // and f/2 up columns
        Gemm1Args gv{};
        gv.sh = GemmShape{T, d, f / 2, E, k, B, 0};
        gv.a = dy;
        gv.w13 = w2;
        gv.w_kn = true;
        gv.sorted_ids = w.sorted_ids;
        gv.sorted_expert_ids = w.seid;
        gv.num_valid = w.num_valid;
        gv.gu_out = w.v;
        HIP_TRY(launch_tiled_gemm1(gv, 0, 0, s), "backward GEMM launch");
        HIP_TRY(launch_bwd_swiglu(w.gu, w.v, w.sorted_ids, w.sorted_w, (int)max_padded(T, k, E, B), T, k, f,
                                  w.h, w.dgu, w.dgu_lo, dtopk_w, s),
                "backward SwiGLU launch");
        // K = 2f split so that there are about four tiles per CU (fp32 atomics into acc)
        const int64_t tiles = max_blocks(T, k, E, B) * (int64_t)(d / tiled_tile_cols(B, 0, false, 0, 0));
        const int cu = cu_count_cached();
        const int ks = (int)std::min<int64_t>(4, std::max<int64_t>(1, (4 * (int64_t)cu + tiles - 1) / tiles));
        g2.w2 = w13;   // W13 [E, 2f, d] read in place as [K][N] weights
        g2.w_kn = true;
        HIP_TRY(launch_tiled_gemm2(g2, 0, 0, ks, s), "backward GEMM launch");
    } else {
        HIP_TRY(launch_stream_gemm1(g, MOE_G1_CT, s), "GEMM1 launch");
        // dg, du and the routing-weight gradients from v = Wd^T dy
        HIP_TRY(launch_stream_bwd_dh(sh, static_cast<const uint16_t *>(dy), w.w2t, w.sorted_ids,
                                     w.sorted_w, w.seid, w.gu, w.h, w.dgu, w.dgu_lo, dtopk_w, s),
                "backward GEMM launch");
        const int ks = auto_ksplit(T, d, 2 * f, E, k, B, 0, cu_count_cached());
        HIP_TRY(launch_stream_gemm2(g2, MOE_G2_CT, ks, s), "backward GEMM launch");
    }
    HIP_TRY(launch_finalize(w.acc, static_cast<uint16_t *>(dx), (size_t)T * d, s), "finalize launch");
    // weight gradients: dWd = sum dz h^T (dz = w dy), dW13 = sum [dg du] x^T, with x and dz
    // gathered into slot order first
    const int P = max_padded(T, k, E, B);
    HIP_TRY(launch_gather_bwd(w.sorted_ids, w.sorted_w, P, T, k, d, static_cast<const uint16_t *>(x),
                              static_cast<const uint16_t *>(dy), w.xs, w.dz_hi, w.dz_lo, s),
            "gather launch");
    const bool short_seg = (int64_t)T * k <= 256;
    if (B >= 64 && !short_seg && d % 256 == 0 && f % 256 == 0) {
        HIP_TRY(launch_wgrad_dma(w.dz_hi, w.dz_lo, w.h, d, f, E, w.offsets, dw2, s),
                "weight-gradient launch");
        HIP_TRY(launch_wgrad_dma(w.dgu, w.dgu_lo, w.xs, 2 * f, d, E, w.offsets, dw13, s),
                "weight-gradient launch");
    } else {
        HIP_TRY(launch_wgrad(w.dz_hi, w.dz_lo, w.h, d, f, E, w.offsets, w.counts, short_seg, dw2, s),
                "weight-gradient launch");
        HIP_TRY(launch_wgrad(w.dgu, w.dgu_lo, w.xs, 2 * f, d, E, w.offsets, w.counts, short_seg, dw13, s),
                "weight-gradient launch");
    }
    return MOE_OK;
}

int moe_load_config_table(const char *path, int *rows) {
    g_err[0] = 0;
    if (rows) *rows = 0;
    if (!path) {
        std::lock_guard<std::mutex> lock(g_table_mu);
        g_table.clear();
        return MOE_OK;
    }
    FILE *fp = fopen(path, "r");
    if (!fp) return fail(MOE_ERR_INVALID_ARG, "cannot open %s", path);
    std::vector<TableRow> table;
    char line[512];
    int lineno = 0, rc = MOE_OK;
    while (fgets(line, sizeof line, fp)) {
        ++lineno;
        char *p = line;
        while (*p == ' ' || *p == '\t') ++p;
        if (*p == '#' || *p == '\n' || *p == '\r' || *p == 0) continue;
        if (*p < '0' || *p > '9') {
            if (table.empty()) continue;   // a header line
            rc = fail(MOE_ERR_INVALID_ARG, "%s:%d: not a row", path, lineno);
            break;
        }
        // cu,T,d,f,E,k,quant,B,stage,ksplit[,anything]
        char qname[32] = {0};
        TableRow r{};
        int n = sscanf(p, "%d,%d,%d,%d,%d,%d,%31[^,],%d,%d,%d", &r.cu, &r.T, &r.d, &r.f, &r.E, &r.k,
                       qname, &r.B, &r.stage, &r.ksplit);
        if (n != 10) {
            rc = fail(MOE_ERR_INVALID_ARG, "%s:%d: expected cu,T,d,f,E,k,quant,B,stage,ksplit", path, lineno);
            break;
        }
        if (!strcmp(qname, "bf16") || !strcmp(qname, "0")) r.quant = 0;
        else if (!strcmp(qname, "fp8_token") || !strcmp(qname, "1")) r.quant = 1;
        else if (!strcmp(qname, "fp8_block") || !strcmp(qname, "2")) r.quant = 2;
        else if (!strcmp(qname, "mxfp4") || !strcmp(qname, "3")) r.quant = MOE_QUANT_MXFP4;
        else {
            rc = fail(MOE_ERR_INVALID_ARG, "%s:%d: unknown quant '%s'", path, lineno, qname);
            break;
        }
        if (r.cu < 1 || r.T < 1 || (r.stage != 1 && r.stage != 2) || r.ksplit < 1) {
            rc = fail(MOE_ERR_INVALID_ARG, "%s:%d: bad cu / T / stage / ksplit", path, lineno);
            break;
        }
        const GemmShape sh{r.T, r.d, r.f, r.E, r.k, r.B, r.quant};
        const int cs = check_shape(r.T, r.d, r.f, r.E, r.k, r.B, r.quant);
        if (cs != MOE_OK) {
            char why[512];
            snprintf(why, sizeof why, "%s", g_err);
            rc = fail(cs, "%s:%d: %s", path, lineno, why);
            break;
        }
        bool ok = true;
        if (r.stage == 1) ok = onestage_supported(sh);
        if (r.stage == 2)
            ok = use_tiled(r.B) ? tiled_gemm_supported(sh)
                                : stream_gemm1_supported(sh) && stream_gemm2_supported(sh);
        if (!ok) {
            rc = fail(MOE_ERR_UNSUPPORTED, "%s:%d: no kernels for B=%d stage=%d at this shape", path,
                      lineno, r.B, r.stage);
            break;
        }
        table.push_back(r);
    }
    fclose(fp);
    if (rc != MOE_OK) return rc;
    std::lock_guard<std::mutex> lock(g_table_mu);
    g_table.swap(table);
    if (rows) *rows = (int)g_table.size();
    return MOE_OK;
}

int moe_select_config(int T, int d, int f, int E, int k, int quant, int cu_count, int *B,
                      int *stage, int *ksplit) {
    g_err[0] = 0;
    if (!B || !stage || !ksplit) return fail(MOE_ERR_INVALID_ARG, "null pointer");
    int rc = check_shape(T, d, f, E, k, 32, quant);
    if (rc) return rc;
    if (cu_count <= 0) cu_count = cu_count_cached();
    Config c = choose(T, d, f, E, k, quant, cu_count);
    *B = c.B;
    *stage = c.stage;
    *ksplit = c.ksplit;
    return MOE_OK;
}

static int resolve(int T, int d, int f, int E, int k, int quant, int *B, int *stage) {
    if (*B == 0 || *stage == 0) {
        Config c = choose(T, d, f, E, k, quant, cu_count_cached());
        if (*B == 0) *B = c.B;
        if (*stage == 0) *stage = c.stage;
    }
    if (*stage != 1 && *stage != 2) return fail(MOE_ERR_INVALID_ARG, "bad stage %d", *stage);
    int rc = check_shape(T, d, f, E, k, *B, quant);
    if (rc) return rc;
    if (*stage == 1 && !onestage_supported(GemmShape{T, d, f, E, k, *B, quant}))
        return fail(MOE_ERR_UNSUPPORTED,
                    "the one-stage kernel takes bf16 with B = 16 or 32 (got quant=%d B=%d)", quant, *B);
    return MOE_OK;
}

size_t fused_moe_workspace_bytes(int T, int d, int f, int E, int k, int quant, int B, int stage) {
    if (resolve(T, d, f, E, k, quant, &B, &stage) != MOE_OK) return 0;
    Carver c(nullptr);
    carve_fused(c, T, d, f, E, k, quant, B, true);
    return c.bytes();
}

}  // extern "C"

namespace {
// The whole layer on a workspace of ws_bytes at ws (fused_moe and its
// no-allocation variant).
int fused_impl(int T, int d, int f, int E, int k, int quant, int score, int renorm,
               const float *logits, const int32_t *topk_ids, const float *topk_w, const void *x,
               const void *w13, const void *w13_scale, const void *w2, const void *w2_scale,
               int B, int stage, int ksplit, void *out, void *ws, size_t ws_bytes, void *stream) {
    int rc = resolve(T, d, f, E, k, quant, &B, &stage);
    if (rc) return rc;
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARG, "bad score %d", score);
    if (T > 0 && (!x || !out || (!logits && (!topk_ids || !topk_w))))
        return fail(MOE_ERR_INVALID_ARG, "null pointer");
    if (!w13 || !w2) return fail(MOE_ERR_INVALID_ARG, "null weights");
    if (quant != 0 && (!w13_scale || !w2_scale)) return fail(MOE_ERR_INVALID_ARG, "fp8 and MXFP4 need scales");
    Carver c(nullptr);
    carve_fused(c, T, d, f, E, k, quant, B, true);
    if (ws_bytes < c.bytes() || !ws)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, c.bytes());
    if (T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    Carver cw(ws);
    FusedWs w = carve_fused(cw, T, d, f, E, k, quant, B, true);
    // the one-stage path needs a cleared accumulator before its kernel; the
    // routing+sort workgroup clears small ones on the way
    const size_t acc_n = (size_t)T * d;
    float *const acc = w.g2.acc;
    // Routing runs inside the sort's single workgroup for small T * E (one
    // launch less); beyond that the one-wave-per-token routing kernel plus the
    // sort is faster (whole layer, MI355X: T=128, E=256 1692 -> 1595 us;
    // T=4096, E=8 2930 -> 2870 us; T=32, E=8 unchanged).
    const bool fuse_route = (int64_t)T * E <= MOE_FUSE_ROUTE_MAX;
    const bool zero_in_sort = stage == 1 && logits && fuse_route && acc_n <= (size_t(1) << 20);
    // With logits, the routing launch also quantises the activations on
    // workgroups of its own (they do not depend on the routing), which then
    // run beside the one-workgroup route+sort or the top-k waves instead of
    // in a launch of their own (per-token e4m3: and clears the row amax of h).
    ActQuant aq{};
    if (logits && quant != 0) {
        aq.x = static_cast<const uint16_t *>(x);
        aq.rows = T;
        aq.cols = d;
        aq.codes = w.g1.qx;
        if (quant == MOE_QUANT_MXFP4) {
            aq.kind = ACT_QUANT_MX;
            aq.mx_scales = w.g1.sxm;
        } else {
            aq.kind = quant == 1 ? ACT_QUANT_ROW : ACT_QUANT_BLOCK;
            aq.scales = w.g1.sx;
            if (quant == 1) {
                aq.zero = w.g1.amax;
                aq.zero_n = (int)max_padded(T, k, E, B);
            }
        }
    }
    const bool x_ready = aq.kind != ACT_QUANT_NONE;
    if (logits && fuse_route) {
        HIP_TRY(launch_route_sort(logits, T, k, E, B, score, renorm, w.topk_ids, w.topk_w,
                                  w.sorted_ids, w.sorted_w, w.seid, w.counts, w.offsets,
                                  w.num_valid, s, zero_in_sort ? acc : nullptr,
                                  zero_in_sort ? (int)acc_n : 0, &aq),
                "route+sort launch");
    } else if (logits) {
        HIP_TRY(launch_topk(logits, T, E, k, score, renorm, w.topk_ids, w.topk_w, s, &aq), "topk launch");
        HIP_TRY(launch_sort(w.topk_ids, w.topk_w, T, k, E, B, w.sorted_ids, w.sorted_w, w.seid,
                            w.counts, w.offsets, w.num_valid, s),
                "sort launch");
    } else {
        HIP_TRY(launch_sort(topk_ids, topk_w, T, k, E, B, w.sorted_ids, w.sorted_w, w.seid,
                            w.counts, w.offsets, w.num_valid, s),
                "sort launch");
    }
    if (stage == 1) {
        if (!zero_in_sort) HIP_TRY(launch_fill_f32(acc, acc_n, 0.0f, s), "fill launch");
        HIP_TRY(launch_moe_1stage(GemmShape{T, d, f, E, k, B, quant}, x, w13, w2, w.sorted_ids,
                                  w.sorted_w, w.seid, acc, s),
                "one-stage launch");
        HIP_TRY(launch_finalize(acc, static_cast<uint16_t *>(out), acc_n, s), "finalize launch");
        return MOE_OK;
    }
    // GEMM1 also clears GEMM2's accumulator (same stream, so it is done first)
    // unless GEMM2 stores whole rows
    if (ksplit <= 0) ksplit = pick_ksplit(T, d, f, E, k, B, quant, cu_count_cached());
    const bool clear = !stored_rows(B, ksplit);
    rc = run_gemm1(T, d, f, E, k, B, quant, x, w13, w13_scale, w.sorted_ids, w.seid, w.num_valid,
                   w.h, w.h_scale, w.g1, s, clear ? acc : nullptr, clear ? (size_t)T * d : 0, x_ready);
    if (rc) return rc;
    return run_gemm2(T, d, f, E, k, B, quant, ksplit, w.h, w.h_scale, w2, w2_scale, w.sorted_ids,
                     w.sorted_w, w.seid, w.num_valid, out, w.g2, logits != nullptr, s, true);
}

// ------------------------------------------------- no-allocation variant
// The workspace of fused_moe_noalloc: one array per GPU, loaded with the
// library's code object and held until the process ends. Host code never
// uses the name `scratch` as an address (on the host it is only a stand-in
// for the device symbol): the device address is looked up per device with
// hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES] = {};

// The current device's scratch address (looked up on the device's first
// call, with that device current).
int scratch_address(void **out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(MOE_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    MAX_DEVICES - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}
}  // namespace

extern "C" {

int fused_moe(int T, int d, int f, int E, int k, int quant, int score, int renorm,
              const float *logits, const int32_t *topk_ids, const float *topk_w, const void *x,
              const void *w13, const void *w13_scale, const void *w2, const void *w2_scale,
              int B, int stage, int ksplit, void *out, void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    return fused_impl(T, d, f, E, k, quant, score, renorm, logits, topk_ids, topk_w, x, w13, w13_scale,
                      w2, w2_scale, B, stage, ksplit, out, ws, ws_bytes, stream);
}

int fused_moe_noalloc(int T, int d, int f, int E, int k, int quant, int score, int renorm,
                      const float *logits, const int32_t *topk_ids, const float *topk_w,
                      const void *x, const void *w13, const void *w13_scale, const void *w2,
                      const void *w2_scale, int B, int stage, int ksplit, void *out, void *stream) {
    g_err[0] = 0;
    int Br = B, stage_r = stage;
    int rc = resolve(T, d, f, E, k, quant, &Br, &stage_r);
    if (rc) return rc;
    Carver c(nullptr);
    carve_fused(c, T, d, f, E, k, quant, Br, true);
    if (c.bytes() > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_UNSUPPORTED,
                    "this layer needs %zu bytes of workspace; the static scratch of fused_moe_noalloc "
                    "holds %zu (use fused_moe with a caller-allocated workspace)",
                    c.bytes(), (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return fused_impl(T, d, f, E, k, quant, score, renorm, logits, topk_ids, topk_w, x, w13, w13_scale,
                      w2, w2_scale, Br, stage_r, ksplit, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
