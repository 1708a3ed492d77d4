// route_sort.hip -- top-k routing and the stable block-padded token sort.
//
// Routing is the gating stage of the fused MoE pipeline and the sort is its
// token re-sort stage (AITER walk-through, itsolotime.com/th/archives/32381,
// section 3 and section 3.1). The sort is an exact counting sort; every rank
// comes from ordered wave ballots and per-wave prefix counts, never from the
// order in which atomics land, so the result is bit-exact and repeatable.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "moe.h"
#include "quant_body.h"

namespace moe {

// workgroups of the sort for large T*k (1 = the single-workgroup sort)
#ifndef MOE_SORT_MAX_PARTS
#define MOE_SORT_MAX_PARTS 64
#endif

// ---------------------------------------------------------------- routing
// One wave per token; lane l holds the logits of experts l, l + 64, ...
// k rounds of a (logit descending, expert ascending) wave argmax pick the
// experts; lane j keeps selection j.
template <int PER_LANE>
__device__ __forceinline__ void topk_wave(const float *__restrict__ logits, int t, int E, int k,
                                          int score, int renorm, int32_t *__restrict__ ids,
                                          float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const float *row = logits + (size_t)t * E;
    float v[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? row[e] : -INFINITY;
    }
    uint32_t taken = 0;
    float my_val = 0.0f;
    int my_id = 0;
    float top = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bi == 0x7fffffff)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_val = bv;
            my_id = bi;
        }
        if (j == 0) top = bv;
    }
    float p;
    if (score == 0) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (lane + 64 * i < E) part += expf(v[i] - top);
        const float den = wave_sum(part);
        p = expf(my_val - top) / den;
    } else {
        p = 1.0f / (1.0f + expf(-my_val));
    }
    // sum of the selected scores in selection order, as one sequential chain
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __shfl(p, j, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        w[(size_t)t * k + lane] = renorm ? p / sum : p;
    }
}

// Workgroups [0, route_wgs) route four tokens each; the ones after carry the
// activation quantisation aq.
template <int PER_LANE>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E,
                                              int k, int score, int renorm,
                                              int32_t *__restrict__ ids,
                                              float *__restrict__ w, ActQuant aq, int route_wgs) {
    if ((int)blockIdx.x >= route_wgs) {
        act_quant_part<256>(aq, blockIdx.x - route_wgs, gridDim.x - route_wgs);
        return;
    }
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave<PER_LANE>(logits, t, E, k, score, renorm, ids, w);
}

// One thread per token, for E <= EMAX <= 64: the same selection and scores,
// with every sum taken in ascending expert / selection order. The row's
// logits are loaded into registers up front (independent loads, one round
// trip), and the selected logits and scores stay in registers.
template <int EMAX>
__device__ __forceinline__ void topk_thread(const float *__restrict__ logits, int t, int E, int k,
                                            int score, int renorm, int32_t *__restrict__ ids,
                                            float *__restrict__ w) {
    const float *row = logits + (size_t)t * E;
    float v[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) v[e] = e < E ? row[e] : 0.0f;
    uint64_t taken = 0;
    float top = 0.0f;
    float sel[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j >= k) break;
        int best = -1;
        float bv = 0.0f;
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            if (e < E && !((taken >> e) & 1ull) && (best < 0 || v[e] > bv)) {
                best = e;
                bv = v[e];
            }
        }
        taken |= 1ull << best;
        if (j == 0) top = bv;
        ids[(size_t)t * k + j] = best;
        sel[j] = bv;   // raw logit for now
    }
    float den = 1.0f;
    if (score == 0) {
        den = 0.0f;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) den += expf(v[e] - top);
    }
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j >= k) break;
        const float l = sel[j];
        const float p = score == 0 ? expf(l - top) / den : 1.0f / (1.0f + expf(-l));
        sel[j] = p;
        sum += p;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j >= k) break;
        w[(size_t)t * k + j] = renorm ? sel[j] / sum : sel[j];
    }
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int score, int renorm,
                       int32_t *ids, float *w, hipStream_t s, const ActQuant *aq) {
    if (T == 0) return hipSuccess;
    const ActQuant q = aq ? *aq : ActQuant{};
    const int route_wgs = (T + 3) / 4;
    const dim3 grid(route_wgs + act_quant_groups(q, 256)), block(256);
    if (E <= 64)
        k_topk<1><<<grid, block, 0, s>>>(logits, T, E, k, score, renorm, ids, w, q, route_wgs);
    else if (E <= 128)
        k_topk<2><<<grid, block, 0, s>>>(logits, T, E, k, score, renorm, ids, w, q, route_wgs);
    else if (E <= 256)
        k_topk<4><<<grid, block, 0, s>>>(logits, T, E, k, score, renorm, ids, w, q, route_wgs);
    else if (E <= 512)
        k_topk<8><<<grid, block, 0, s>>>(logits, T, E, k, score, renorm, ids, w, q, route_wgs);
    else
        k_topk<16><<<grid, block, 0, s>>>(logits, T, E, k, score, renorm, ids, w, q, route_wgs);
    return hipGetLastError();
}

// ------------------------------------------------------------------- sort
// The N = T*k assignments are cut into `nparts` contiguous chunks, one per
// workgroup of SORT_WAVES waves, and each chunk into SORT_WAVES contiguous
// segments, one per wave, so that "earlier wave" (or "earlier workgroup")
// means "smaller assignment index". No workgroup needs another's results:
//   1. count: every workgroup counts all N assignments: cnt[w][e] for wave
//      w's segment of its own chunk, below[e] / after[e] for the
//      assignments before / after the chunk (LDS atomics; counts are
//      order-free);
//   2. scan: the totals give the padded expert sizes, scanned into off[]
//      (the same in every workgroup), and cnt[w][e] becomes below[e] plus the
//      exclusive prefix over the chunk's waves;
//   3. scatter: each wave walks its segment 64 assignments at a time; the
//      rank of an assignment among equal experts in the chunk comes from a
//      peer mask built from log2(E) bit-plane ballots;
//   4. the padding slots of a share of the experts, a share of the tail and
//      of the per-block expert ids are filled by each workgroup.
// With one workgroup this is the whole sort in one launch (below = after = 0).
constexpr int SORT_WAVES = 8;
constexpr int SORT_THREADS = SORT_WAVES * 64;

__device__ __forceinline__ void sort_part(
    const int32_t *__restrict__ ids, const float *__restrict__ wts, int N, int E, int B, int P,
    int NB, int part, int nparts, int32_t *__restrict__ sorted_ids, float *__restrict__ sorted_w,
    int32_t *__restrict__ seid, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ num_valid) {
    extern __shared__ int lds[];
    int *cnt = lds;                     // [SORT_WAVES][E]
    int *tot = cnt + SORT_WAVES * E;    // [E]
    int *off = tot + E;                 // [E + 1]
    int *below = off + E + 1;           // [E]
    int *after = below + E;             // [E]
    __shared__ int wave_sum_lds[SORT_WAVES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < SORT_WAVES * E; i += SORT_THREADS) cnt[i] = 0;
    for (int i = tid; i < E; i += SORT_THREADS) below[i] = after[i] = 0;
    __syncthreads();

    // this workgroup's chunk [cbeg, cend) and this wave's segment of it
    const int chunk = (((N + nparts - 1) / nparts) + 63) / 64 * 64;
    const int cbeg = min(N, part * chunk), cend = min(N, cbeg + chunk);
    const int seg = ((((cend - cbeg) + SORT_WAVES - 1) / SORT_WAVES) + 63) / 64 * 64;
    const int beg = min(cend, cbeg + wave * seg), end = min(cend, beg + seg);
    for (int a = beg + lane; a < end; a += 64) {
        const int e = ids[a];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[wave * E + e], 1);
    }
    if (nparts > 1) {
        // the assignments outside the chunk, 8 independent loads per thread
        // ahead of their atomics
        auto count_range = [&](int lo, int hi, int *h) {
            for (int a0 = lo + tid; a0 < hi; a0 += 8 * SORT_THREADS) {
                int e[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int a = a0 + u * SORT_THREADS;
                    e[u] = a < hi ? ids[a] : -1;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if ((unsigned)e[u] < (unsigned)E) atomicAdd(&h[e[u]], 1);
            }
        };
        count_range(0, cbeg, below);
        count_range(cend, N, after);
    }
    __syncthreads();

    int carry = 0;
    for (int base = 0; base < E; base += SORT_THREADS) {
        const int e = base + tid;
        int pad = 0;
        if (e < E) {
            int t = below[e];
            for (int w = 0; w < SORT_WAVES; ++w) {
                const int c = cnt[w * E + e];
                cnt[w * E + e] = t;
                t += c;
            }
            t += after[e];
            tot[e] = t;
            if (part == 0) counts[e] = t;
            pad = (t + B - 1) / B * B;
        }
        int incl = pad;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
        }
        if (lane == 63) wave_sum_lds[wave] = incl;
        __syncthreads();
        int before = 0, all = 0;
        for (int w = 0; w < SORT_WAVES; ++w) {
            const int ws = wave_sum_lds[w];
            before += (w < wave) ? ws : 0;
            all += ws;
        }
        if (e < E) off[e] = carry + before + incl - pad;
        carry += all;
        __syncthreads();
    }
    if (tid == 0) off[E] = carry;
    __syncthreads();
    const int nv = off[E];
    if (part == 0) {
        for (int e = tid; e <= E; e += SORT_THREADS) offsets[e] = off[e];
        if (tid == 0) *num_valid = nv;
    }

    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const uint64_t lt = lanemask_lt();
    for (int a0 = beg; a0 < end; a0 += 64) {
        const int a = a0 + lane;
        int e = a < end ? ids[a] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        int basecnt = 0, rank = 0;
        if (valid) {
            rank = __popcll(peers & lt);
            basecnt = cnt[wave * E + e];
            const int pos = off[e] + basecnt + rank;
            sorted_ids[pos] = a;
            sorted_w[pos] = wts[a];
        }
        if (valid && rank == 0) cnt[wave * E + e] = basecnt + __popcll(peers);
    }

    // this part's share of the slots: the padding at the end of each
    // expert's segment, the tail after the last segment, and the per-block
    // expert ids. A slot's expert is the last e with off[e] <= slot (a
    // binary search over off[], so the work spreads over every thread
    // whatever E is).
    auto owner_of = [&](int slot) {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= slot) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    const int gtid = part * SORT_THREADS + tid, gstride = nparts * SORT_THREADS;
    for (int i = gtid; i < P; i += gstride) {
        bool pad = i >= nv;
        if (!pad) {
            const int e = owner_of(i);
            pad = i >= off[e] + tot[e];
        }
        if (pad) {
            sorted_ids[i] = N;
            sorted_w[i] = 0.0f;
        }
    }
    for (int b = gtid; b < NB; b += gstride) {
        const int slot = b * B;
        seid[b] = slot < nv ? owner_of(slot) : -1;
    }
}

__global__ __launch_bounds__(SORT_THREADS) void k_sort(
    const int32_t *__restrict__ ids, const float *__restrict__ wts, int N, int E, int B, int P,
    int NB, int32_t *__restrict__ sorted_ids, float *__restrict__ sorted_w,
    int32_t *__restrict__ seid, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ num_valid) {
    sort_part(ids, wts, N, E, B, P, NB, blockIdx.x, gridDim.x, sorted_ids, sorted_w, seid, counts,
              offsets, num_valid);
}

// Routing and sort in one launch (one workgroup): top-k of every token into
// ids / w, a workgroup barrier (which also orders the global writes for the
// workgroup), then the sort. Workgroups after the first carry the activation
// quantisation aq.
constexpr int ROUTE_SORT_MAX_N = 512;   // assignments T * k of the one-workgroup form
template <int PER_LANE>
__global__ __launch_bounds__(SORT_THREADS) void k_route_sort(
    const float *__restrict__ logits, int T, int k, int E, int B, int score, int renorm,
    int32_t *__restrict__ ids, float *__restrict__ wts, int P, int NB,
    int32_t *__restrict__ sorted_ids, float *__restrict__ sorted_w, int32_t *__restrict__ seid,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ num_valid,
    float *__restrict__ zero, int zero_n, ActQuant aq) {
    if (blockIdx.x > 0) {
        act_quant_part<SORT_THREADS>(aq, blockIdx.x - 1, gridDim.x - 1);
        return;
    }
    // optionally clear a (small) fp32 accumulator for the next stage
    if (zero)
        for (int i = threadIdx.x; i < zero_n / 4; i += SORT_THREADS)
            reinterpret_cast<float4 *>(zero)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    // the selections go to LDS, where the sort reads them, and are copied
    // out to ids / wts afterwards (T * k <= ROUTE_SORT_MAX_N, checked by the
    // launcher)
    __shared__ int32_t s_ids[ROUTE_SORT_MAX_N];
    __shared__ float s_w[ROUTE_SORT_MAX_N];
    if constexpr (PER_LANE <= 0) {
        // one thread per token, E <= -PER_LANE
        for (int t = threadIdx.x; t < T; t += SORT_THREADS)
            topk_thread<PER_LANE < 0 ? -PER_LANE : 1>(logits, t, E, k, score, renorm, s_ids, s_w);
    } else {
        for (int t = threadIdx.x >> 6; t < T; t += SORT_WAVES)
            topk_wave<PER_LANE <= 0 ? 1 : PER_LANE>(logits, t, E, k, score, renorm, s_ids, s_w);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * k; i += SORT_THREADS) {
        ids[i] = s_ids[i];
        wts[i] = s_w[i];
    }
    sort_part(s_ids, s_w, T * k, E, B, P, NB, 0, 1, sorted_ids, sorted_w, seid, counts, offsets,
              num_valid);
}

hipError_t launch_route_sort(const float *logits, int T, int k, int E, int B, int score,
                             int renorm, int32_t *ids, float *w, int32_t *sorted_ids,
                             float *sorted_w, int32_t *sorted_expert_ids, int32_t *counts,
                             int32_t *offsets, int32_t *num_valid, hipStream_t s, float *zero,
                             int zero_n, const ActQuant *aq) {
    if ((int64_t)T * k > ROUTE_SORT_MAX_N) return hipErrorInvalidValue;
    const ActQuant q = aq ? *aq : ActQuant{};
    const unsigned wgs = 1 + (unsigned)act_quant_groups(q, SORT_THREADS);
    const int P = T * k + E * B - k;
    const int NB = (P + B - 1) / B;
    const size_t lds = sizeof(int) * ((size_t)SORT_WAVES * E + 4 * (size_t)E + 1);
#define MOE_ROUTE_SORT(PL)                                                                    \
    k_route_sort<PL><<<wgs, SORT_THREADS, lds, s>>>(logits, T, k, E, B, score, renorm, ids, w, P, \
                                                     NB, sorted_ids, sorted_w, sorted_expert_ids, \
                                                     counts, offsets, num_valid, zero, zero_n, q)
    if (E <= 8) MOE_ROUTE_SORT(-8);
    else if (E <= 16) MOE_ROUTE_SORT(-16);
    else if (E <= 32) MOE_ROUTE_SORT(-32);
    else if (E <= 64) MOE_ROUTE_SORT(-64);
    else if (E <= 128) MOE_ROUTE_SORT(2);
    else if (E <= 256) MOE_ROUTE_SORT(4);
    else if (E <= 512) MOE_ROUTE_SORT(8);
    else MOE_ROUTE_SORT(16);
#undef MOE_ROUTE_SORT
    return hipGetLastError();
}

hipError_t launch_sort(const int32_t *ids, const float *w, int T, int k, int E, int B,
                       int32_t *sorted_ids, float *sorted_w, int32_t *sorted_expert_ids,
                       int32_t *counts, int32_t *offsets, int32_t *num_valid, hipStream_t s) {
    const int N = T * k;
    const int P = N + E * B - k;
    const int NB = (P + B - 1) / B;
    const size_t lds = sizeof(int) * ((size_t)SORT_WAVES * E + 4 * (size_t)E + 1);
    // chunks of at least 512 assignments (one 64-assignment step per wave),
    // at most 64 workgroups (each counts all N assignments)
    const int parts = std::max(1, std::min(MOE_SORT_MAX_PARTS, N / 512));
    k_sort<<<parts, SORT_THREADS, lds, s>>>(ids, w, N, E, B, P, NB, sorted_ids, sorted_w,
                                            sorted_expert_ids, counts, offsets, num_valid);
    return hipGetLastError();
}

}  // namespace moe
