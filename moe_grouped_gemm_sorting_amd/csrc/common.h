// common.h -- device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    __bf16 b = (__bf16)v;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}

// Two fp32 -> two OCP e4m3 codes (low 16 bits), round to nearest even,
// saturating at +-448 (the clamp makes saturation independent of the
// converter's overflow mode). Inputs are finite.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// z * sigmoid(z) from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32; about 1 ulp each): the relative error, near 1e-6,
// is far below the bf16 rounding that follows. exp2 overflowing to +inf for
// very negative z gives 1/inf = 0, the limit.
// MXFP4 (per_1x32): E2M1 code of r (round to nearest, ties to the code with
// mantissa 0, saturating at +-6): the magnitude code counts the rounding
// thresholds below |r|, which are the midpoints between neighbouring values
// (0.25 .. 5); a tie goes up where the upper neighbour has mantissa 0.
__device__ __forceinline__ uint32_t e2m1_code(float r) {
    const float a = fabsf(r);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return m | ((__float_as_uint(r) >> 28) & 8u);
}

// Eight E2M1 codes packed in a dword (v[i] in nibble i) by gfx950's
// v_cvt_scalef32_pk_fp4_f32 at unit scale, two values per instruction. It
// rounds exactly as e2m1_code (checked on the GPU against it for every
// threshold and its neighbouring floats, denormals, signed zeros and values
// past 6, in each byte position).
__device__ __forceinline__ uint32_t e2m1_pack8(const float *v) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
    return w;
}

// Shared exponent of an MXFP4 block from its amax: floor(log2(amax)) - 2,
// clamped to [-127, 127] (-127 for zero or subnormal amax), read off the
// fp32 exponent field. Returns E; the E8M0 code is E + 127.
__device__ __forceinline__ int mx_block_exp(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 255u);
    return ef == 0 ? -127 : max(-127, ef - 127 - 2);
}

// 2^-E as an fp32 (E in [-127, 126], so 127 - E is a normal exponent field)
__device__ __forceinline__ float mx_inv_scale(int E) { return __uint_as_float((uint32_t)(127 - E) << 23); }

__device__ __forceinline__ float silu(float z) {
    constexpr float kLog2e = 1.44269504088896341f;
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// logistic sigmoid and the derivative of silu: silu'(z) = s (1 + z (1 - s))
__device__ __forceinline__ float sigmoid(float z) {
    constexpr float kLog2e = 1.44269504088896341f;
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}
__device__ __forceinline__ float silu_grad(float z) {
    const float s = sigmoid(z);
    return s * (1.0f + z * (1.0f - s));
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (WAVE - 1);
    return lane == 0 ? 0ull : (~0ull >> (WAVE - lane));
}

// Non-returning fp32 atomic add to global memory (global_atomic_add_f32).
__device__ __forceinline__ void atomic_add_f32(float *p, float v) { unsafeAtomicAdd(p, v); }

// Max of non-negative floats through their bit patterns (monotone for >= 0).
__device__ __forceinline__ void atomic_max_nonneg(float *p, float v) {
    atomicMax(reinterpret_cast<unsigned int *>(p), __float_as_uint(v));
}

// compile-time integer, and f(IC<0>{}), ..., f(IC<N-1>{})
template <int I>
struct IC {
    static constexpr int value = I;
};
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(IC<I>{});
        static_for<N, I + 1>(f);
    }
}

}  // namespace moe
