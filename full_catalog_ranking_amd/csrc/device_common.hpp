// Device-side helpers shared by the ranking-head kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace genrec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Order-preserving map float -> uint32 (larger float -> larger key).  -0 is
// folded onto +0 first so that equal scores give equal keys.
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// 64-bit ranking key: score in the high word, inverted id in the low word, so
// that a larger key means "ranks earlier" (score descending, id ascending).
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t id) {
    return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }
__device__ __forceinline__ float key_score(uint64_t k) { return key_to_score((uint32_t)(k >> 32)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (the conversion of the __bf16 type).
__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Online log-sum-exp state: sum_i exp(s_i) = l * exp(m).
struct LseState {
    float m, l;
    __device__ __forceinline__ void init() { m = -INFINITY; l = 0.f; }
    __device__ __forceinline__ void add(float s) {
        if (s > m) {
            l = l * fast_exp2((m - s) * kLog2e) + 1.f;
            m = s;
        } else {
            l += fast_exp2((s - m) * kLog2e);
        }
    }
    __device__ __forceinline__ void merge(float m2, float l2) {
        if (l2 == 0.f) return;
        if (l == 0.f) { m = m2; l = l2; return; }
        if (m2 > m) { l = l * fast_exp2((m - m2) * kLog2e) + l2; m = m2; }
        else { l += l2 * fast_exp2((m2 - m) * kLog2e); }
    }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace genrec
