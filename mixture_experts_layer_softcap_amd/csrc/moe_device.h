// moe_device.h -- device helpers shared by the gfx950 kernels: bf16 and E4M3 conversions,
// wave64 reductions, vector types.  Kernel-side code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest, ties to even (finite inputs; NaN maps to a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP E4M3FN encoding of an fp32 value: round to nearest even on the 3-bit mantissa,
// |y| >= 448 saturates to 0x7E|sign (never NaN), values below 2^-6 use the subnormal grid
// m * 2^-9, underflow keeps the sign.  NaN input gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;
    if (a >= 0x43E00000u) return sign | 0x7Eu;            // 448.0f
    if (a < 0x3C800000u) {                                 // 2^-6: subnormal grid
        const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scale, RNE
        return sign | (uint32_t)q;                         // 0..8 (8 = smallest normal)
    }
    uint32_t e = (a >> 23) - 120u;                         // biased E4M3 exponent, 1..15
    uint32_t m = a & 0x7FFFFFu;
    uint32_t keep = m >> 20;                               // 3 mantissa bits
    const uint32_t rest = m & 0xFFFFFu;                    // 20 dropped bits
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) { keep = 0u; ++e; }
    return sign | (e << 3) | keep;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Max over each aligned group of 16 lanes (one 128-wide block of 8-element lanes).
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 1));
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

// The fp32 block-quantisation constants of one 128-value block: scale = amax/448 and its
// reciprocal, both correctly rounded (plain fp32 division compiles to the IEEE sequence).
struct QScale {
    float scale;
    float inv;
};

__device__ __forceinline__ QScale block_scale(float amax) {
    QScale q;
    if (amax == 0.0f) {
        q.scale = 0.0f;
        q.inv = 0.0f;  // x*0 keeps each zero's sign, which is all an all-zero block holds
    } else {
        q.scale = amax / 448.0f;
        q.inv = 1.0f / q.scale;
    }
    return q;
}

}  // namespace moe
