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
    // normal range [2^-6, 448): keep 3 of the 23 mantissa bits, round to nearest even by
    // adding 0x7FFFF plus the lowest kept bit (a carry out of the mantissa bumps the exponent),
    // then rebias the exponent from 127 to 7 (120 << 3 in the code's units)
    const uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    // below 2^-6: the subnormal grid m * 2^-9, m = RNE(|y| * 512) in 0..8 (exact scaling)
    const uint32_t sub =
        (uint32_t)__builtin_rintf(__uint_as_float(a < 0x3C800000u ? a : 0u) * 512.0f);
    uint32_t code = a < 0x3C800000u ? sub : normal;
    code = a >= 0x43E00000u ? 0x7Eu : code;               // |y| >= 448 saturates
    return a > 0x7F800000u ? 0x7Fu : (sign | code);       // NaN
}

// Four values to OCP E4M3FN codes with the hardware converter (gfx950 V_CVT_PK_FP8_F32:
// round to nearest even, subnormals m * 2^-9, signed zeros kept), bytes in argument order.
// The inputs are clamped to [-448, 448] first, so |y| >= 448 gives 0x7E|sign as in
// e4m3_encode: the same codes for every finite input (checked against it and the oracle by a
// dense sweep of fp32 bit patterns).
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Router selection key of logit v of expert e: the high word orders the float (-0 ranks equal
// to +0; a NaN ranks below every number, -inf included, and NaNs tie with each other), the low
// word holds 0xFFFFFFFF - e so equal logits resolve to the lower expert index.  Keys of one
// token's experts are distinct; its top-k are the k largest keys.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) ord = 0u;    // NaN: below -inf (0x007FFFFF)
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
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

// monotone 32-bit image of a logit (the high word of route_key)
__device__ __forceinline__ uint32_t logit_ord(float v) { return (uint32_t)(route_key(v, 0) >> 32); }

// maximum over the 64 lanes: inclusive max-scans inside each row of 16 lanes (row_shr 1, 2, 4,
// 8), then the row totals carried across rows (row_bcast 15 into rows 1 and 3, row_bcast 31
// into rows 2 and 3); lane 63 ends with the wave's maximum.  Lanes a shift leaves without a
// source take 0, which is below or equal to every image.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define MOE_DPP_MAX(ctrl, rows) \
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, rows, 0xf, false))
    MOE_DPP_MAX(0x111, 0xf);
    MOE_DPP_MAX(0x112, 0xf);
    MOE_DPP_MAX(0x114, 0xf);
    MOE_DPP_MAX(0x118, 0xf);
    MOE_DPP_MAX(0x142, 0xa);
    MOE_DPP_MAX(0x143, 0xc);
#undef MOE_DPP_MAX
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One token's routing by one wave ([FMF8] "Baseline: 7 kernels", item 1): the E logits of
// `row`, VPL per lane (expert lane + 64 i; loads past E clamped), first loaded by
// route_load_row, then route_select: k rounds of a wave-wide maximum of the monotone image
// (ties to the lower expert index), the k winners' values capped by softcap * tanh(v /
// softcap) (softcap <= 0: no cap) and renormalised by a softmax over the k.  Lane j < k ends
// with the j-th selected expert (descending order) and its weight.
template <int VPL>
__device__ __forceinline__ void route_load_row(const float* row, int E, int lane,
                                               float (&val)[VPL]) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) val[i] = row[min(lane + 64 * i, E - 1)];
}

template <int VPL>
__device__ __forceinline__ void route_select(const float (&val)[VPL], int E, int k,
                                             float softcap, int lane, int& my_e, float& my_w) {
    uint32_t ord[VPL];
    uint64_t avail[VPL];                        // experts not yet taken (bit per lane)
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        ord[i] = logit_ord(val[i]);
        avail[i] = __ballot(lane + 64 * i < E);
    }
    my_e = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t loc = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            loc = max(loc, (avail[i] >> lane) & 1ull ? ord[i] : 0u);
        const uint32_t m = wave_max_u32(loc);
        // the lowest-index available expert holding the maximum
        int win_i = -1, win_l = 0;
#pragma unroll
        for (int i = VPL - 1; i >= 0; --i) {
            const uint64_t hit = __ballot(ord[i] == m) & avail[i];
            if (hit) {
                win_i = i;
                win_l = __builtin_ctzll(hit);
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (i == win_i) avail[i] &= ~(1ull << win_l);
        float wl = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (i == win_i)
                wl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val[i]), win_l));
        if (lane == j) {
            my_e = win_l + 64 * win_i;
            my_l = wl;
        }
    }
    const bool active = lane < k;
    float c = my_l;
    if (softcap > 0.0f) c = softcap * tanhf(my_l / softcap);
    const float c0 = __shfl(c, 0);                         // the largest selected value
    const float ex = active ? expf(c - c0) : 0.0f;
    const float sum = wave_sum(ex);
    my_w = ex / sum;
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

// Quantise 8 consecutive bf16 values (one 16-byte load) that belong to a 128-value block
// spread over an aligned group of 16 lanes: the block amax is reduced over the group, then
// every value is encoded with the block's reciprocal scale.  Lanes with valid == false add
// nothing to the amax.
struct Quant8 {
    uint2 codes;
    float scale;
};

// The same on 8 fp32 values (the requantiser of the expert MLP's activations).
__device__ __forceinline__ Quant8 quantise8_f32(const float (&v)[8], bool valid) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = max16(valid ? amax : 0.0f);
    const QScale q = block_scale(amax);
    Quant8 out;
    out.codes.x = e4m3_encode4(v[0] * q.inv, v[1] * q.inv, v[2] * q.inv, v[3] * q.inv);
    out.codes.y = e4m3_encode4(v[4] * q.inv, v[5] * q.inv, v[6] * q.inv, v[7] * q.inv);
    out.scale = q.scale;
    return out;
}

__device__ __forceinline__ Quant8 quantise8(uint4 raw, bool valid) {
    float v[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    return quantise8_f32(v, valid);
}

// Token t's values [k_lo, k_hi) of x bf16 [M][K] (whole 128-value blocks) quantised by one
// wave with the rule of the QSG stage into token-major codes x_q [M][K] and scales
// x_scales [K/128][M].  512 values per pass: lane l holds values [8l, 8l+8) of the pass, so a
// 128-value block is an aligned group of 16 lanes, wholly inside or outside the slice.
__device__ __forceinline__ void quantise_token_slice(const uint16_t* __restrict__ x, int M,
                                                     int K, int t, int k_lo, int k_hi,
                                                     uint8_t* __restrict__ x_q,
                                                     float* __restrict__ x_scales, int lane) {
    constexpr int kPasses = 2;
    for (int base = k_lo; base < k_hi; base += kPasses * 512) {
        uint4 xr[kPasses];
#pragma unroll
        for (int q = 0; q < kPasses; ++q) {
            const int k0 = base + q * 512 + lane * 8;
            xr[q] = make_uint4(0u, 0u, 0u, 0u);
            if (k0 < k_hi) xr[q] = *reinterpret_cast<const uint4*>(x + (size_t)t * K + k0);
        }
#pragma unroll
        for (int q = 0; q < kPasses; ++q) {
            const int k0 = base + q * 512 + lane * 8;
            const bool valid = k0 < k_hi;
            const Quant8 qv = quantise8(xr[q], valid);
            if (valid) {
                *reinterpret_cast<uint2*>(x_q + (size_t)t * K + k0) = qv.codes;
                if ((lane & 15) == 0) x_scales[(size_t)(k0 >> 7) * M + t] = qv.scale;
            }
        }
    }
}

// ---- matrix-core operands and vector-memory ordering ----

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i pack8(uint4 lo, uint4 hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__device__ __forceinline__ v8i pack8v(u32x4 lo, u32x4 hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima): gfx9 encoding,
// vmcnt bits [3:0] and [15:14]
#define MOE_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Workgroup barrier that leaves the newest VM vector-memory operations of each wave in flight.
// Every LDS operation has completed (lgkmcnt 0) and every LDS DMA older than those VM loads
// has landed (DMA counts in vmcnt and decrements once its data is in LDS), so what was written
// to LDS before it is visible after it.  The compiler's own barrier would drain vmcnt to zero
// and with it a weight stream in flight; the signal fences only keep the compiler from moving
// memory operations across the barrier.
template <int VM>
__device__ __forceinline__ void barrier_keep_vm() {
    static_assert(VM >= 0 && VM < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 512-column piece (item = row * ceil(I/512) + piece) of the FP8 MLP's activation step
// by one wave: act = silu(g) * u in fp32 from the gate+up rows h [R][2I] (gate columns
// first), requantised per 128 columns with the QSG rule into codes [R][I] and scales
// [I/128][R].  Lane l holds columns [8l, 8l+8) of the piece, so a 128-column block is an
// aligned group of 16 lanes (I is a multiple of 128: a group lies wholly inside or outside
// the row).
// act = silu(g) * u in fp32 for 8 columns: gate values g0, g1 and up values u0, u1
__device__ __forceinline__ void silu_mul8(const float4& g0, const float4& g1, const float4& u0,
                                          const float4& u1, float (&v)[8]) {
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
}

// the same for columns [c, c+8) of one gate+up row hr [2I] (gate columns first; c a multiple
// of 8 below I)
__device__ __forceinline__ void swiglu8(const float* __restrict__ hr, int I, int c, float (&v)[8]) {
    silu_mul8(*reinterpret_cast<const float4*>(hr + c), *reinterpret_cast<const float4*>(hr + c + 4),
              *reinterpret_cast<const float4*>(hr + I + c),
              *reinterpret_cast<const float4*>(hr + I + c + 4), v);
}

__device__ __forceinline__ void swiglu_quant_piece(const float* __restrict__ h, int R, int I,
                                                   uint8_t* __restrict__ a_q,
                                                   float* __restrict__ a_scales,
                                                   long long item, int lane) {
    const int pieces = (I + 511) >> 9;
    if (item >= (long long)R * pieces) return;
    const int r = (int)(item / pieces);
    const int c = (int)(item % pieces) * 512 + lane * 8;
    const bool valid = c < I;
    float v[8];
    if (valid) {
        swiglu8(h + (size_t)r * 2 * I, I, c, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    const Quant8 q = quantise8_f32(v, valid);
    if (valid) {
        *reinterpret_cast<uint2*>(a_q + (size_t)r * I + c) = q.codes;
        if ((lane & 15) == 0) a_scales[(size_t)(c >> 7) * R + r] = q.scale;
    }
}

}  // namespace moe
