// Device helpers shared by the quantisation and linear-layer kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "internal.h"

namespace qn {

// Value of OCP FP8 E4M3 code byte u (sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent 0 is subnormal, m * 2^-9). Exact in float32.
__device__ __forceinline__ float e4m3_value(uint32_t u) {
    const uint32_t e = (u >> 3) & 0xFu, m = u & 0x7u;
    const float mag = e == 0 ? static_cast<float>(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (u & 0x80u) ? -mag : mag;
}

// Nearest E4M3 code of v, |v| <= 448, ties to the even code; the sign bit is v's.
// From 2^-6 up the float32 mantissa is rounded to 3 bits (nearest, even; a carry
// moves into the exponent); below, the value is a multiple of 2^-9 rounded to
// nearest even.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    uint32_t code;
    if (mag >= 0x3C800000u) {
        const uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    } else {
        code = static_cast<uint32_t>(rintf(__uint_as_float(mag) * 512.0f));
    }
    return ((bits >> 24) & 0x80u) | code;
}

// r_hat = T[q]: q / 127 (INT8) or e4m3(q) / 448 (FP8), one float32 division.
__device__ __forceinline__ float dq_step(int fmt, int8_t q) {
    if (fmt == kDqFp8) return e4m3_value(static_cast<uint8_t>(q)) / static_cast<float>(kE4m3Max);
    return static_cast<float>(q) / static_cast<float>(kInt8Step);
}

// a_hat = mu + b * r_hat (separate float32 multiply and add); with no second level
// the stored constant itself.
__device__ __forceinline__ float block_constant(int fmt, int8_t q, float b, float mu) {
    if (fmt == kDqNone) return b;
    const float prod = b * dq_step(fmt, q);
    return mu + prod;
}

// block_constant with selects in place of branches (the same float32 operations and
// the same result), for loops where a branch would split the instruction schedule
__device__ __forceinline__ float block_constant_nb(int fmt, int8_t q, float b, float mu) {
    const uint32_t u = static_cast<uint8_t>(q);
    const uint32_t e = (u >> 3) & 0xFu, m = u & 0x7u;
    const float mag = e == 0 ? static_cast<float>(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float f8 = (u & 0x80u) ? -mag : mag;
    const bool fp8 = fmt == kDqFp8;
    const float num = fp8 ? f8 : static_cast<float>(q);
    const float den = fp8 ? static_cast<float>(kE4m3Max) : static_cast<float>(kInt8Step);
    const float prod = b * (num / den);
    return fmt == kDqNone ? b : mu + prod;
}

// Ordered sums over K-split partials: v = p[0] + p[stride] + ... + p[(n-1) stride], float32
// adds from +0.0 in that order. The loads are issued B at a time (slices past n re-read
// the last one and are masked to +0.0, which leaves a sum that started at +0.0
// unchanged), so n slices cost ceil(n / B) memory round trips instead of n.
template <int Bt>
__device__ __forceinline__ float ordered_sum(const float* __restrict__ p, int64_t stride, int n) {
    float v = 0.0f;
    for (int s0 = 0; s0 < n; s0 += Bt) {
        float t[Bt];
#pragma unroll
        for (int i = 0; i < Bt; ++i) t[i] = p[static_cast<int64_t>(min(s0 + i, n - 1)) * stride];
#pragma unroll
        for (int i = 0; i < Bt; ++i) v += s0 + i < n ? t[i] : 0.0f;
    }
    return v;
}

template <int Bt>
__device__ __forceinline__ float4 ordered_sum4(const float* __restrict__ p, int64_t stride, int n) {
    float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < n; s0 += Bt) {
        float4 t[Bt];
#pragma unroll
        for (int i = 0; i < Bt; ++i)
            t[i] = *reinterpret_cast<const float4*>(p + static_cast<int64_t>(min(s0 + i, n - 1)) * stride);
#pragma unroll
        for (int i = 0; i < Bt; ++i) {
            const bool ok = s0 + i < n;
            v.x += ok ? t[i].x : 0.0f; v.y += ok ? t[i].y : 0.0f;
            v.z += ok ? t[i].z : 0.0f; v.w += ok ? t[i].w : 0.0f;
        }
    }
    return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);    // round to nearest even (v_cvt_pk_bf16_f32)
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint16_t bf16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

}  // namespace qn
