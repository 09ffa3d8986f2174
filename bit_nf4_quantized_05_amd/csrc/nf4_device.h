// Device helpers shared by the quantisation and linear-layer kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "internal.h"

namespace qn {

// a_hat = mu + b * (q / 127): separate float32 division, multiply and add.
__device__ __forceinline__ float block_constant(int8_t q, float b, float mu) {
    const float rhat = static_cast<float>(q) / static_cast<float>(kInt8Step);
    const float prod = b * rhat;
    return mu + prod;
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
