// Device helpers shared by the MFMA kernels of the library (gfx950).
#ifndef QN_MFMA_DEVICE_H
#define QN_MFMA_DEVICE_H

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace qn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static __device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef const __attribute__((address_space(1))) void* global_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from global memory straight into LDS: lane i's data lands at
// byte 16*i after the wave-uniform LDS address `l`.
static __device__ __forceinline__ void load_lds16(const void* g, void* l) {
    __builtin_amdgcn_global_load_lds((global_ptr)g, (lds_ptr)l, 16, 0, 0);
}

static __device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// LDS byte address of a pointer into a __shared__ object
static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}

// s_waitcnt vmcnt(n) (n < 64; vmcnt is bits [3:0] and [15:14]), other counters untouched
#define QN_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8))

}  // namespace qn

#endif  // QN_MFMA_DEVICE_H
