// Measurement aids (libqn_calibrate.so, declared in include/qn_calibrate.h): plain
// streaming reads that set the floor a kernel of the layer is measured against. They
// compute nothing of the layer; each folds what it reads into one XOR word so the
// loads cannot be removed.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/qn_calibrate.h"

namespace {

constexpr int kRows = 16;          // rows per workgroup, one per wave (as the decode GEMV)
constexpr int kSeg = 4096;         // weights per row segment

// The decode GEMV's loads without its arithmetic: wave w of workgroup g reads row
// 16 g + w; per 4096-weight segment, lane l reads the 16-byte code words l and 64 + l
// and block l's 8-bit constant and group scale (as the GEMV's lanes do), all loads of a
// segment in flight before any is used.
__global__ __launch_bounds__(1024)
void code_stream_kernel(const uint4* __restrict__ codes, const int8_t* __restrict__ qconst,
                        const float* __restrict__ qscale, int d_out, int d_in, uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = min(static_cast<int>(blockIdx.x) * kRows + wave, d_out - 1);
    const int nbpr = d_in / 64;
    const int64_t row_u = static_cast<int64_t>(row) * (d_in / 32);
    uint32_t v = 0;
    for (int s = 0; s * kSeg < d_in; ++s) {
        const int c0 = s * kSeg + lane * 32, c1 = c0 + 2048;
        const int64_t b = static_cast<int64_t>(row) * nbpr + min(s * 64 + lane, nbpr - 1);
        const uint4 a = codes[row_u + (c0 < d_in ? c0 / 32 : 0)];
        const uint4 e = codes[row_u + (c1 < d_in ? c1 / 32 : 0)];
        const int8_t q = qconst[b];
        const float sc = qscale[b >> 8];
        v ^= a.x ^ a.y ^ a.z ^ a.w ^ e.x ^ e.y ^ e.z ^ e.w ^ static_cast<uint32_t>(q) ^ __float_as_uint(sc);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off);
    if (lane == 0 && static_cast<int>(blockIdx.x) * kRows + wave < d_out) out[static_cast<int64_t>(blockIdx.x) * kRows + wave] = v;
}

// A plain read of n16 16-byte pieces: thread t of the grid reads pieces t + k G
// (G = grid threads), kUnroll of them in flight at a time.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256)
void read_kernel(const uint4* __restrict__ src, int64_t n16, uint32_t* __restrict__ out) {
    const int64_t G = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t v = 0;
    for (int64_t i = t; i < n16; i += kUnroll * G) {
        uint4 r[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) r[k] = src[min(i + k * G, n16 - 1)];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) v ^= r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

extern "C" {

int qn_calibrate_code_stream(const uint8_t* codes, const int8_t* qconst, const float* qscale, int64_t d_out,
                             int64_t d_in, uint32_t* out, void* stream) {
    if (!codes || !qconst || !qscale || !out) return -1;
    if (d_out < 1 || d_in < 64 || d_in % 64 != 0 || d_out > INT32_MAX / kRows || d_in > INT32_MAX / 2) return -1;
    if ((reinterpret_cast<uintptr_t>(codes) & 15) || (reinterpret_cast<uintptr_t>(qscale) & 3)) return -1;
    hipLaunchKernelGGL(code_stream_kernel, dim3(static_cast<unsigned>((d_out + kRows - 1) / kRows)), dim3(64 * kRows),
                       0, static_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(codes), qconst, qscale,
                       static_cast<int>(d_out), static_cast<int>(d_in), out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int qn_calibrate_read(const void* src, int64_t bytes, int grid, uint32_t* out, void* stream) {
    if (!src || !out || bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > 65536) return -1;
    if (reinterpret_cast<uintptr_t>(src) & 15) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(src), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
