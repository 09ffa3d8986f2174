// 8-bit block quantisation for the low-rank factors of the W ~ Q + L R form.
//
// gist.science "Sintesi Tecnica: GPTQ-intrinsic LoRA" ("Risultati Chiave", "Empirici")
// keeps the factors L and R at 4 or 8 bits. The 4-bit factor uses the NF4 quantiser
// without a second level; the 8-bit one is symmetric absmax INT8 per block of 64 flat
// elements (jjjymmm.cn "量化原理": scale by 127 / absmax and round):
//     a_j = max |w|,  q = round-half-even(fl32(fl32(w / a_j) * 127)),  q = 0 if a_j = 0,
//     w_hat = bf16(fl32(fl32(q / 127) * a_j)).
// Both kernels give a thread 8 consecutive elements, so 8 lanes hold one block and
// the block max is three cross-lane max steps. Factors are small (r x d_in, d_out x r),
// so these kernels are simple rather than tuned.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "nf4_device.h"

namespace qn {
namespace {

constexpr int kFThreads = 256;

__global__ __launch_bounds__(kFThreads)
void int8_quant_blocks(const float* __restrict__ W, int64_t n, int8_t* __restrict__ q, float* __restrict__ absmax) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x;
    const int64_t e0 = t * 8;
    const int64_t n_pad = (n + 63) / 64 * 64;
    // every lane of a live block takes part in the max, so whole groups of 8 stay together
    const bool live = e0 < n_pad;
    float w[8];
    if (live && e0 + 8 <= n) {                      // 32-byte aligned: W is 16-byte aligned, e0 % 8 == 0
        const float4 lo = *reinterpret_cast<const float4*>(W + e0);
        const float4 hi = *reinterpret_cast<const float4*>(W + e0 + 4);
        w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
        w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = live && e0 + e < n ? W[e0 + e] : 0.0f;   // +0.0 padding
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(w[e]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    if (!live) return;
    uint32_t packed[2] = {0u, 0u};
    if (m > 0.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = w[e] / m;
            const int v = static_cast<int>(rintf(x * static_cast<float>(kInt8Step)));
            packed[e >> 2] |= (static_cast<uint32_t>(v) & 0xFFu) << (8 * (e & 3));
        }
    }
    *reinterpret_cast<uint2*>(q + e0) = uint2{packed[0], packed[1]};
    if ((threadIdx.x & 7) == 0) absmax[e0 >> 6] = m;
}

__global__ __launch_bounds__(kFThreads)
void int8_dequant_rows(const int8_t* __restrict__ q, const float* __restrict__ absmax, int64_t n,
                       uint16_t* __restrict__ out) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x;
    const int64_t e0 = t * 8;
    if (e0 >= n) return;
    const uint2 v = *reinterpret_cast<const uint2*>(q + e0);
    const float a = absmax[e0 >> 6];
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int8_t qe = static_cast<int8_t>(((e < 4 ? v.x : v.y) >> (8 * (e & 3))) & 0xFFu);
        const float rhat = static_cast<float>(qe) / static_cast<float>(kInt8Step);
        w[e] = rhat * a;
    }
    if (e0 + 8 <= n) {                              // out + e0 is 16-byte aligned
        *reinterpret_cast<uint4*>(out + e0) = uint4{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                                                   pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
    } else {
        for (int e = 0; e < 8 && e0 + e < n; ++e) out[e0 + e] = bf16_bits(w[e]);
    }
}

}  // namespace

hipError_t launch_int8_quantize(const float* W, int64_t n, int8_t* q, float* absmax, hipStream_t st) {
    const int64_t threads = (n + 63) / 64 * 8;
    const int64_t grid = (threads + kFThreads - 1) / kFThreads;
    QN_LAUNCH("int8_quant_blocks", st, int8_quant_blocks, dim3(static_cast<unsigned>(grid)), dim3(kFThreads), 0, st,
              W, n, q, absmax);
    return hipGetLastError();
}

hipError_t launch_int8_dequant(const int8_t* q, const float* absmax, int64_t n, uint16_t* out, hipStream_t st) {
    const int64_t threads = (n + 7) / 8;
    const int64_t grid = (threads + kFThreads - 1) / kFThreads;
    QN_LAUNCH("int8_dequant_rows", st, int8_dequant_rows, dim3(static_cast<unsigned>(grid)), dim3(kFThreads), 0, st,
              q, absmax, n, out);
    return hipGetLastError();
}

}  // namespace qn
