// NF4 quantisation with Double Quantisation, and double dequantisation, for gfx950.
//
// Method (QLoRA pages): whoami-wesleyyou.top "LoRA 与 QLoRA" sections "归一化与匹配"
// (normalise a block by its absmax, match to the normalised quantiles) and
// "2. Double Quantization (DQ)" (r_j = (a_j - mu)/b, 8-bit r_hat, a_hat = mu + b r_hat);
// jjjymmm.cn 2024/03 "Double Quantization" (blocks of 64 weights, 8-bit constants in
// groups of 256 with one fp32 scale each) and "QLoRA" (dequantise the constants first,
// then the weights); learn.ifs.name QLoRA deck cards 1-4.
//
// Every float step that decides a stored bit is one IEEE float32 operation in the
// order written (this file is built with -ffp-contract=off and correctly rounded
// division), so the results are bit-identical to any faithful implementation.
//
// Kernels:
//   quant_blocks   - HBM-streaming pass over W: per 64-block absmax (8-lane DPP max),
//                    codes by a 32-cell threshold table in LDS, packed nibbles, the
//                    block constants, and an exact per-workgroup sum of the
//                    constants as 32-bit-limb integers (order-free).
//   mean_finalize  - one workgroup: adds the per-workgroup limb sums, divides by n_b
//                    with integer long division and rounds once to float32 -> mu.
//   dq_encode      - one workgroup per group of 256 constants: centre, absmax, INT8.
//   dequant_rows / dequant_transposed - double dequantisation to bf16, row-major or
//                    transposed through an LDS tile (for the input-gradient GEMM).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Max over each aligned group of 8 lanes (quad xor 1, quad xor 2, half-row mirror).
__device__ __forceinline__ uint32_t max8(uint32_t v) {
    v = max(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max(v, dpp_mov<0x141>(v));   // row_half_mirror
    return v;
}

// ---------------------------------------------------------------------------
// Level 1. A wave handles a tile of 8 blocks (512 floats): lane l owns floats
// [8l, 8l+8) of the tile, so 8 lanes share a block and each lane emits one
// 32-bit word of codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads)
void quant_blocks(const float* __restrict__ W, int64_t n, int64_t n_b,
                  uint32_t* __restrict__ codes32, float* __restrict__ absmax,
                  unsigned long long* __restrict__ limb_part, NF4Tables tab) {
    __shared__ float s_thr[kCells];
    __shared__ uint32_t s_base[kCells];
    __shared__ unsigned long long s_limb[kLimbs];
    const int tid = threadIdx.x;
    if (tid < kCells) {
        s_thr[tid] = tab.cell_thr[tid];
        s_base[tid] = tab.cell_base[tid];
    }
    if (tid < kLimbs) s_limb[tid] = 0ull;
    __syncthreads();

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t n_tiles = (n_b + 7) >> 3;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave; t < n_tiles; t += stride) {
        const int64_t e0 = t * 512 + lane * 8;
        float v[8];
        if (e0 + 8 <= n) {
            const float4 lo = *reinterpret_cast<const float4*>(W + e0);
            const float4 hi = *reinterpret_cast<const float4*>(W + e0 + 4);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (e0 + e < n) ? W[e0 + e] : 0.0f;
        }
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(v[e]) & 0x7FFFFFFFu);
        m = max8(m);                         // exact absmax bits of the block
        const float a = __uint_as_float(m);

        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = (m == 0) ? 0.0f : v[e] / a;       // IEEE division, |x| <= 1
            const int cell = min(max(static_cast<int>((x + 1.0f) * 16.0f), 0), kCells - 1);
            const uint32_t c = s_base[cell] + (x > s_thr[cell] ? 1u : 0u);
            packed |= c << (4 * e);
        }
        const int64_t blk = t * 8 + (lane >> 3);
        if (blk < n_b) {
            codes32[t * 64 + lane] = packed;
            if ((lane & 7) == 0) {
                absmax[blk] = a;
                // a = mant * 2^(p - 149) exactly; add mant << p into 32-bit limbs
                const uint32_t ex = m >> 23;
                const uint32_t mant = (m & 0x7FFFFFu) | (ex ? 0x800000u : 0u);
                const uint32_t p = (ex ? ex : 1u) - 1u;
                const unsigned long long wide = static_cast<unsigned long long>(mant) << (p & 31u);
                const uint32_t li = p >> 5;
                atomicAdd(&s_limb[li], wide & 0xFFFFFFFFull);
                if (wide >> 32) atomicAdd(&s_limb[li + 1], wide >> 32);
            }
        }
    }
    __syncthreads();
    if (tid < kLimbs) limb_part[static_cast<int64_t>(blockIdx.x) * kLimbs + tid] = s_limb[tid];
}

// ---------------------------------------------------------------------------
// mu = RoundNearestEven_f32( (sum_j a_j) / n_b ), exact.
// The sum is an integer S in units of 2^-149 held as 32-bit limbs.
// ---------------------------------------------------------------------------
__device__ inline bool bit_of(const uint32_t* q, int k) { return (q[k >> 5] >> (k & 31)) & 1u; }

__device__ inline bool any_below(const uint32_t* q, int k) {   // any of bits [0, k)
    for (int w = 0; w < (k >> 5); ++w)
        if (q[w]) return true;
    const int r = k & 31;
    return r ? (q[k >> 5] & ((1u << r) - 1u)) != 0u : false;
}

__global__ __launch_bounds__(kThreads)
void mean_finalize(const unsigned long long* __restrict__ limb_part, int parts, int64_t n_b,
                   float* __restrict__ qmean) {
    __shared__ unsigned long long s_sum[kThreads];
    const int tid = threadIdx.x;
    constexpr int kSlices = kThreads / kLimbs;   // 25
    unsigned long long acc = 0ull;
    if (tid < kSlices * kLimbs) {
        const int limb = tid % kLimbs;
        for (int g = tid / kLimbs; g < parts; g += kSlices) acc += limb_part[static_cast<int64_t>(g) * kLimbs + limb];
    }
    s_sum[tid] = acc;
    __syncthreads();
    if (tid != 0) return;

    // normalise to 32-bit limbs (the total of each limb column is < n_b * 2^32 < 2^64)
    constexpr int kQ = kLimbs + 1;
    uint32_t N[kQ];
    unsigned long long carry = 0ull;
    for (int L = 0; L < kLimbs; ++L) {
        unsigned long long col = 0ull;
        for (int sl = 0; sl < kSlices; ++sl) col += s_sum[sl * kLimbs + L];
        const unsigned long long low = (col & 0xFFFFFFFFull) + (carry & 0xFFFFFFFFull);
        N[L] = static_cast<uint32_t>(low);
        carry = (col >> 32) + (carry >> 32) + (low >> 32);
    }
    N[kLimbs] = static_cast<uint32_t>(carry);

    // long division by n_b (< 2^32)
    const unsigned long long d = static_cast<unsigned long long>(n_b);
    uint32_t Q[kQ];
    unsigned long long rem = 0ull;
    for (int L = kQ - 1; L >= 0; --L) {
        const unsigned long long cur = (rem << 32) | N[L];
        Q[L] = static_cast<uint32_t>(cur / d);
        rem = cur % d;
    }
    int len = 0;   // bit length of Q
    for (int L = kQ - 1; L >= 0; --L)
        if (Q[L]) { len = 32 * L + (32 - __clz(Q[L])); break; }

    uint32_t bits;
    if (len >= 24) {
        int shift = len - 24;
        uint32_t mant = 0;
        for (int k = 0; k < 24; ++k) mant |= static_cast<uint32_t>(bit_of(Q, shift + k)) << k;
        bool up;
        if (shift == 0) {
            up = (2ull * rem > d) || (2ull * rem == d && (mant & 1u));
        } else {
            const bool guard = bit_of(Q, shift - 1);
            const bool sticky = any_below(Q, shift - 1) || rem != 0ull;
            up = guard && (sticky || (mant & 1u));
        }
        if (up && ++mant == (1u << 24)) { mant >>= 1; ++shift; }
        bits = (static_cast<uint32_t>(shift + 1) << 23) | (mant & 0x7FFFFFu);
    } else {   // below 2^-126: fixed 2^-149 grid
        uint32_t mant = Q[0];
        if ((2ull * rem > d) || (2ull * rem == d && (mant & 1u))) ++mant;
        bits = mant;
    }
    qmean[0] = __uint_as_float(bits);
}

// ---------------------------------------------------------------------------
// Level 2: one workgroup per group of 256 block constants.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads)
void dq_encode(const float* __restrict__ absmax, int64_t n_b, const float* __restrict__ qmean,
               int8_t* __restrict__ qconst, float* __restrict__ qscale) {
    __shared__ uint32_t s_max[kThreads / 64];
    const int tid = threadIdx.x;
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kGroup + tid;
    const float mu = qmean[0];
    const bool valid = j < n_b;
    const float d = valid ? absmax[j] - mu : 0.0f;
    uint32_t m = __float_as_uint(d) & 0x7FFFFFFFu;
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32)));
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16)));
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 8)));
    m = max8(m);
    if ((tid & 63) == 0) s_max[tid >> 6] = m;
    __syncthreads();
    const uint32_t mb = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    const float b = __uint_as_float(mb);
    if (valid) {
        int8_t q = 0;
        if (mb != 0) {
            const float r = d / b;                                  // in [-1, 1]
            q = static_cast<int8_t>(static_cast<int>(rintf(r * static_cast<float>(kInt8Step))));
        }
        qconst[j] = q;
    }
    if (tid == 0) qscale[blockIdx.x] = b;
}

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

// ---------------------------------------------------------------------------
// Dequantisation, row-major: one thread per 8 consecutive weights.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads)
void dequant_rows(const uint32_t* __restrict__ codes32, const int8_t* __restrict__ qconst,
                  const float* __restrict__ qscale, const float* __restrict__ qmean, int64_t n,
                  uint16_t* __restrict__ out, NF4Tables tab) {
    __shared__ float s_code[16];
    if (threadIdx.x < 16) s_code[threadIdx.x] = tab.code[threadIdx.x];
    __syncthreads();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t e0 = t * 8;
    if (e0 >= n) return;
    const int64_t blk = t >> 3;
    const float ahat = block_constant(qconst[blk], qscale[blk / kGroup], qmean[0]);
    const uint32_t word = codes32[t];
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = s_code[(word >> (4 * e)) & 0xFu] * ahat;
    if (e0 + 8 <= n) {
        uint4 o;
        o.x = pack_bf16x2(w[0], w[1]);
        o.y = pack_bf16x2(w[2], w[3]);
        o.z = pack_bf16x2(w[4], w[5]);
        o.w = pack_bf16x2(w[6], w[7]);
        *reinterpret_cast<uint4*>(out + e0) = o;
    } else {
        for (int e = 0; e < 8 && e0 + e < n; ++e)
            out[e0 + e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(w[e]));
    }
}

// ---------------------------------------------------------------------------
// Transposed dequantisation: W_hat^T [d_in, d_out] through a 64x64 LDS tile.
// d_in % 64 == 0, so each tile row is exactly one block.
// ---------------------------------------------------------------------------
constexpr int kTP = 64 + 8;   // LDS pitch in bf16 (keeps 16-byte rows aligned)

__global__ __launch_bounds__(kThreads)
void dequant_transposed(const uint8_t* __restrict__ codes, const int8_t* __restrict__ qconst,
                        const float* __restrict__ qscale, const float* __restrict__ qmean,
                        int64_t d_out, int64_t d_in, uint16_t* __restrict__ outT, NF4Tables tab) {
    __shared__ float s_code[16];
    __shared__ uint16_t tile[64 * kTP];
    const int tid = threadIdx.x;
    if (tid < 16) s_code[tid] = tab.code[tid];
    __syncthreads();
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t o0 = static_cast<int64_t>(blockIdx.y) * 64;
    const int ol = tid >> 2;             // local row (output column of W_hat^T)
    const int q4 = tid & 3;              // which 16 of the 64 columns
    const int64_t o = o0 + ol;
    if (o < d_out) {
        const int64_t e0 = o * d_in + i0 + q4 * 16;
        const int64_t blk = e0 >> 6;
        const float ahat = block_constant(qconst[blk], qscale[blk / kGroup], qmean[0]);
        const uint2 cw = *reinterpret_cast<const uint2*>(codes + (e0 >> 1));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t word = e < 8 ? cw.x : cw.y;
            const float w = s_code[(word >> (4 * (e & 7))) & 0xFu] * ahat;
            tile[(q4 * 16 + e) * kTP + ol] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(w));
        }
    }
    __syncthreads();
    // row il of the output tile = 64 consecutive o values
    const int il = tid >> 2;
    const int seg = (tid & 3) * 16;
    const int64_t i = i0 + il;
    const int64_t oc = o0 + seg;
    if (oc < d_out) {
        const uint4* src = reinterpret_cast<const uint4*>(&tile[il * kTP + seg]);
        uint4* dst = reinterpret_cast<uint4*>(outT + i * d_out + oc);
        if (oc + 16 <= d_out) {
            dst[0] = src[0];
            dst[1] = src[1];
        } else {
            for (int e = 0; e < 16 && oc + e < d_out; ++e) outT[i * d_out + oc + e] = tile[il * kTP + seg + e];
        }
    }
}

}  // namespace

int quant_grid(int64_t n_b) {
    const int64_t tiles = (n_b + 7) / 8;
    const int64_t want = (tiles + 3) / 4;
    return static_cast<int>(want < 1024 ? (want < 1 ? 1 : want) : 1024);
}

hipError_t launch_quantize(const float* W, int64_t n, int64_t n_b, int64_t n_g,
                           uint8_t* codes, int8_t* qconst, float* qscale, float* qmean,
                           float* ws_absmax, unsigned long long* ws_limbs, int grid,
                           hipStream_t st) {
    const NF4Tables& tab = tables();
    QN_LAUNCH("quant_blocks", st, quant_blocks, dim3(grid), dim3(kThreads), 0, st, W, n, n_b,
                       reinterpret_cast<uint32_t*>(codes), ws_absmax, ws_limbs, tab);
    QN_LAUNCH("mean_finalize", st, mean_finalize, dim3(1), dim3(kThreads), 0, st, ws_limbs, grid, n_b, qmean);
    QN_LAUNCH("dq_encode", st, dq_encode, dim3(static_cast<unsigned>(n_g)), dim3(kThreads), 0, st,
                       ws_absmax, n_b, qmean, qconst, qscale);
    return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                               const float* qmean, int64_t n, uint16_t* out, hipStream_t st) {
    const int64_t threads = (n + 7) / 8;
    const int64_t grid = (threads + kThreads - 1) / kThreads;
    QN_LAUNCH("dequant_rows", st, dequant_rows, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st,
                       reinterpret_cast<const uint32_t*>(codes), qconst, qscale, qmean, n, out, tables());
    return hipGetLastError();
}

hipError_t launch_dequant_transposed(const uint8_t* codes, const int8_t* qconst,
                                     const float* qscale, const float* qmean, int64_t d_out,
                                     int64_t d_in, uint16_t* outT, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(d_in / 64), static_cast<unsigned>((d_out + 63) / 64));
    QN_LAUNCH("dequant_transposed", st, dequant_transposed, grid, dim3(kThreads), 0, st, codes, qconst, qscale,
                       qmean, d_out, d_in, outT, tables());
    return hipGetLastError();
}

}  // namespace qn
