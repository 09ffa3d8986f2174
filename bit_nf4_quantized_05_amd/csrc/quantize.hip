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
//   quant_blocks   - HBM-streaming pass over W (16 waves per workgroup, each with the
//                    next tile's loads in flight while it codes the current one):
//                    per 64-block absmax (8-lane DPP max), w / a by a per-block
//                    reciprocal and one correction, codes by a 32-cell threshold table
//                    in LDS, packed nibbles, the block constants, and an exact
//                    per-workgroup sum of the constants as 32-bit-limb integers.
//   dq_encode      - each workgroup first forms mu itself: it adds the per-workgroup
//                    limb sums (integers, so the order is free and every workgroup gets
//                    the same bits) and rounds their exact mean once to float32 (a float64
//                    estimate decides unless it is too close to a rounding midpoint, then
//                    integer long division); then, for its kDqGroups groups of 256
//                    constants: centre, absmax, INT8.
//   dequant_rows   - double dequantisation to bf16 (the standalone entry point; the
//                    linear calls dequantise inside their prologue launch).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "nf4_device.h"

#include <algorithm>

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
// 32-bit word of codes. Tiles are strided over the grid; a wave issues the loads of
// its next tile before coding the current one.
// ---------------------------------------------------------------------------
constexpr int kQuantThreads = 1024;

struct Tile8 { float v[8]; };

__device__ __forceinline__ Tile8 load_tile8(const float* __restrict__ W, int64_t n, int64_t e0) {
    Tile8 t;
    if (e0 + 8 <= n) {
        const float4 lo = *reinterpret_cast<const float4*>(W + e0);
        const float4 hi = *reinterpret_cast<const float4*>(W + e0 + 4);
        t.v[0] = lo.x; t.v[1] = lo.y; t.v[2] = lo.z; t.v[3] = lo.w;
        t.v[4] = hi.x; t.v[5] = hi.y; t.v[6] = hi.z; t.v[7] = hi.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) t.v[e] = (e0 + e < n) ? W[e0 + e] : 0.0f;
    }
    return t;
}

__global__ __launch_bounds__(kQuantThreads)
void quant_blocks(const float* __restrict__ W, int64_t n, int64_t n_b,
                  uint32_t* __restrict__ codes32, float* __restrict__ absmax,
                  unsigned long long* __restrict__ limb_part, NF4Tables tab) {
    __shared__ float2 s_cell[kCells];               // (threshold, base) of each cell: one 8-byte read
    __shared__ unsigned long long s_limb[kLimbs];
    const int tid = threadIdx.x;
    if (tid < kCells) s_cell[tid] = float2{tab.cell_thr[tid], __uint_as_float(tab.cell_base[tid])};
    if (tid < kLimbs) s_limb[tid] = 0ull;
    __syncthreads();

    constexpr int kWaves = kQuantThreads / 64;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t n_tiles = (n_b + 7) >> 3;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
    int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    Tile8 cur;
    if (t < n_tiles) cur = load_tile8(W, n, t * 512 + lane * 8);
    for (; t < n_tiles; t += stride) {
        Tile8 nxt;
        if (t + stride < n_tiles) nxt = load_tile8(W, n, (t + stride) * 512 + lane * 8);
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(cur.v[e]) & 0x7FFFFFFFu);
        m = max8(m);                         // exact absmax bits of the block
        const float a = __uint_as_float(m);
        // x = w / a. For 2^-96 <= a < 2^126: y = 1/a correctly rounded once per block,
        // q0 = w y, then one correction q0 + y (w - a q0) with the residual exact by
        // FMA, which yields the correctly rounded quotient wherever |x| is at least
        // ~1e-9 (Markstein); below that every x codes to 7 either way, since the
        // thresholds nearest zero are about +-0.04. Other blocks divide directly.
        const bool fast = m >= 0x0F800000u && m < 0x7E800000u;
        const float y = fast ? 1.0f / a : 0.0f;

        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x;
            if (fast) {
                const float q0 = cur.v[e] * y;
                const float r = __builtin_fmaf(-q0, a, cur.v[e]);
                x = __builtin_fmaf(r, y, q0);
            } else {
                x = (m == 0) ? 0.0f : cur.v[e] / a;   // IEEE division, |x| <= 1
            }
            const int cell = min(max(static_cast<int>((x + 1.0f) * 16.0f), 0), kCells - 1);
            const float2 cl = s_cell[cell];
            const uint32_t c = __float_as_uint(cl.y) + (x > cl.x ? 1u : 0u);
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
        cur = nxt;
    }
    __syncthreads();
    // limb-major: limb L of workgroup g at limb_part[L * gridDim.x + g]
    if (tid < kLimbs) limb_part[static_cast<int64_t>(tid) * gridDim.x + blockIdx.x] = s_limb[tid];
}

// ---------------------------------------------------------------------------
// mu = RoundNearestEven_f32( (sum_j a_j) / n_b ), exact. The sum is an integer S
// in units of 2^-149 given as per-limb column totals colsum[L] (limb L weighs
// 2^(32 L)); each column total is < n_b * 2^32 < 2^64. Every limb array below is
// indexed by compile-time constants only (fully unrolled), so it stays in registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float mean_from_limbs(const unsigned long long* colsum, int64_t n_b) {
    // carry-normalise to 32-bit limbs (each column total is < n_b * 2^32 < 2^64)
    constexpr int kQ = kLimbs + 1;
    uint32_t N[kQ];
    unsigned long long carry = 0ull;
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) {
        const unsigned long long col = colsum[L];
        const unsigned long long low = (col & 0xFFFFFFFFull) + (carry & 0xFFFFFFFFull);
        N[L] = static_cast<uint32_t>(low);
        carry = (col >> 32) + (carry >> 32) + (low >> 32);
    }
    N[kLimbs] = static_cast<uint32_t>(carry);

    // Q = floor(S / n_b), rem = S mod n_b (n_b < 2^32)
    const unsigned long long d = static_cast<unsigned long long>(n_b);
    uint32_t Q[kQ];
    unsigned long long rem = 0ull;
#pragma unroll
    for (int L = kQ - 1; L >= 0; --L) {
        const unsigned long long cur = (rem << 32) | N[L];
        Q[L] = static_cast<uint32_t>(cur / d);
        rem = cur % d;
    }
    // 96-bit window of Q holding its top limb, and whether anything lies below it
    int top = -1;
#pragma unroll
    for (int L = 0; L < kQ; ++L)
        if (Q[L]) top = L;
    uint32_t w2 = 0, w1 = 0, w0 = 0;
    bool below = false;
#pragma unroll
    for (int L = 0; L < kQ; ++L) {
        if (L == top) w2 = Q[L];
        else if (L == top - 1) w1 = Q[L];
        else if (L == top - 2) w0 = Q[L];
        else if (L < top - 2 && Q[L] != 0u) below = true;
    }
    uint32_t bits;
    const int len = top < 0 ? 0 : 32 * top + (32 - __clz(w2));   // bit length of Q
    if (len >= 24) {
        // left-align the window: bit (len-1) of Q moves to bit 95
        const int lz = __clz(w2);
        const unsigned long long hi = ((static_cast<unsigned long long>(w2) << 32) | w1) << lz |
                                      (lz ? (static_cast<unsigned long long>(w0) >> (32 - lz)) : 0ull);
        const uint32_t lo32 = lz ? (w0 << lz) : w0;   // remaining low bits of the window
        uint32_t mant = static_cast<uint32_t>(hi >> 40);               // top 24 bits
        const bool guard = (hi >> 39) & 1ull;
        const bool sticky = (hi & ((1ull << 39) - 1ull)) != 0ull || lo32 != 0u || below || rem != 0ull;
        int shift = len - 24;                                            // value = mant * 2^(shift-149)
        if (guard && (sticky || (mant & 1u))) {
            if (++mant == (1u << 24)) { mant >>= 1; ++shift; }
        }
        bits = (static_cast<uint32_t>(shift + 1) << 23) | (mant & 0x7FFFFFu);
    } else {   // below 2^-126: fixed 2^-149 grid, Q fits in one limb
        uint32_t mant = Q[0];
        if ((2ull * rem > d) || (2ull * rem == d && (mant & 1u))) ++mant;
        bits = mant;
    }
    return __uint_as_float(bits);
}

// The same mu, usually without the long division: the column totals summed in float64
// (each limb scaled by its power of two) and divided by n_b give the exact mean within
// a relative 20 * 2^-53 (19 roundings of positive terms, one division). Rounding that
// estimate to float32 gives the float nearest the exact mean unless the estimate lies
// within x 2^-46 of a midpoint between neighbouring floats (sums of two adjacent floats
// are exact in float64); only then does the integer division above decide.
__device__ __forceinline__ float mean_of_columns(const unsigned long long* colsum, int64_t n_b) {
    double s = 0.0;
#pragma unroll
    for (int L = kLimbs - 1; L >= 0; --L) s += ldexp(static_cast<double>(colsum[L]), 32 * L - 149);
    const double x = s / static_cast<double>(n_b);
    const float f = static_cast<float>(x);
    const uint32_t fb = __float_as_uint(f);
    const double up = (static_cast<double>(f) + static_cast<double>(__uint_as_float(fb + 1u))) * 0.5;
    const double dn = fb ? (static_cast<double>(f) + static_cast<double>(__uint_as_float(fb - 1u))) * 0.5 : -1.0;
    const double tol = x * 0x1p-46;
    if (up - x > tol && x - dn > tol) return f;
    return mean_from_limbs(colsum, n_b);
}


// ---------------------------------------------------------------------------
// Level 2. A workgroup of 1024 threads forms mu (waves 0..9 add one limb column
// each over the quant_blocks workgroups; one thread then divides), then encodes
// `passes` consecutive spans of kDqGroups groups of 256 block constants, one group
// per 4 waves. mu is the serial part of a workgroup, so a large weight gives each
// workgroup several spans (their constants are loaded before mu is formed).
// ---------------------------------------------------------------------------
constexpr int kDqThreads = 1024;
constexpr int kDqGroups = kDqThreads / kGroup;
constexpr int kDqMaxPasses = 16;
constexpr int kLimbBatch = 4;

__global__ __launch_bounds__(kDqThreads)
void dq_encode(const float* __restrict__ absmax, int64_t n_b, const unsigned long long* __restrict__ limb_part,
               int parts, int passes, int fmt, float* __restrict__ qmean, int8_t* __restrict__ qconst,
               float* __restrict__ qscale) {
    __shared__ unsigned long long s_col[kLimbs];
    __shared__ float s_mu;
    __shared__ uint32_t s_max[2][kDqThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * passes * kDqThreads + tid;
    float av[kDqMaxPasses];
#pragma unroll
    for (int p = 0; p < kDqMaxPasses; ++p) {
        const int64_t j = j0 + static_cast<int64_t>(p) * kDqThreads;
        av[p] = p < passes && j < n_b ? absmax[j] : 0.0f;
    }
    if (wave < kLimbs) {
        unsigned long long acc = 0ull;
        const unsigned long long* colp = limb_part + static_cast<int64_t>(wave) * parts;
        for (int g0 = 0; g0 < parts; g0 += 64 * kLimbBatch) {   // kLimbBatch loads in flight per lane
            unsigned long long v[kLimbBatch];
#pragma unroll
            for (int b = 0; b < kLimbBatch; ++b) v[b] = colp[min(g0 + 64 * b + lane, parts - 1)];
#pragma unroll
            for (int b = 0; b < kLimbBatch; ++b) acc += g0 + 64 * b + lane < parts ? v[b] : 0ull;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc & 0xFFFFFFFFull), off));
            const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc >> 32), off));
            acc += (static_cast<unsigned long long>(hi) << 32) | lo;
        }
        if (lane == 0) s_col[wave] = acc;
    }
    __syncthreads();
    if (tid == 0) {
        unsigned long long col[kLimbs];
#pragma unroll
        for (int L = 0; L < kLimbs; ++L) col[L] = s_col[L];
        s_mu = mean_of_columns(col, n_b);
        if (blockIdx.x == 0) qmean[0] = s_mu;
    }
    __syncthreads();
    const float mu = s_mu;
    const int g0 = (wave >> 2) << 2;             // the 4 waves of this thread's group
#pragma unroll
    for (int p = 0; p < kDqMaxPasses; ++p) {
        if (p >= passes) break;
        const int64_t j = j0 + static_cast<int64_t>(p) * kDqThreads;
        const bool valid = j < n_b;
        const float d = valid ? av[p] - mu : 0.0f;
        uint32_t m = __float_as_uint(d) & 0x7FFFFFFFu;
        m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32)));
        m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16)));
        m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 8)));
        m = max8(m);
        // s_max alternates between two buffers, so one barrier per span suffices
        if (lane == 0) s_max[p & 1][wave] = m;
        __syncthreads();
        const uint32_t* sm = s_max[p & 1];
        const uint32_t mb = max(max(sm[g0], sm[g0 + 1]), max(sm[g0 + 2], sm[g0 + 3]));
        const float b = __uint_as_float(mb);
        if (valid) {
            int8_t q = 0;
            if (mb != 0) {
                const float r = d / b;                              // in [-1, 1]
                if (fmt == kDqFp8)
                    q = static_cast<int8_t>(e4m3_encode(r * static_cast<float>(kE4m3Max)));
                else
                    q = static_cast<int8_t>(static_cast<int>(rintf(r * static_cast<float>(kInt8Step))));
            }
            qconst[j] = q;
        }
        const int64_t grp = (j0 - tid) / kGroup + static_cast<int64_t>(p) * kDqGroups + (wave >> 2);
        if ((tid & (kGroup - 1)) == 0 && grp * kGroup < n_b) qscale[grp] = b;
    }
}

// ---------------------------------------------------------------------------
// Dequantisation, row-major: one thread per 8 consecutive weights.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads)
void dequant_rows(const uint32_t* __restrict__ codes32, BlockConsts bc, int64_t n,
                  uint16_t* __restrict__ out, NF4Tables tab) {
    __shared__ float s_code[16];
    if (threadIdx.x < 16) s_code[threadIdx.x] = tab.code[threadIdx.x];
    __syncthreads();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t e0 = t * 8;
    if (e0 >= n) return;
    const int64_t blk = t >> 3;
    const float ahat = block_constant(bc.fmt, bc.q[blk], bc.scale[blk >> bc.gshift], bc.mean[0]);
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

}  // namespace

int quant_grid(int64_t n_b) {
    // one 16-wave workgroup per CU, fewer for small inputs (one tile per wave at least)
    const int64_t tiles = (n_b + 7) / 8;
    const int64_t want = (tiles + 15) / 16;
    return static_cast<int>(want < 256 ? (want < 1 ? 1 : want) : 256);
}

hipError_t launch_quantize(const float* W, int64_t n, int64_t n_b, int64_t n_g, int fmt,
                           uint8_t* codes, int8_t* qconst, float* qscale, float* qmean,
                           float* ws_absmax, unsigned long long* ws_limbs, int grid,
                           hipStream_t st) {
    const NF4Tables& tab = tables();
    // with no second level the block constants are the output itself
    float* absmax = fmt == kDqNone ? qscale : ws_absmax;
    QN_LAUNCH("quant_blocks", st, quant_blocks, dim3(grid), dim3(kQuantThreads), 0, st, W, n, n_b,
              reinterpret_cast<uint32_t*>(codes), absmax, ws_limbs, tab);
    if (fmt != kDqNone) {
        // spans of kDqGroups groups: about 256 workgroups, at most kDqMaxPasses spans each
        const int64_t spans = (n_g + kDqGroups - 1) / kDqGroups;
        const int passes = static_cast<int>(std::min<int64_t>(kDqMaxPasses, std::max<int64_t>(1, spans / 256)));
        const int64_t dq_grid = (spans + passes - 1) / passes;
        QN_LAUNCH("dq_encode", st, dq_encode, dim3(static_cast<unsigned>(dq_grid)), dim3(kDqThreads), 0, st,
                  ws_absmax, n_b, ws_limbs, grid, passes, fmt, qmean, qconst, qscale);
    }
    return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* codes, const BlockConsts& bc, int64_t n, uint16_t* out,
                               hipStream_t st) {
    const int64_t threads = (n + 7) / 8;
    const int64_t grid = (threads + kThreads - 1) / kThreads;
    QN_LAUNCH("dequant_rows", st, dequant_rows, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st,
                       reinterpret_cast<const uint32_t*>(codes), bc, n, out, tables());
    return hipGetLastError();
}

}  // namespace qn
