// BF16 MFMA contractions of the QLoRA linear layer on gfx950.
//
// Forward (whoami-wesleyyou.top "LoRA": Y = W0 X + s B (A X)) and input gradient
// (learn.ifs.name deck card 1: gradients flow through the dequantised BF16 weights)
// are both written as an "NT" product of two K-contiguous operands,
//     C[M, N] = P[M, K] Q[N, K]^T  (+ P2[M, K2] Q2[N, K2]^T),
// with M = tokens. The rank-r LoRA branch is the second term, folded in as extra
// K-steps of the same accumulators:
//     forward : P = X,  Q = W_hat,    P2 = s (X A^T),   Q2 = B
//     dX      : P = dY, Q = W_hat^T,  P2 = s (dY B),    Q2 = A^T
// so it costs r extra K (1.6 % of the flops at r = 64, K = 4096).
//
// gemm_nt: 256x256 output tile per workgroup, 4 waves in a 2x2 grid, each wave a
// 128x128 sub-tile of 4x4 v_mfma_f32_32x32x16_bf16 accumulators (fp32). K-steps of
// 64 are double-buffered in LDS (2 x 64 KB); rows of 128 B are stored with their
// eight 16-byte chunks XOR-swizzled by (row & 7) so that the 32-row fragment reads
// (ds_read_b128) hit every bank once. Tiles are handed to the 8 XCDs in contiguous
// ranges so each XCD's L2 sees a compact block of P and Q panels.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace qn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

typedef const __attribute__((address_space(1))) void* global_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from global memory straight into LDS: lane i's data lands at
// byte 16*i after the wave-uniform LDS address `l`.
__device__ __forceinline__ void load_lds16(const void* g, void* l) {
    __builtin_amdgcn_global_load_lds((global_ptr)g, (lds_ptr)l, 16, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// ---------------------------------------------------------------------------
// Main NT GEMM
// ---------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGT = 256;                       // threads
constexpr int kChunks = BM * BK / 8;           // 16-byte chunks per operand tile (2048)
constexpr int kGroupM = 4;                     // tile rows per raster group

// Two LDS stages as two distinct objects, so the compiler can tell that reads of
// one stage do not depend on the in-flight direct-to-LDS loads into the other.
// Each holds [P tile | Q tile], 2 x 2048 chunks = 64 KB.
__shared__ uint4 g_stage0[2 * kChunks];
__shared__ uint4 g_stage1[2 * kChunks];

// Scheduling hints: interleave `n` groups of (1 LDS read, 2 MFMA).
#define QN_INTERLEAVE_DS_MFMA(n)                                  \
    _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {          \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);        \
    }

struct GemmArgs {
    const uint16_t* P; int64_t ldp;
    const uint16_t* Q; int64_t ldq; int kt1;
    const uint16_t* P2; int64_t ldp2;
    const uint16_t* Q2; int64_t ldq2; int kt2;
    uint16_t* C; int64_t ldc; int M, N, tiles_m, tiles_n;
};

// Issue the direct-to-LDS loads of K-step kt into `stage` (64 rows per wave, both
// operands). Offsets are 32-bit per lane on a wave-uniform base pointer.
__device__ __forceinline__ void gemm_issue(const GemmArgs& g, int kt, uint4* stage, int wave,
                                           const uint32_t* rowP, const uint32_t* rowQ, uint32_t kc16) {
    const bool main = kt < g.kt1;
    const int64_t kb = static_cast<int64_t>(main ? kt : kt - g.kt1) * (BK * 2);
    const char* bp = reinterpret_cast<const char*>(main ? g.P : g.P2) + kb;
    const char* bq = reinterpret_cast<const char*>(main ? g.Q : g.Q2) + kb;
    const uint32_t lp = static_cast<uint32_t>((main ? g.ldp : g.ldp2) * 2);
    const uint32_t lq = static_cast<uint32_t>((main ? g.ldq : g.ldq2) * 2);
    uint4* sp = stage + wave * 512;
    uint4* sq = sp + kChunks;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        load_lds16(bp + (rowP[j] * lp + kc16), sp + 64 * j);
        load_lds16(bq + (rowQ[j] * lq + kc16), sq + 64 * j);
    }
}

// fragments of k16 sub-step kk: f[0..3] = P (m sub-tiles), f[4..7] = Q (n sub-tiles)
__device__ __forceinline__ void gemm_frags(const uint4* stage, uint32_t pidx, uint32_t qidx, uint4* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = stage[pidx + i * 256];
        f[4 + i] = stage[qidx + i * 256];
    }
}

__device__ __forceinline__ void gemm_mfmas(f32x16 (&acc)[4][4], const uint4* f) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(f[4 + a], f[b], acc[a][b]);
}

__global__ __launch_bounds__(kGT, 1)
void gemm_nt_kernel(GemmArgs g) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = g.M, N = g.N;

    // ---- tile assignment: contiguous logical ranges per XCD, grouped raster
    const int T = g.tiles_m * g.tiles_n;
    const int w = blockIdx.x;
    const int logical = (T % 8 == 0) ? (w & 7) * (T >> 3) + (w >> 3) : w;
    const int gsize = kGroupM * g.tiles_n;
    const int grp = logical / gsize;
    const int first_m = grp * kGroupM;
    const int gm = min(g.tiles_m - first_m, kGroupM);
    const int tm = first_m + (logical % gsize) % gm;
    const int tn = (logical % gsize) / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- global -> LDS: direct 16-byte loads into LDS (global_load_lds_dwordx4).
    // One instruction fills a 1 KB LDS segment = 8 rows x 8 chunks; lane i lands at
    // chunk i of the segment, i.e. row i/8, stored chunk i%8, so it fetches the
    // global chunk (i%8) ^ (row & 7) = (i%8) ^ (i/8) of that row (XOR swizzle).
    // Wave w fills rows 64w .. 64w+63 of both operand tiles.
    const uint32_t kc16 = static_cast<uint32_t>((lane & 7) ^ (lane >> 3)) * 16u;
    uint32_t rowP[8], rowQ[8];                  // clamped rows (ragged M / N tiles)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        rowP[j] = static_cast<uint32_t>(min(m0 + 64 * wave + 8 * j + (lane >> 3), M - 1));
        rowQ[j] = static_cast<uint32_t>(min(n0 + 64 * wave + 8 * j + (lane >> 3), N - 1));
    }
    const int KT = g.kt1 + g.kt2;

    // fragment read indices (in 16-byte chunks) per k16 sub-step
    const uint32_t frow = lane & 31;
    const uint32_t fsw = lane & 7;
    const uint32_t prow = (wm * 128 + frow) * 8;
    const uint32_t qrow = kChunks + (wn * 128 + frow) * 8;
    uint32_t ch[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ch[kk] = (2 * kk + (lane >> 5)) ^ fsw;

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    uint4 fa[8], fb[8];
    gemm_issue(g, 0, g_stage0, wave, rowP, rowQ, kc16);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    gemm_frags(g_stage0, prow + ch[0], qrow + ch[0], fa);

    // One K-step on stage CUR while stage NXT receives step kt+1. Enters with the
    // kk = 0 fragments of CUR in fa, leaves with the kk = 0 fragments of NXT in fa.
#define QN_STEP(KTV, CUR, NXT)                                                  \
    {                                                                           \
        const int kt_ = (KTV);                                                  \
        const bool more_ = kt_ + 1 < KT;                                        \
        if (more_) gemm_issue(g, kt_ + 1, NXT, wave, rowP, rowQ, kc16);         \
        gemm_frags(CUR, prow + ch[1], qrow + ch[1], fb);                        \
        gemm_mfmas(acc, fa);                                                    \
        QN_INTERLEAVE_DS_MFMA(8);                                               \
        gemm_frags(CUR, prow + ch[2], qrow + ch[2], fa);                        \
        gemm_mfmas(acc, fb);                                                    \
        QN_INTERLEAVE_DS_MFMA(8);                                               \
        gemm_frags(CUR, prow + ch[3], qrow + ch[3], fb);                        \
        gemm_mfmas(acc, fa);                                                    \
        QN_INTERLEAVE_DS_MFMA(8);                                               \
        __builtin_amdgcn_s_waitcnt(0);                                          \
        __syncthreads();                                                        \
        if (more_) gemm_frags(NXT, prow + ch[0], qrow + ch[0], fa);             \
        gemm_mfmas(acc, fb);                                                    \
        QN_INTERLEAVE_DS_MFMA(8);                                               \
    }

    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        QN_STEP(kt, g_stage0, g_stage1)
        QN_STEP(kt + 1, g_stage1, g_stage0)
    }
    if (kt < KT) QN_STEP(kt, g_stage0, g_stage1)
#undef QN_STEP

    // ---- epilogue: lane holds C[m][n..n+3] for 4 groups per accumulator
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = m0 + wm * 128 + b * 32 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int n = n0 + wn * 128 + a * 32 + 8 * gq + 4 * (lane >> 5);
                if (n < N) {
                    uint2 o;
                    o.x = pack_bf16x2(acc[a][b][4 * gq + 0], acc[a][b][4 * gq + 1]);
                    o.y = pack_bf16x2(acc[a][b][4 * gq + 2], acc[a][b][4 * gq + 3]);
                    *reinterpret_cast<uint2*>(g.C + static_cast<int64_t>(m) * g.ldc + n) = o;
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// LoRA pre-pass: OUT[M, r_pad] = bf16(s * P[M, K] R[r, K]^T). One workgroup per
// 32 rows of P; the four waves take quarters of K and are summed through LDS.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256)
void lora_prepass_kernel(const uint16_t* __restrict__ P, int64_t ldp, int M, int K,
                         const uint16_t* __restrict__ R, int64_t ldr, int r, float s,
                         uint16_t* __restrict__ OUT, int r_pad) {
    __shared__ f32x16 red[2][NT][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = blockIdx.x * 32;
    const int64_t rowm = min(m0 + (lane & 31), M - 1);
    const int nchunk = K / 64;                 // whole 64-wide K chunks, split over 4 waves
    const int kbeg = (wave * nchunk / 4) * 64;
    const int kend = ((wave + 1) * nchunk / 4) * 64;
    const int ksub = 8 * (lane >> 5);
    const uint16_t* prow = P + rowm * ldp + ksub;
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    const uint16_t* rrow[NT];
    bool rok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int rr = t * 32 + (lane & 31);
        rok[t] = rr < r;
        rrow[t] = R + static_cast<int64_t>(rok[t] ? rr : 0) * ldr + ksub;
    }
    for (int k = kbeg; k < kend; k += 64) {
        uint4 pf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) pf[u] = *reinterpret_cast<const uint4*>(prow + k + 16 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint4 rf = *reinterpret_cast<const uint4*>(rrow[t] + k + 16 * u);
                if (!rok[t]) rf = uint4{0, 0, 0, 0};
                acc[t] = mfma32(rf, pf[u], acc[t]);
            }
        }
    }
    // sum the four K-quarters: waves 2,3 -> 0,1, then 1 -> 0
    if (wave >= 2)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[wave - 2][t][lane] = acc[t];
    __syncthreads();
    if (wave < 2)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] += red[wave][t][lane];
    __syncthreads();
    if (wave == 1)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[0][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
    const int m = m0 + (lane & 31);
    if (m >= M) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const f32x16 v = acc[t] + red[0][t][lane];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int n = t * 32 + 8 * gq + 4 * (lane >> 5);
            if (n < r_pad) {
                uint2 o;
                o.x = pack_bf16x2(s * v[4 * gq + 0], s * v[4 * gq + 1]);
                o.y = pack_bf16x2(s * v[4 * gq + 2], s * v[4 * gq + 3]);
                *reinterpret_cast<uint2*>(OUT + static_cast<int64_t>(m) * r_pad + n) = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small layout helpers for the adapter matrices.
// ---------------------------------------------------------------------------
__global__ void transpose_pad_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                     uint16_t* __restrict__ dst, int64_t ld_dst) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= cols * ld_dst) return;
    const int64_t j = idx / ld_dst, i = idx % ld_dst;
    dst[idx] = i < rows ? src[i * cols + j] : static_cast<uint16_t>(0);
}

__global__ void pad_cols_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                uint16_t* __restrict__ dst, int64_t ld_dst) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= rows * ld_dst) return;
    const int64_t i = idx / ld_dst, j = idx % ld_dst;
    dst[idx] = j < cols ? src[i * cols + j] : static_cast<uint16_t>(0);
}

// ---------------------------------------------------------------------------
// d_seq = 1: t = s (A x) in fp32, then a GEMV streaming the packed codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void lora_ax_kernel(const uint16_t* __restrict__ A, int d_in, const uint16_t* __restrict__ x,
                    float s, float* __restrict__ t) {
    __shared__ float red[4];
    const int k = blockIdx.x;
    float acc = 0.0f;
    for (int i = threadIdx.x * 8; i < d_in; i += 256 * 8) {
        const uint4 av = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(k) * d_in + i);
        const uint4 xv = *reinterpret_cast<const uint4*>(x + i);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += __uint_as_float(aw[e] << 16) * __uint_as_float(xw[e] << 16);
            acc += __uint_as_float(aw[e] & 0xFFFF0000u) * __uint_as_float(xw[e] & 0xFFFF0000u);
        }
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) t[k] = s * (red[0] + red[1] + red[2] + red[3]);
}

// One wave per row at a time; lane j takes blocks j, j+64, ... of the row. Per block
// the 32 code bytes are looked up as bf16 code pairs and dotted with bf16 x pairs
// (v_dot2_f32_bf16); the block constant a_hat multiplies the block's partial sum
// once (a per-block scale factors out of the sum over the block).
constexpr int kRowsPerWave = 4;

__global__ __launch_bounds__(256)
void gemv_nf4_kernel(const uint4* __restrict__ codes, const int8_t* __restrict__ qconst,
                     const float* __restrict__ qscale, const float* __restrict__ qmean,
                     int d_out, int d_in, const uint16_t* __restrict__ x,
                     const uint16_t* __restrict__ B, int r, const float* __restrict__ t,
                     uint16_t* __restrict__ y, NF4Tables tab) {
    __shared__ uint32_t lut2[256];
    __shared__ float qlut[256];
    __shared__ float s_t[256];
    const int tid = threadIdx.x;
    lut2[tid] = pack_bf16x2(tab.code[tid & 15], tab.code[tid >> 4]);
    qlut[tid] = static_cast<float>(tid - 128) / static_cast<float>(kInt8Step);
    if (tid < r) s_t[tid] = t[tid];
    __syncthreads();
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float mu = qmean[0];
    const int nbpr = d_in / 64;
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    const int rowbase = (blockIdx.x * 4 + wave) * kRowsPerWave;
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int o = rowbase + rr;
        if (o >= d_out) break;
        float acc = 0.0f;
        for (int jb = lane; jb < nbpr; jb += 64) {
            const int64_t blk = static_cast<int64_t>(o) * nbpr + jb;
            const uint4 c0 = codes[blk * 2];
            const uint4 c1 = codes[blk * 2 + 1];
            const float ahat = mu + qscale[blk >> 8] * qlut[qconst[blk] + 128];
            const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const uint4* xb = reinterpret_cast<const uint4*>(x32 + static_cast<int64_t>(jb) * 32);
            float part = 0.0f;
#pragma unroll
            for (int w4 = 0; w4 < 8; ++w4) {
                const uint4 xv = xb[w4];
                const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t byte = (cw[w4] >> (8 * b)) & 0xFFu;
                    part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lut2[byte]),
                                                           __builtin_bit_cast(bf16x2, xw[b]), part, false);
                }
            }
            acc += ahat * part;
        }
        for (int k = lane; k < r; k += 64) acc += bf16_to_f32(B[static_cast<int64_t>(o) * r + k]) * s_t[k];
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) y[o] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc));
    }
}

}  // namespace

hipError_t launch_gemm_nt(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, int64_t K1,
                          const uint16_t* P2, int64_t ldp2, const uint16_t* Q2, int64_t ldq2,
                          int64_t K2, uint16_t* C, int64_t ldc, int64_t M, int64_t N,
                          hipStream_t st) {
    GemmArgs g;
    g.tiles_m = static_cast<int>((M + BM - 1) / BM);
    g.tiles_n = static_cast<int>((N + BN - 1) / BN);
    if (P2 == nullptr) { P2 = P; Q2 = Q; ldp2 = ldp; ldq2 = ldq; K2 = 0; }
    g.P = P; g.ldp = ldp; g.Q = Q; g.ldq = ldq; g.kt1 = static_cast<int>(K1 / BK);
    g.P2 = P2; g.ldp2 = ldp2; g.Q2 = Q2; g.ldq2 = ldq2; g.kt2 = static_cast<int>(K2 / BK);
    g.C = C; g.ldc = ldc; g.M = static_cast<int>(M); g.N = static_cast<int>(N);
    QN_LAUNCH("gemm_nt_kernel", st, gemm_nt_kernel, dim3(g.tiles_m * g.tiles_n), dim3(kGT), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_lora_prepass(const uint16_t* P, int64_t ldp, int64_t M, int64_t K,
                               const uint16_t* R, int64_t ldr, int r, float s,
                               uint16_t* OUT, int r_pad, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((M + 31) / 32));
    const int Mi = static_cast<int>(M), Ki = static_cast<int>(K);
    switch (r_pad / 32) {
        case 2: QN_LAUNCH("lora_prepass_kernel", st, lora_prepass_kernel<2>, grid, dim3(256), 0, st, P, ldp, Mi, Ki, R, ldr, r, s, OUT, r_pad); break;
        case 4: QN_LAUNCH("lora_prepass_kernel", st, lora_prepass_kernel<4>, grid, dim3(256), 0, st, P, ldp, Mi, Ki, R, ldr, r, s, OUT, r_pad); break;
        case 6: QN_LAUNCH("lora_prepass_kernel", st, lora_prepass_kernel<6>, grid, dim3(256), 0, st, P, ldp, Mi, Ki, R, ldr, r, s, OUT, r_pad); break;
        case 8: QN_LAUNCH("lora_prepass_kernel", st, lora_prepass_kernel<8>, grid, dim3(256), 0, st, P, ldp, Mi, Ki, R, ldr, r, s, OUT, r_pad); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_transpose_pad(const uint16_t* src, int64_t rows, int64_t cols,
                                uint16_t* dst, int64_t ld_dst, hipStream_t st) {
    const int64_t total = cols * ld_dst;
    QN_LAUNCH("transpose_pad_kernel", st, transpose_pad_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st,
                       src, rows, cols, dst, ld_dst);
    return hipGetLastError();
}

hipError_t launch_pad_cols(const uint16_t* src, int64_t rows, int64_t cols,
                           uint16_t* dst, int64_t ld_dst, hipStream_t st) {
    const int64_t total = rows * ld_dst;
    QN_LAUNCH("pad_cols_kernel", st, pad_cols_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st,
                       src, rows, cols, dst, ld_dst);
    return hipGetLastError();
}

hipError_t launch_gemv_nf4(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                           const float* qmean, int64_t d_out, int64_t d_in,
                           const uint16_t* A, const uint16_t* B, int r, float s,
                           const uint16_t* x, uint16_t* y, float* ws_t, hipStream_t st) {
    QN_LAUNCH("lora_ax_kernel", st, lora_ax_kernel, dim3(r), dim3(256), 0, st, A, static_cast<int>(d_in), x, s, ws_t);
    const int64_t rows_per_wg = 4 * kRowsPerWave;
    const dim3 grid(static_cast<unsigned>((d_out + rows_per_wg - 1) / rows_per_wg));
    QN_LAUNCH("gemv_nf4_kernel", st, gemv_nf4_kernel, grid, dim3(256), 0, st, reinterpret_cast<const uint4*>(codes),
                       qconst, qscale, qmean, static_cast<int>(d_out), static_cast<int>(d_in), x, B, r,
                       ws_t, y, tables());
    return hipGetLastError();
}

}  // namespace qn
