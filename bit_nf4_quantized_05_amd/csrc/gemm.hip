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
// gemm_nt: 256x256 output tile per workgroup, 8 waves (two per SIMD, so one wave's
// MFMAs cover the other's waits) in a 2x4 grid, each wave a 128x64 sub-tile of 4x2
// v_mfma_f32_32x32x16_bf16 accumulators (fp32). K-steps of 64 are double-buffered
// in LDS (2 x 64 KB) and filled by buffer_load ... lds (direct to LDS, no staging
// registers): a tile row is then 128 B, one whole cache line per row and load, which
// halves the L2 requests per byte compared with 64-byte rows. Rows are stored with
// their 16-byte chunks XOR-swizzled by ((row >> 1) & 7), which makes the 32-row
// fragment reads (ds_read_b128) free of bank conflicts on the 64-bank LDS. The stage
// barrier sits before the last k16 sub-step, so the next stage's first fragments are
// read under the last MFMAs. Tiles are handed to the 8 XCDs in contiguous ranges so
// each XCD's L2 sees a compact block of P and Q panels.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "nf4_device.h"

#include <algorithm>

namespace qn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
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
constexpr int kChunks = BM * BK / 8;           // 16-byte chunks per operand tile (2048)
constexpr int kGroupM = 4;                     // tile rows per raster group

// Two LDS stages as distinct objects, so the compiler can tell that reads of one
// stage do not depend on in-flight direct-to-LDS loads into the other. Each holds
// [P tile | Q tile] = 2 x 2048 chunks = 64 KB.
__shared__ uint4 g_st0[2 * kChunks];
__shared__ uint4 g_st1[2 * kChunks];

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
    uint32_t bytesP, bytesQ, bytesP2, bytesQ2;   // buffer extents for the load descriptors
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// s_waitcnt vmcnt(n) (n < 64; vmcnt is bits [3:0] and [15:14]), other counters untouched
#define QN_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8))
// Workgroup barrier without the memory fence __syncthreads() adds (which would wait
// for every in-flight load, including the stages fetched ahead). The loads a barrier
// certifies are waited for explicitly with QN_WAIT_VM before it; LDS has no cache.
// The "memory" clobber keeps the compiler from moving memory accesses across it.
#define QN_BARRIER() asm volatile("s_barrier" ::: "memory")

// WM x WN waves; each wave owns a (256/WM) x (256/WN) sub-tile of 32x32 MFMA tiles.
template <int WM, int WN>
__device__ __forceinline__ void gemm_nt_body(const GemmArgs& g) {
    constexpr int NW = WM * WN;                 // waves
    constexpr int NT = 64 * NW;                 // threads
    constexpr int TM = BM / WM / 32;            // m sub-tiles per wave
    constexpr int TN = BN / WN / 32;            // n sub-tiles per wave
    constexpr int SEG = BM / NW / 8;            // 8-row load segments per wave and operand
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
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

    // ---- global -> LDS with buffer_load ... lds (16 B per lane). A tile row is 64
    // bf16 = 128 B = 8 chunks; chunk c of tile row r is stored at c ^ ((r >> 1) & 7).
    // The LDS has 64 banks of 4 B, so two consecutive rows cover all banks once, and
    // 16 lanes reading one logical chunk of 16 consecutive rows hit 16 distinct 4-bank
    // groups. One load fills a 1 KB segment = 8 rows: lane i lands at row i/8,
    // position i%8, so it fetches chunk (i%8) ^ ((r >> 1) & 7). Wave w fills rows
    // 8*SEG*w .. of both operand tiles; the per-lane byte offsets are fixed for the
    // whole K loop, the K position goes in the scalar offset.
    // 128-B rows, chunk c of row r at c ^ ((r >> 1) & 7); segment j = 8 rows starting
    // at 8 (SEG w + j): (r >> 1) & 7 = 4 ((SEG w + j) & 1) + i/16 for lane i.
    const uint32_t kcE = static_cast<uint32_t>((lane & 7) ^ (lane >> 4)) * 16u;
    const uint32_t kcO = static_cast<uint32_t>((lane & 7) ^ (4 | (lane >> 4))) * 16u;
    uint32_t voP[SEG], voQ[SEG], voP2[SEG], voQ2[SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        const int rr = 8 * SEG * wave + 8 * j + (lane >> 3);
        const uint32_t kc16 = (((SEG * wave + j) & 1) ? kcO : kcE);
        const uint32_t rp = static_cast<uint32_t>(min(m0 + rr, M - 1));
        const uint32_t rq = static_cast<uint32_t>(min(n0 + rr, N - 1));
        voP[j] = rp * static_cast<uint32_t>(g.ldp * 2) + kc16;
        voQ[j] = rq * static_cast<uint32_t>(g.ldq * 2) + kc16;
        voP2[j] = rp * static_cast<uint32_t>(g.ldp2 * 2) + kc16;
        voQ2[j] = rq * static_cast<uint32_t>(g.ldq2 * 2) + kc16;
    }
    const __amdgpu_buffer_rsrc_t rsP = make_rsrc(g.P, g.bytesP);
    const __amdgpu_buffer_rsrc_t rsQ = make_rsrc(g.Q, g.bytesQ);
    const __amdgpu_buffer_rsrc_t rsP2 = make_rsrc(g.P2, g.bytesP2);
    const __amdgpu_buffer_rsrc_t rsQ2 = make_rsrc(g.Q2, g.bytesQ2);
    const int KT = g.kt1 + g.kt2;
    constexpr int kLoadsPerStep = 2 * SEG;      // per wave

#define QN_ISSUE(KTV, ST)                                                                         \
    {                                                                                             \
        const int kk_ = (KTV);                                                                    \
        uint4* sp_ = (ST) + wave * (64 * SEG);                                                    \
        uint4* sq_ = sp_ + kChunks;                                                               \
        if (kk_ < g.kt1) {                                                                        \
            const int so_ = kk_ * (BK * 2);                                                       \
            _Pragma("unroll") for (int j = 0; j < SEG; ++j) {                                     \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP, (lds_ptr_t)(sp_ + 64 * j), 16, voP[j], so_, 0, 0); \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQ, (lds_ptr_t)(sq_ + 64 * j), 16, voQ[j], so_, 0, 0); \
            }                                                                                     \
        } else {                                                                                  \
            const int so_ = (kk_ - g.kt1) * (BK * 2);                                             \
            _Pragma("unroll") for (int j = 0; j < SEG; ++j) {                                     \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP2, (lds_ptr_t)(sp_ + 64 * j), 16, voP2[j], so_, 0, 0); \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQ2, (lds_ptr_t)(sq_ + 64 * j), 16, voQ2[j], so_, 0, 0); \
            }                                                                                     \
        }                                                                                         \
    }

    // ---- fragments: 32-row x 16-K reads per k16 sub-step kk (0..3)
    const uint32_t frow = lane & 31;
    const uint32_t fsw = (frow >> 1) & 7;
    const uint32_t prow = (wm * (TM * 32) + frow) * 8;
    const uint32_t qrow = kChunks + (wn * (TN * 32) + frow) * 8;
    uint32_t chs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) chs[kk] = (2 * kk + (lane >> 5)) ^ fsw;
#define QN_FRAGS(ST, CH, F)                                             \
    {                                                                   \
        F[0] = (ST)[qrow + (CH)];                                       \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) F[TN + i] = (ST)[prow + i * 256 + (CH)]; \
        _Pragma("unroll") for (int i = 1; i < TN; ++i) F[i] = (ST)[qrow + i * 256 + (CH)];      \
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = f32x16{};
#define QN_MFMAS(F)                                                            \
    _Pragma("unroll") for (int a = 0; a < TN; ++a)                             \
        _Pragma("unroll") for (int b = 0; b < TM; ++b)                         \
            acc[a][b] = mfma32(F[a], F[TN + b], acc[a][b]);

    uint4 fa[TM + TN], fb[TM + TN];
    // One K-step on stage CUR (its kk = 0 fragments already in fa) while NXT receives
    // step k+1; NXT last held step k-1, whose reads all finished before the previous
    // step's barrier. Before the last sub-step every wave waits for its own loads and
    // the barrier certifies NXT complete, so NXT's first fragments are read under the
    // last MFMAs; CUR's reads are all done by then, so the next step may refill it.
#define QN_STEP(KTV, CUR, NXT)                                                 \
    {                                                                          \
        const int k_ = (KTV);                                                  \
        if (k_ + 1 < KT) QN_ISSUE(k_ + 1, NXT)                                 \
        QN_FRAGS(CUR, chs[1], fb)                                              \
        QN_MFMAS(fa)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
        QN_FRAGS(CUR, chs[2], fa)                                              \
        QN_MFMAS(fb)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
        QN_FRAGS(CUR, chs[3], fb)                                              \
        QN_MFMAS(fa)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
        __builtin_amdgcn_s_waitcnt(0);                                         \
        QN_BARRIER();                                                          \
        if (k_ + 1 < KT) QN_FRAGS(NXT, chs[0], fa)                             \
        QN_MFMAS(fb)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
    }

    QN_ISSUE(0, g_st0)
    QN_WAIT_VM(0);
    QN_BARRIER();
    QN_FRAGS(g_st0, chs[0], fa)
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        QN_STEP(kt, g_st0, g_st1)
        QN_STEP(kt + 1, g_st1, g_st0)
    }
    if (kt < KT) QN_STEP(kt, g_st0, g_st1)
#undef QN_STEP
#undef QN_MFMAS
#undef QN_FRAGS
#undef QN_ISSUE

    // ---- epilogue. Every wave is past the last barrier, so the LDS stages are free
    // and no load is in flight. The bf16 C tile (256 rows x 512 B) goes to LDS: rows
    // 128q .. 128q+127 in stage q (q = 0, 1), 16-byte chunk j of row r at position
    // j ^ (r & 31) (two-pass, conflict-free 8-byte writes, conflict-free 16-byte
    // reads); then each row leaves as 512 contiguous bytes, 16 B per lane.
    // The lane holds C[m][n..n+3] for m = tile row frow + 32 b + 32 TM wm and
    // n = 8 gq + 4 (lane >> 5) + 32 a + 32 TN wn.
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const int rl = wm * (TM * 32) + b * 32 + static_cast<int>(frow);
        uint4* arr = (rl >> 7) ? g_st1 : g_st0;
        char* rowp = reinterpret_cast<char*>(arr) + (rl & 127) * 512;
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int nl = wn * (TN * 32) + a * 32 + 8 * gq + 4 * (lane >> 5);
                uint2 o;
                o.x = pack_bf16x2(acc[a][b][4 * gq + 0], acc[a][b][4 * gq + 1]);
                o.y = pack_bf16x2(acc[a][b][4 * gq + 2], acc[a][b][4 * gq + 3]);
                *reinterpret_cast<uint2*>(rowp + (((nl >> 3) ^ (rl & 31)) << 4) + ((nl & 7) << 1)) = o;
            }
        }
    }
    __syncthreads();
    const int cj = tid & 31;                     // 16-byte chunk of the row
    constexpr int kRowsPerPass = NT / 32;
#pragma unroll
    for (int i = 0; i < BM / kRowsPerPass; ++i) {
        const int r = i * kRowsPerPass + (tid >> 5);
        const uint4* arr = (r >> 7) ? g_st1 : g_st0;
        const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(arr) + (r & 127) * 512 +
                                                        ((cj ^ (r & 31)) << 4));
        const int m = m0 + r;
        const int n = n0 + cj * 8;
        if (m < M && n < N) *reinterpret_cast<uint4*>(g.C + static_cast<int64_t>(m) * g.ldc + n) = v;
    }
}

#ifndef QN_GEMM_WAVES_N
#define QN_GEMM_WAVES_N 4
#endif
constexpr int kGemmWM = 2, kGemmWN = QN_GEMM_WAVES_N;

__global__ __launch_bounds__(64 * kGemmWM * kGemmWN, 1)
void gemm_nt_kernel(GemmArgs g) {
    gemm_nt_body<kGemmWM, kGemmWN>(g);
}

// ---------------------------------------------------------------------------
// Prologue of a linear call: one launch whose workgroups take three independent
// jobs, all memory-bound, so they overlap on the chip:
//   [0, n_pre)            LoRA pre-pass  OUT[M, r_pad] = bf16(s * P[M,K] R[r,K]^T),
//                         32 tokens per workgroup, the 4 waves on K-quarters,
//                         summed through LDS; columns r..r_pad-1 come out 0.
//   [n_pre, +n_adapt)     adapter layout: B padded to r_pad columns (forward) or
//                         A^T padded to r_pad columns (input gradient).
//   [.., +n_deq)          double dequantisation to bf16: W_hat row-major
//                         (forward) or W_hat^T through a 64x64 LDS tile (dX).
// ---------------------------------------------------------------------------
struct PrologueArgs {
    const uint8_t* codes; const int8_t* qconst; const float* qscale; const float* qmean;
    int64_t d_out, d_in;
    int transposed;                 // dequant to W_hat^T [d_in, d_out] instead of W_hat
    uint16_t* what;
    const uint16_t* P; int64_t ldp; int M, K;
    const uint16_t* R; int64_t ldr; int r; float s;
    uint16_t* OUT; int r_pad;
    int adapt_mode;                 // 0 none, 1 pad columns, 2 transpose + pad
    const uint16_t* asrc; uint16_t* adst; int64_t arows, acols;
    int n_pre, n_adapt, n_deq;
};

constexpr int kDeqIters = 4;                     // 8-weight groups per thread per workgroup
constexpr int kDeqPerWG = 256 * 8 * kDeqIters;   // weights per row-major dequant workgroup
constexpr int kTP = 64 + 8;                      // LDS pitch (bf16) of the transpose tile

// NT = ceil(r / 32) rank tiles are computed; columns NT*32 .. r_pad-1 are written as
// zeros. Chunks of 64 K of X and (for NT <= 2) of R are prefetched one chunk ahead.
template <int NT>
__device__ __forceinline__ void prepass_job(const PrologueArgs& a, int b, char* lds) {
    constexpr bool kPrefR = NT <= 2;
    f32x16* red = reinterpret_cast<f32x16*>(lds);      // [2][NT][64]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = b * 32;
    const int64_t rowm = min(m0 + (lane & 31), a.M - 1);
    const int nchunk = a.K / 64;                       // whole 64-wide K chunks, split over 4 waves
    const int kbeg = (wave * nchunk / 4) * 64;
    const int kend = ((wave + 1) * nchunk / 4) * 64;
    const int ksub = 8 * (lane >> 5);
    const uint16_t* prow = a.P + rowm * a.ldp + ksub;
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    const uint16_t* rrow[NT];
    bool rok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int rr = t * 32 + (lane & 31);
        rok[t] = rr < a.r;
        rrow[t] = a.R + static_cast<int64_t>(rok[t] ? rr : 0) * a.ldr + ksub;
    }
    // X chunks (64 K each) are loaded kDepth chunks ahead into a ring of registers;
    // R chunks (for NT <= 2) one chunk ahead. Rows of R at or beyond r are not loaded
    // (they contribute zeros).
    constexpr int kDepth = 4;
    uint4 px[kDepth][4];
    uint4 ra[kPrefR ? NT : 1][4], rb[kPrefR ? NT : 1][4];
#define QN_XLOAD(K0, PF)                                                                       \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) PF[u] = *reinterpret_cast<const uint4*>(prow + (K0) + 16 * u);
#define QN_RLOAD(K0, RF)                                                                       \
    if constexpr (kPrefR) {                                                                    \
        _Pragma("unroll") for (int t = 0; t < NT; ++t)                                         \
            _Pragma("unroll") for (int u = 0; u < 4; ++u)                                      \
                RF[t % (kPrefR ? NT : 1)][u] = rok[t] ? *reinterpret_cast<const uint4*>(rrow[t] + (K0) + 16 * u) : uint4{0, 0, 0, 0}; \
    }
#define QN_PCOMP(K0, PF, RF)                                                                   \
    {                                                                                          \
        if constexpr (kPrefR) {                                                                \
            _Pragma("unroll") for (int u = 0; u < 4; ++u)                                      \
                _Pragma("unroll") for (int t = 0; t < NT; ++t) acc[t] = mfma32(RF[t % (kPrefR ? NT : 1)][u], PF[u], acc[t]); \
        } else {                                                                               \
            _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                   \
                uint4 rf[4];                                                                   \
                _Pragma("unroll") for (int u = 0; u < 4; ++u)                                  \
                    rf[u] = rok[t] ? *reinterpret_cast<const uint4*>(rrow[t] + (K0) + 16 * u) : uint4{0, 0, 0, 0}; \
                _Pragma("unroll") for (int u = 0; u < 4; ++u) acc[t] = mfma32(rf[u], PF[u], acc[t]); \
            }                                                                                  \
        }                                                                                      \
    }
    // chunk c (0-based from kbeg) lives in px[c % kDepth]; R alternates ra / rb
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
        if (kbeg + 64 * d < kend) QN_XLOAD(kbeg + 64 * d, px[d])
    if (kbeg < kend) QN_RLOAD(kbeg, ra)
    for (int k = kbeg; k < kend; k += 64 * kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int kc = k + 64 * d;
            if (kc < kend) {
                if (kc + 64 * (kDepth - 1) < kend) QN_XLOAD(kc + 64 * (kDepth - 1), px[(d + kDepth - 1) % kDepth])
                if (d % 2 == 0) {
                    if (kc + 64 < kend) QN_RLOAD(kc + 64, rb)
                    QN_PCOMP(kc, px[d], ra)
                } else {
                    if (kc + 64 < kend) QN_RLOAD(kc + 64, ra)
                    QN_PCOMP(kc, px[d], rb)
                }
            }
        }
    }
#undef QN_XLOAD
#undef QN_RLOAD
#undef QN_PCOMP
    // sum the four K-quarters: waves 2,3 -> 0,1, then 1 -> 0
    if (wave >= 2)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[((wave - 2) * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wave < 2)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] += red[(wave * NT + t) * 64 + lane];
    __syncthreads();
    if (wave == 1)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[t * 64 + lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
    const int m = m0 + (lane & 31);
    if (m >= a.M) return;
    uint16_t* orow = a.OUT + static_cast<int64_t>(m) * a.r_pad;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const f32x16 v = acc[t] + red[t * 64 + lane];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int n = t * 32 + 8 * gq + 4 * (lane >> 5);
            uint2 o;
            o.x = pack_bf16x2(a.s * v[4 * gq + 0], a.s * v[4 * gq + 1]);
            o.y = pack_bf16x2(a.s * v[4 * gq + 2], a.s * v[4 * gq + 3]);
            *reinterpret_cast<uint2*>(orow + n) = o;
        }
    }
    // zero padding columns NT*32 .. r_pad-1 (lanes 0..31 own this row, 4 bf16 per store)
    for (int n = NT * 32 + 4 * (lane >> 5); n < a.r_pad; n += 8)
        *reinterpret_cast<uint2*>(orow + n) = uint2{0u, 0u};
}

// Adapter layouts; destination is [rows, r_pad] (pad) or [acols, r_pad] (transpose).
__device__ __forceinline__ void adapt_job(const PrologueArgs& a, int b) {
    const int64_t total = (a.adapt_mode == 1 ? a.arows : a.acols) * a.r_pad;
    for (int64_t idx = static_cast<int64_t>(b) * 256 + threadIdx.x; idx < total;
         idx += static_cast<int64_t>(a.n_adapt) * 256) {
        const int64_t i = idx / a.r_pad, j = idx % a.r_pad;
        uint16_t v = 0;
        if (a.adapt_mode == 1) {
            if (j < a.acols) v = a.asrc[i * a.acols + j];          // B [arows, acols=r] -> [arows, r_pad]
        } else {
            if (j < a.arows) v = a.asrc[j * a.acols + i];          // A [arows=r, acols] -> A^T [acols, r_pad]
        }
        a.adst[idx] = v;
    }
}

__device__ __forceinline__ void dequant_rows_job(const PrologueArgs& a, int b, const float* s_code) {
    const int64_t n = a.d_out * a.d_in;           // multiple of 64 on this path
    const float mu = a.qmean[0];
    const uint32_t* codes32 = reinterpret_cast<const uint32_t*>(a.codes);
    int64_t t[kDeqIters];
    uint32_t word[kDeqIters];
    int8_t q[kDeqIters];
    float bs[kDeqIters];
#pragma unroll
    for (int it = 0; it < kDeqIters; ++it) {
        t[it] = static_cast<int64_t>(b) * (kDeqPerWG / 8) + it * 256 + threadIdx.x;
        const bool ok = t[it] * 8 < n;
        const int64_t blk = ok ? t[it] >> 3 : 0;
        word[it] = ok ? codes32[t[it]] : 0u;
        q[it] = a.qconst[blk];
        bs[it] = a.qscale[blk / kGroup];
    }
#pragma unroll
    for (int it = 0; it < kDeqIters; ++it) {
        if (t[it] * 8 >= n) break;
        const float ahat = block_constant(q[it], bs[it], mu);
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = s_code[(word[it] >> (4 * e)) & 0xFu] * ahat;
        uint4 o;
        o.x = pack_bf16x2(w[0], w[1]);
        o.y = pack_bf16x2(w[2], w[3]);
        o.z = pack_bf16x2(w[4], w[5]);
        o.w = pack_bf16x2(w[6], w[7]);
        *reinterpret_cast<uint4*>(a.what + t[it] * 8) = o;
    }
}

__device__ __forceinline__ void dequant_transposed_job(const PrologueArgs& a, int b, const float* s_code,
                                                       uint16_t* tile) {
    const int tid = threadIdx.x;
    const int tiles_i = static_cast<int>(a.d_in / 64);
    const int64_t i0 = static_cast<int64_t>(b % tiles_i) * 64;
    const int64_t o0 = static_cast<int64_t>(b / tiles_i) * 64;
    const int ol = tid >> 2;             // local row o (becomes the output column)
    const int q4 = tid & 3;              // which 16 of the 64 columns
    const int64_t o = o0 + ol;
    if (o < a.d_out) {
        const int64_t e0 = o * a.d_in + i0 + q4 * 16;
        const int64_t blk = e0 >> 6;
        const float ahat = block_constant(a.qconst[blk], a.qscale[blk / kGroup], a.qmean[0]);
        const uint2 cw = *reinterpret_cast<const uint2*>(a.codes + (e0 >> 1));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t word = e < 8 ? cw.x : cw.y;
            tile[(q4 * 16 + e) * kTP + ol] = bf16_bits(s_code[(word >> (4 * (e & 7))) & 0xFu] * ahat);
        }
    }
    __syncthreads();
    const int il = tid >> 2;
    const int seg = (tid & 3) * 16;
    const int64_t i = i0 + il;
    const int64_t oc = o0 + seg;
    if (oc < a.d_out) {                  // d_out % 64 == 0 on this path: whole 16-wide segments
        const uint4* src = reinterpret_cast<const uint4*>(&tile[il * kTP + seg]);
        uint4* dst = reinterpret_cast<uint4*>(a.what + i * a.d_out + oc);
        dst[0] = src[0];
        dst[1] = src[1];
    }
}

template <int NT>
__global__ __launch_bounds__(256)
void prologue_kernel(PrologueArgs a, NF4Tables tab) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int b = blockIdx.x;
    if (b < a.n_pre) {
        prepass_job<NT>(a, b, lds);
        return;
    }
    if (b < a.n_pre + a.n_adapt) {
        adapt_job(a, b - a.n_pre);
        return;
    }
    float* s_code = reinterpret_cast<float*>(lds);
    if (threadIdx.x < 16) s_code[threadIdx.x] = tab.code[threadIdx.x];
    __syncthreads();
    const int bd = b - a.n_pre - a.n_adapt;
    if (a.transposed)
        dequant_transposed_job(a, bd, s_code, reinterpret_cast<uint16_t*>(lds + 64));
    else
        dequant_rows_job(a, bd, s_code);
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

// Each wave takes kRowsPerWave consecutive rows; lane j takes blocks j, j+64, ... of
// every row, so its x blocks are loaded once for all the rows. All code words,
// constants and scales of the wave's rows are loaded before any arithmetic. Per block
// the 32 code bytes are looked up as bf16 code pairs and dotted with bf16 x pairs
// (v_dot2_f32_bf16); the block constant a_hat multiplies the block's partial sum
// once (a per-block scale factors out of the sum over the block).
constexpr int kRowsPerWave = 4;

__device__ __forceinline__ float gemv_block(const uint4 c0, const uint4 c1, const uint4* xv, const uint32_t* lut2) {
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float part = 0.0f;
#pragma unroll
    for (int w4 = 0; w4 < 8; ++w4) {
        const uint32_t xw[4] = {xv[w4].x, xv[w4].y, xv[w4].z, xv[w4].w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (cw[w4] >> (8 * b)) & 0xFFu;
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lut2[byte]),
                                                   __builtin_bit_cast(bf16x2, xw[b]), part, false);
        }
    }
    return part;
}

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
    const int row0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
    if (row0 >= d_out) return;
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    float acc[kRowsPerWave];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) acc[rr] = 0.0f;
    for (int jb = lane; jb < nbpr; jb += 64) {
        uint4 c[kRowsPerWave][2];
        int8_t q[kRowsPerWave];
        float bsc[kRowsPerWave];
#pragma unroll
        for (int rr = 0; rr < kRowsPerWave; ++rr) {
            const int o = min(row0 + rr, d_out - 1);
            const int64_t blk = static_cast<int64_t>(o) * nbpr + jb;
            c[rr][0] = codes[blk * 2];
            c[rr][1] = codes[blk * 2 + 1];
            q[rr] = qconst[blk];
            bsc[rr] = qscale[blk >> 8];
        }
        uint4 xv[8];
#pragma unroll
        for (int w4 = 0; w4 < 8; ++w4) xv[w4] = x4[static_cast<int64_t>(jb) * 8 + w4];
#pragma unroll
        for (int rr = 0; rr < kRowsPerWave; ++rr) {
            const float ahat = mu + bsc[rr] * qlut[q[rr] + 128];
            acc[rr] += ahat * gemv_block(c[rr][0], c[rr][1], xv, lut2);
        }
    }
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int o = min(row0 + rr, d_out - 1);
        for (int k = lane; k < r; k += 64) acc[rr] += bf16_to_f32(B[static_cast<int64_t>(o) * r + k]) * s_t[k];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int rr = 0; rr < kRowsPerWave; ++rr) acc[rr] += __shfl_xor(acc[rr], off);
    if (lane < kRowsPerWave) {
        float v = acc[0];
#pragma unroll
        for (int rr = 1; rr < kRowsPerWave; ++rr)
            if (lane == rr) v = acc[rr];
        if (row0 + lane < d_out) y[row0 + lane] = bf16_bits(v);
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
    // every operand is < 4 GiB (checked by the caller): the extents fit 32 bits
    g.bytesP = static_cast<uint32_t>(2 * ldp * M);
    g.bytesQ = static_cast<uint32_t>(2 * ldq * N);
    g.bytesP2 = static_cast<uint32_t>(2 * ldp2 * M);
    g.bytesQ2 = static_cast<uint32_t>(2 * ldq2 * N);
    QN_LAUNCH("gemm_nt_kernel", st, gemm_nt_kernel, dim3(g.tiles_m * g.tiles_n), dim3(64 * kGemmWM * kGemmWN), 0,
              st, g);
    return hipGetLastError();
}

hipError_t launch_prologue(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                           const float* qmean, int64_t d_out, int64_t d_in, bool transposed,
                           uint16_t* what, const uint16_t* P, int64_t ldp, int64_t M, int64_t K,
                           const uint16_t* R, int64_t ldr, int r, float s, uint16_t* OUT, int r_pad,
                           int adapt_mode, const uint16_t* asrc, uint16_t* adst, int64_t arows,
                           int64_t acols, hipStream_t st) {
    PrologueArgs a;
    a.codes = codes; a.qconst = qconst; a.qscale = qscale; a.qmean = qmean;
    a.d_out = d_out; a.d_in = d_in; a.transposed = transposed ? 1 : 0; a.what = what;
    a.P = P; a.ldp = ldp; a.M = static_cast<int>(M); a.K = static_cast<int>(K);
    a.R = R; a.ldr = ldr; a.r = r; a.s = s; a.OUT = OUT; a.r_pad = r_pad;
    a.adapt_mode = adapt_mode; a.asrc = asrc; a.adst = adst; a.arows = arows; a.acols = acols;
    a.n_pre = static_cast<int>((M + 31) / 32);
    const int64_t adapt_elems = adapt_mode == 0 ? 0 : (adapt_mode == 1 ? arows : acols) * r_pad;
    a.n_adapt = static_cast<int>(adapt_elems == 0 ? 0 : std::min<int64_t>(64, (adapt_elems + 255) / 256));
    const int64_t n = d_out * d_in;
    a.n_deq = static_cast<int>(transposed ? (d_in / 64) * ((d_out + 63) / 64) : (n + kDeqPerWG - 1) / kDeqPerWG);
    const int NT = (r + 31) / 32;
    const size_t lds_pre = static_cast<size_t>(2) * NT * 64 * sizeof(f32x16);
    const size_t lds_deq = 64 + static_cast<size_t>(64) * kTP * sizeof(uint16_t);
    const size_t lds = std::max(lds_pre, lds_deq);
    const dim3 grid(static_cast<unsigned>(a.n_pre + a.n_adapt + a.n_deq));
    const NF4Tables& tab = tables();
    switch (NT) {
#define QN_PRO_CASE(T) \
        case T: QN_LAUNCH("prologue_kernel", st, prologue_kernel<T>, grid, dim3(256), lds, st, a, tab); break;
        QN_PRO_CASE(1) QN_PRO_CASE(2) QN_PRO_CASE(3) QN_PRO_CASE(4)
        QN_PRO_CASE(5) QN_PRO_CASE(6) QN_PRO_CASE(7) QN_PRO_CASE(8)
#undef QN_PRO_CASE
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
