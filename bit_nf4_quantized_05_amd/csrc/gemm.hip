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

constexpr int kDeqPerWG = 8192;                  // weights per row-major dequant workgroup (128 blocks)
constexpr int kTP = 64 + 8;                      // LDS pitch (bf16) of the transpose tile

// Three LDS ring slots of the pre-pass, as distinct objects (each 4 waves x 32 rows x
// 128 B) so the compiler can tell that reading one does not depend on direct-to-LDS
// loads into another. The other prologue jobs use them as scratch.
__shared__ uint4 g_pre0[4 * 256];
__shared__ uint4 g_pre1[4 * 256];
__shared__ uint4 g_pre2[4 * 256];

// NT = ceil(r / 32) rank tiles are computed; columns NT*32 .. r_pad-1 are written as
// zeros. The 4 waves take K-quarters; each streams its quarter in chunks of 32 rows
// x 64 K of X through a ring of 3 LDS slots, two chunks ahead: a chunk is loaded
// by 4 direct-to-LDS loads of 8 whole 128-byte rows each (coalesced), with the
// 16-byte pieces of row r XOR-swizzled by ((r >> 1) & 7) so the MFMA fragment
// reads (32 rows, one piece each) are free of bank conflicts. For NT <= 2 the
// matching chunk of R is fetched into registers with the chunk of X (vector loads
// complete in issue order, so both must run equally far ahead); for NT > 2 (rank
// >= 96) R fragments are loaded at their use.
template <int NT>
__device__ __forceinline__ void prepass_job(const PrologueArgs& a, int b) {
    constexpr bool kPrefR = NT <= 2;
    constexpr int kRS = kPrefR ? NT : 1;               // R tiles held per ring slot
    constexpr int kLoads = 4 + (kPrefR ? 4 * NT : 0);  // vector loads per chunk
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = b * 32;
    const int nchunk = a.K / 64;                       // whole 64-wide K chunks, split over 4 waves
    const int kbeg = (wave * nchunk / 4) * 64;
    const int kend = ((wave + 1) * nchunk / 4) * 64;
    const int ksub = 8 * (lane >> 5);
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
    // DMA source of lane i in load u: row 8u + i/8 of the chunk, piece (i%8) ^ swz
    const uint16_t* xsrc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 8 * u + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        xsrc[u] = a.P + static_cast<int64_t>(min(m0 + r, a.M - 1)) * a.ldp + 8 * c;
    }
    // fragment of sub-step u: row lane%32, piece (2u + lane/32) ^ ((row >> 1) & 7)
    const int frow = lane & 31;
    int fpos[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) fpos[u] = frow * 8 + ((2 * u + (lane >> 5)) ^ ((frow >> 1) & 7));
    uint4 pr[3][kRS][4];
#define QN_CLOAD(K0, SL, S)                                                                    \
    {                                                                                          \
        uint4* sl_ = (SL) + wave * 256;                                                        \
        _Pragma("unroll") for (int u = 0; u < 4; ++u)                                          \
            __builtin_amdgcn_global_load_lds((global_ptr)(xsrc[u] + (K0)), (lds_ptr)(sl_ + 64 * u), 16, 0, 0); \
        if constexpr (kPrefR) {                                                                \
            _Pragma("unroll") for (int t = 0; t < kRS; ++t)                                    \
                _Pragma("unroll") for (int u = 0; u < 4; ++u)                                  \
                    pr[S][t][u] = rok[t] ? *reinterpret_cast<const uint4*>(rrow[t] + (K0) + 16 * u) \
                                         : uint4{0, 0, 0, 0};                                  \
        }                                                                                      \
    }
#define QN_PCOMP(K0, SL, S)                                                                    \
    {                                                                                          \
        const uint4* sl_ = (SL) + wave * 256;                                                  \
        uint4 xf[4];                                                                           \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) xf[u] = sl_[fpos[u]];                    \
        if constexpr (kPrefR) {                                                                \
            _Pragma("unroll") for (int u = 0; u < 4; ++u)                                      \
                _Pragma("unroll") for (int t = 0; t < NT; ++t)                                 \
                    acc[t] = mfma32(pr[S][t % kRS][u], xf[u], acc[t]);                         \
        } else {                                                                               \
            _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                   \
                uint4 rf[4];                                                                   \
                _Pragma("unroll") for (int u = 0; u < 4; ++u)                                  \
                    rf[u] = rok[t] ? *reinterpret_cast<const uint4*>(rrow[t] + (K0) + 16 * u) : uint4{0, 0, 0, 0}; \
                _Pragma("unroll") for (int u = 0; u < 4; ++u) acc[t] = mfma32(rf[u], xf[u], acc[t]); \
            }                                                                                  \
        }                                                                                      \
    }
    // chunk kc: wait until its loads are done (those of the up to two later chunks may
    // still be in flight), compute, then refill its slot with chunk kc + 3
#define QN_PSTEP(KC, SL, S)                                                                    \
    if ((KC) < kend) {                                                                         \
        if ((KC) + 128 < kend) { QN_WAIT_VM(2 * kLoads); }                                    \
        else if ((KC) + 64 < kend) { QN_WAIT_VM(kLoads); }                                    \
        else { QN_WAIT_VM(0); }                                                                \
        QN_PCOMP(KC, SL, S)                                                                    \
        if ((KC) + 192 < kend) QN_CLOAD((KC) + 192, SL, S)                                     \
    }
    if (kbeg < kend) QN_CLOAD(kbeg, g_pre0, 0)
    if (kbeg + 64 < kend) QN_CLOAD(kbeg + 64, g_pre1, 1)
    if (kbeg + 128 < kend) QN_CLOAD(kbeg + 128, g_pre2, 2)
    for (int k = kbeg; k < kend; k += 192) {
        QN_PSTEP(k, g_pre0, 0)
        QN_PSTEP(k + 64, g_pre1, 1)
        QN_PSTEP(k + 128, g_pre2, 2)
    }
#undef QN_PSTEP
#undef QN_CLOAD
#undef QN_PCOMP
    // sum the four K-quarters, one rank tile at a time through g_pre0 (every load
    // has landed: each wave's last step waited for all of its loads)
    f32x16* red = reinterpret_cast<f32x16*>(g_pre0);   // [2][64]
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        __syncthreads();
        if (wave >= 2) red[(wave - 2) * 64 + lane] = acc[t];
        __syncthreads();
        if (wave < 2) acc[t] += red[wave * 64 + lane];
        __syncthreads();
        if (wave == 1) red[lane] = acc[t];
        __syncthreads();
        if (wave == 0) acc[t] += red[lane];
    }
    if (wave != 0) return;
    const int m = m0 + (lane & 31);
    if (m >= a.M) return;
    uint16_t* orow = a.OUT + static_cast<int64_t>(m) * a.r_pad;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const f32x16 v = acc[t];
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
// Thread t of the job writes 16-byte destination chunk t (8 entries of one row), so
// every load it needs is independent and issued at once (one memory round trip).
__device__ __forceinline__ void adapt_job(const PrologueArgs& a, int b) {
    const int cpr = a.r_pad / 8;                                   // chunks per destination row
    const int64_t rows = a.adapt_mode == 1 ? a.arows : a.acols;
    const int64_t c = static_cast<int64_t>(b) * 256 + threadIdx.x;
    if (c >= rows * cpr) return;
    const int64_t i = c / cpr;
    const int j0 = static_cast<int>(c % cpr) * 8;
    uint16_t v[8];
    if (a.adapt_mode == 1) {                                       // B [arows, r] -> [arows, r_pad]
        if (j0 + 8 <= a.acols && (a.acols & 7) == 0) {
            const uint4 w = *reinterpret_cast<const uint4*>(a.asrc + i * a.acols + j0);
            *reinterpret_cast<uint4*>(a.adst + c * 8) = w;
            return;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = j0 + e < a.acols ? a.asrc[i * a.acols + j0 + e] : uint16_t{0};
    } else {                                                       // A [r, acols] -> A^T [acols, r_pad]
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = j0 + e < a.arows ? a.asrc[static_cast<int64_t>(j0 + e) * a.acols + i] : uint16_t{0};
    }
    *reinterpret_cast<uint4*>(a.adst + c * 8) =
        uint4{v[0] | (static_cast<uint32_t>(v[1]) << 16), v[2] | (static_cast<uint32_t>(v[3]) << 16),
              v[4] | (static_cast<uint32_t>(v[5]) << 16), v[6] | (static_cast<uint32_t>(v[7]) << 16)};
}

// Row-major dequantisation of kDeqPerWG = 8192 weights (128 blocks): threads 0..127
// form a_hat of one block each into LDS (the constants are loaded once per block,
// not per weight); thread t takes the 8-weight code words t + 256 q (q = 0..3), so
// every load and 16-byte store of a wave is contiguous.
__device__ __forceinline__ void dequant_rows_job(const PrologueArgs& a, int b, const float* s_code,
                                                 float* s_ahat) {
    constexpr int kWords = kDeqPerWG / 8 / 256;  // code words per thread
    const int tid = threadIdx.x;
    const int64_t n = a.d_out * a.d_in;           // multiple of 64 on this path
    const int64_t w0 = static_cast<int64_t>(b) * kDeqPerWG;
    const uint32_t* codes32 = reinterpret_cast<const uint32_t*>(a.codes);
    // code words first (the a_hat loads below are waited for before these)
    uint32_t cw[kWords];
#pragma unroll
    for (int q = 0; q < kWords; ++q) cw[q] = codes32[min(w0 + 8 * (tid + 256 * q), n - 8) / 8];
    if (tid < kDeqPerWG / 64) {
        const int64_t blk = min(w0 / 64 + tid, n / 64 - 1);
        s_ahat[tid] = block_constant(a.qconst[blk], a.qscale[blk / kGroup], a.qmean[0]);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
        const int t = tid + 256 * q;
        const int64_t e0 = w0 + 8 * t;
        if (e0 >= n) break;
        const float ahat = s_ahat[t >> 3];
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = s_code[(cw[q] >> (4 * e)) & 0xFu] * ahat;
        *reinterpret_cast<uint4*>(a.what + e0) = uint4{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                                                      pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
    }
}

// Transposed dequantisation of a 64 (o) x 64 (i) tile: each row o of the tile is one
// 64-block, whose a_hat threads 0..63 form into LDS; thread (o, q4) dequantises 16
// weights into the LDS tile, which is written out transposed as W_hat^T rows.
__device__ __forceinline__ void dequant_transposed_job(const PrologueArgs& a, int b, const float* s_code,
                                                       float* s_ahat, uint16_t* tile) {
    const int tid = threadIdx.x;
    const int tiles_i = static_cast<int>(a.d_in / 64);
    const int64_t i0 = static_cast<int64_t>(b % tiles_i) * 64;
    const int64_t o0 = static_cast<int64_t>(b / tiles_i) * 64;
    const int ol = tid >> 2;             // local row o (becomes the output column)
    const int q4 = tid & 3;              // which 16 of the 64 columns
    const int64_t o = min(o0 + ol, a.d_out - 1);
    const int64_t e0 = o * a.d_in + i0 + q4 * 16;
    const uint2 cw = *reinterpret_cast<const uint2*>(a.codes + (e0 >> 1));
    if (tid < 64) {
        const int64_t blk = (min(o0 + tid, a.d_out - 1) * a.d_in + i0) >> 6;
        s_ahat[tid] = block_constant(a.qconst[blk], a.qscale[blk / kGroup], a.qmean[0]);
    }
    __syncthreads();
    const float ahat = s_ahat[ol];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t word = e < 8 ? cw.x : cw.y;
        tile[(q4 * 16 + e) * kTP + ol] = bf16_bits(s_code[(word >> (4 * (e & 7))) & 0xFu] * ahat);
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
    char* lds = reinterpret_cast<char*>(g_pre1);          // 16 KB of scratch for the other jobs
    const int b = blockIdx.x;
    if (b < a.n_pre) {
        prepass_job<NT>(a, b);
        return;
    }
    if (b < a.n_pre + a.n_adapt) {
        adapt_job(a, b - a.n_pre);
        return;
    }
    float* s_code = reinterpret_cast<float*>(lds);             // 16 floats
    float* s_ahat = reinterpret_cast<float*>(lds + 64);        // up to 128 floats
    if (threadIdx.x < 16) s_code[threadIdx.x] = tab.code[threadIdx.x];
    const int bd = b - a.n_pre - a.n_adapt;
    if (a.transposed)
        dequant_transposed_job(a, bd, s_code, s_ahat, reinterpret_cast<uint16_t*>(lds + 64 + 512));
    else
        dequant_rows_job(a, bd, s_code, s_ahat);
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
// d_seq = 1 (decode), two launches:
//   lora_ax_partial: the 64-column blocks of x are split into nparts contiguous
//     slices (nparts * r <= 1024); workgroup w writes, for every rank row j, the dot
//     product of A[j] and x over slice w to part[w][j] (fixed summation order).
//   gemv_nf4: streams the packed codes once and adds B (s A x), summing the slice
//     partials in a fixed order: y = W_hat x + B (s A x). Deterministic.
// ---------------------------------------------------------------------------
constexpr int kAxMaxParts = 16;

__global__ __launch_bounds__(256)
void lora_ax_partial_kernel(const uint16_t* __restrict__ A, int d_in, const uint16_t* __restrict__ x,
                            int r, int blocks_per_part, float* __restrict__ part) {
    __shared__ float red[256];
    const int tid = threadIdx.x;
    const int groups = 256 / r;                   // threads per rank row
    const int nb64 = d_in / 64;
    const int b_lo = blockIdx.x * blocks_per_part;
    const int b_hi = min(b_lo + blocks_per_part, nb64);
    float acc = 0.0f;
    if (tid < groups * r) {
        const int j = tid % r;
        for (int b = b_lo + tid / r; b < b_hi; b += groups) {
            const uint4* ar = reinterpret_cast<const uint4*>(A + static_cast<int64_t>(j) * d_in + b * 64);
            const uint4* xr = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(b) * 64);
            uint4 av[8], xv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { av[e] = ar[e]; xv[e] = xr[e]; }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t aw[4] = {av[e].x, av[e].y, av[e].z, av[e].w};
                const uint32_t xw[4] = {xv[e].x, xv[e].y, xv[e].z, xv[e].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[q]),
                                                          __builtin_bit_cast(bf16x2, xw[q]), acc, false);
            }
        }
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < r) {
        float t = 0.0f;
        for (int g = 0; g < groups; ++g) t += red[g * r + tid];
        part[static_cast<int64_t>(blockIdx.x) * r + tid] = t;
    }
}

// gemv_nf4: a workgroup of 16 waves takes 16 consecutive rows, one per wave (four
// waves per SIMD hide each other's latencies). A row is walked in segments of 4096
// weights = 64 blocks; in a segment, lane l of a wave owns block l's constant and
// two chunks of 2048 weights, in each the weights [32 l, 32 l + 32) = 16 code bytes
// (one 16-byte load; the wave reads 1 KB contiguous), half of block 32 h + l/2.
// The vector-memory address unit takes about as long for a 1-byte load as for a
// 16-byte one, so everything but the codes is loaded once per workgroup with wide
// loads by one wave each and passed through LDS: the x segment (waves 0..7), the
// 16 rows' 8-bit constants (wave 8, when the rows' 64-block runs are 16-byte
// aligned; else each wave loads its own), their group scales (wave 9), the A x
// slice partials (waves 10..13) and the 16 rows of B (wave 14). Every wave issues
// the loads it must wait for before its code loads, so that wait never covers the
// codes, and the next segment's loads go out before the current one is computed.
// A lane forms a_hat of block l and hands it to the two lanes owning the block's
// halves by a cross-lane read. Each code byte (two weights) is looked up as a pair
// of bf16 code values and dotted with the bf16 x pair (v_dot2_f32_bf16); a_hat
// multiplies each half-block partial once (the constant factors out of the sum
// over its block). The lookup table is replicated kLutCopies times with copy c in
// bank c, so a half-wave never collides, and the x chunks are XOR-swizzled so the
// 16-byte reads of 16 lanes hit 16 distinct bank groups. s (A x) is formed before
// the weight loop, so each wave finishes on its own.
constexpr int kGvWaves = 16;
constexpr int kGvSeg = 4096;
constexpr int kLutCopies = 32;

struct GvRowSeg {
    uint4 cw[2];            // code words of the two chunks
    int8_t qv;              // constant of block l (only when each wave loads its own)
    float sv;               // its group scale (idem)
};

struct GvStage {            // per-workgroup staging loads of one segment
    uint4 v;                // x (waves 0..7) or constants (wave 8)
    float sc;               // group scale (wave 9, lanes < 32)
};

__device__ __forceinline__ float gemv_half_block(const uint4 c, const uint4* xv, const uint32_t* lut,
                                                 uint32_t lane_off) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float part = 0.0f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        const uint32_t xw[4] = {xv[w4].x, xv[w4].y, xv[w4].z, xv[w4].w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (cw[w4] >> (8 * b)) & 0xFFu;
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lut[byte * kLutCopies + lane_off]),
                                                   __builtin_bit_cast(bf16x2, xw[b]), part, false);
        }
    }
    return part;
}

// position of 16-byte x chunk c of a segment in LDS: lane l = (c >> 2) & 63 reads
// chunks 4 l .. 4 l + 3; their order is XORed with bits 2..3 of l
__device__ __forceinline__ int gv_xpos(int c) { return (c & ~3) | ((c & 3) ^ ((c >> 4) & 3)); }

template <bool kStageQ>
__global__ __launch_bounds__(1024)
void gemv_nf4_kernel(const uint4* __restrict__ codes, const int8_t* __restrict__ qconst,
                     const float* __restrict__ qscale, const float* __restrict__ qmean,
                     int d_out, int d_in, const uint16_t* __restrict__ x,
                     const uint16_t* __restrict__ B, int r, float s, const float* __restrict__ part,
                     int nparts, uint16_t* __restrict__ y, NF4Tables tab) {
    __shared__ uint4 lut4[256 * kLutCopies / 4];
    __shared__ uint4 xs[2][kGvSeg / 8];
    __shared__ uint4 qcs[2][kGvWaves * 64 / 16];      // row i's 64 constants at bytes 64 i ..
    __shared__ float qss[2][2 * kGvWaves];            // row i: scales of groups base_i, base_i + 1
    __shared__ float tvs[1024];
    __shared__ uint4 bs[kGvWaves * 256 * 2 / 16];     // the 16 rows of B (r <= 256)
    __shared__ float qlut[256];
    __shared__ float s_t[256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (a scalar), so the per-wave roles below are scalar branches and
    // no wave waits on loads of a role it does not have
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = blockIdx.x * kGvWaves;
    const int row = min(row0 + wave, d_out - 1);
    const int nbpr = d_in / 64;
    const int upr = d_in / 32;                    // 16-byte code words per row
    const int nseg = (d_in + kGvSeg - 1) / kGvSeg;
    const int64_t n_b = static_cast<int64_t>(d_out) * nbpr;
    const int64_t n_g = (n_b + 255) / 256;
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    const int64_t row_u = static_cast<int64_t>(row) * upr;

    // first block of row i's run in segment S, and the first group it touches
    auto run0 = [&](int i, int S) { return static_cast<int64_t>(min(row0 + i, d_out - 1)) * nbpr + S * 64; };
    auto stage_issue = [&](GvStage& g, int S) {
        if (wave < 8) {
            const int col = S * kGvSeg + 8 * tid;
            g.v = x4[min(col, d_in - 8) / 8];
        } else if (kStageQ && wave == 8) {
            // row lane/4, bytes 16 (lane%4) .. of its 64-block run (16-byte aligned);
            // the tail of the last row is clamped into the array (those bytes are unused)
            const int64_t b = min(run0(lane >> 2, S) + 16 * (lane & 3), n_b - 16);
            g.v = *reinterpret_cast<const uint4*>(qconst + b);
        } else if (wave == 9 && lane < 2 * kGvWaves) {
            g.sc = qscale[min((run0(lane >> 1, S) >> 8) + (lane & 1), n_g - 1)];
        }
    };
    auto stage_store = [&](const GvStage& g, int S) {
        const int k = S & 1;
        if (wave < 8) xs[k][gv_xpos(tid)] = S * kGvSeg + 8 * tid < d_in ? g.v : uint4{0, 0, 0, 0};
        else if (kStageQ && wave == 8) qcs[k][lane] = g.v;
        else if (wave == 9 && lane < 2 * kGvWaves) qss[k][lane] = g.sc;
    };
    auto seg_issue = [&](GvRowSeg& k, int S) {
        if (!kStageQ) {
            const int64_t b = static_cast<int64_t>(row) * nbpr + min(S * 64 + lane, nbpr - 1);
            k.qv = qconst[b];
            k.sv = qscale[b >> 8];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = S * kGvSeg + h * 2048 + lane * 32;
            k.cw[h] = codes[row_u + (col < d_in ? col / 32 : 0)];
        }
    };

    // ---- loads: staged data first, then the codes
    GvStage st;
    st.v = uint4{0, 0, 0, 0};
    st.sc = 0.0f;
    stage_issue(st, 0);
    const int nval = nparts * r;                  // <= 1024
    uint4 tst = uint4{0, 0, 0, 0};
    if (wave >= 10 && wave < 14)
        tst = reinterpret_cast<const uint4*>(part)[min(tid - 640, (nval + 3) / 4 - 1)];
    const int nbv = 2 * r;                        // 16-byte pieces of the 16 rows of B
    const uint4* b4 = reinterpret_cast<const uint4*>(B + static_cast<int64_t>(row0) * r);
    uint4 bst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) bst[i] = uint4{0, 0, 0, 0};
    if (wave == 14) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (64 * i < nbv) bst[i] = b4[min(lane + 64 * i, nbv - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
    GvRowSeg g0, g1;
    seg_issue(g0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- tables and staged data to LDS; the barriers wait for LDS writes only
    if (tid < 256) {
        // code-book values picked from the (scalar) kernel arguments by selects: an
        // indexed read would be a memory load
        float lo = tab.code[0], hi = tab.code[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            lo = (tid & 15) == i ? tab.code[i] : lo;
            hi = (tid >> 4) == i ? tab.code[i] : hi;
        }
        const uint32_t v = pack_bf16x2(lo, hi);
#pragma unroll
        for (int c = 0; c < kLutCopies / 4; ++c) lut4[tid * (kLutCopies / 4) + c] = uint4{v, v, v, v};
        qlut[tid] = static_cast<float>(tid - 128) / static_cast<float>(kInt8Step);
    }
    stage_store(st, 0);
    if (wave >= 10 && wave < 14) reinterpret_cast<uint4*>(tvs)[tid - 640] = tst;
    if (wave == 14) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (lane + 64 * i < nbv) bs[lane + 64 * i] = bst[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // s (A x), summed per rank row in slice order
    if (tid < r) {
        float t = 0.0f;
        for (int p = 0; p < nparts; ++p) t += tvs[p * r + tid];
        s_t[tid] = s * t;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const uint32_t* lut = reinterpret_cast<const uint32_t*>(lut4);
    const uint32_t lane_off = static_cast<uint32_t>(lane & (kLutCopies - 1));
    const float mu = qmean[0];
    float acc = 0.0f;
    auto compute = [&](const GvRowSeg& k, int S) {
        const int kb = S & 1;
        const int64_t b = static_cast<int64_t>(row) * nbpr + S * 64 + lane;
        const bool bok = S * 64 + lane < nbpr;
        int q;
        float sc;
        if (kStageQ) {
            q = reinterpret_cast<const int8_t*>(qcs[kb])[wave * 64 + lane];
            sc = qss[kb][2 * wave + static_cast<int>((b >> 8) - (run0(wave, S) >> 8))];
        } else {
            q = k.qv;
            sc = k.sv;
        }
        const float ah = bok ? mu + sc * qlut[q + 128] : 0.0f;
        const uint4* xb = xs[kb];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float a = __shfl(ah, h * 32 + (lane >> 1));
            uint4 xv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] = xb[h * 256 + 4 * lane + (e ^ ((lane >> 2) & 3))];
            acc += a * gemv_half_block(k.cw[h], xv, lut, lane_off);
        }
    };
    // segment S+1's loads go out before segment S is computed; its staged data is
    // stored to the other LDS buffers after, behind a barrier
    auto step = [&](GvRowSeg& cur, GvRowSeg& nxt, int S) {
        const bool more = S + 1 < nseg;
        if (more) {
            stage_issue(st, S + 1);
            __builtin_amdgcn_sched_barrier(0);
            seg_issue(nxt, S + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        compute(cur, S);
        if (more) {
            stage_store(st, S + 1);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };
    for (int sg = 0; sg < nseg; sg += 2) {
        step(g0, g1, sg);
        if (sg + 1 < nseg) step(g1, g0, sg + 1);
    }

    // ---- rank-r term of this wave's row, row sum, store
    const uint16_t* brow = reinterpret_cast<const uint16_t*>(bs) + wave * r;
    for (int k = lane; k < r; k += 64) acc += bf16_to_f32(brow[k]) * s_t[k];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0 && row0 + wave < d_out) y[row0 + wave] = bf16_bits(acc);
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
    a.n_adapt = static_cast<int>((adapt_elems / 8 + 255) / 256);    // one 8-entry chunk per thread
    const int64_t n = d_out * d_in;
    a.n_deq = what == nullptr ? 0   // pre-pass (and adapter layout) only
                              : static_cast<int>(transposed ? (d_in / 64) * ((d_out + 63) / 64)
                                                            : (n + kDeqPerWG - 1) / kDeqPerWG);
    const int NT = (r + 31) / 32;
    static_assert(64 + 512 + 64 * kTP * sizeof(uint16_t) <= sizeof(g_pre1), "dequant scratch fits a ring slot");
    const dim3 grid(static_cast<unsigned>(a.n_pre + a.n_adapt + a.n_deq));
    const NF4Tables& tab = tables();
    switch (NT) {
#define QN_PRO_CASE(T) \
        case T: QN_LAUNCH("prologue_kernel", st, prologue_kernel<T>, grid, dim3(256), 0, st, a, tab); break;
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
                           const uint16_t* x, uint16_t* y, float* ws_part, hipStream_t st) {
    // slices of A x: at most 16, and nparts * r <= 1024 partials in all
    const int nb64 = static_cast<int>(d_in / 64);
    const int want = std::max(1, std::min({kAxMaxParts, nb64, 1024 / r}));
    const int per = (nb64 + want - 1) / want;
    const int nparts = (nb64 + per - 1) / per;   // <= want
    QN_LAUNCH("lora_ax_partial_kernel", st, lora_ax_partial_kernel, dim3(nparts), dim3(256), 0, st, A,
              static_cast<int>(d_in), x, r, per, ws_part);
    const dim3 grid(static_cast<unsigned>((d_out + kGvWaves - 1) / kGvWaves));
    if ((d_in / 64) % 16 == 0) {
        QN_LAUNCH("gemv_nf4_kernel", st, gemv_nf4_kernel<true>, grid, dim3(64 * kGvWaves), 0, st,
                  reinterpret_cast<const uint4*>(codes), qconst, qscale, qmean, static_cast<int>(d_out),
                  static_cast<int>(d_in), x, B, r, s, ws_part, nparts, y, tables());
    } else {
        QN_LAUNCH("gemv_nf4_kernel", st, gemv_nf4_kernel<false>, grid, dim3(64 * kGvWaves), 0, st,
                  reinterpret_cast<const uint4*>(codes), qconst, qscale, qmean, static_cast<int>(d_out),
                  static_cast<int>(d_in), x, B, r, s, ws_part, nparts, y, tables());
    }
    return hipGetLastError();
}

}  // namespace qn
