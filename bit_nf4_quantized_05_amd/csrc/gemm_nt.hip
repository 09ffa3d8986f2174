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
//
// gemm_nt_split: the same body when the last round of tiles would leave most CUs idle
// (T tiles, T mod 256 <= 128): the first 256 floor(T / 256) tiles run whole, and the
// K-steps of each of the R = T mod 256 others are split over S = min(4, 256 / R)
// workgroups (the LoRA K-steps go to the last split), each writing its fp32 partial
// tile; gemm_split_reduce adds a tile's S partials in split order and rounds to bf16.
#include <hip/hip_runtime.h>

#include "gemm_common.h"
#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

#include <algorithm>

namespace qn {
namespace {

// ---------------------------------------------------------------------------
// Main NT GEMM
// ---------------------------------------------------------------------------
// Two LDS stages as distinct objects, so the compiler can tell that reads of one
// stage do not depend on in-flight direct-to-LDS loads into the other. Each holds
// [P tile | Q tile] = 2 x 2048 chunks = 64 KB.
__shared__ uint4 g_st0[2 * kChunks];
__shared__ uint4 g_st1[2 * kChunks];

// WM x WN waves; each wave owns a (256/WM) x (256/WN) sub-tile of 32x32 MFMA tiles.
template <int WM, int WN, bool kSplit>
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

    // ---- tile assignment: contiguous logical ranges per XCD, grouped raster. On the
    // split path, workgroups [0, full) take whole tiles, the rest (tile full + j % rem,
    // split j / rem) the split ones.
    const int bid = static_cast<int>(blockIdx.x);
    const bool split_wg = kSplit && bid >= g.full;
    const int T = kSplit ? g.full : g.tiles_m * g.tiles_n;
    const int w = split_wg ? 0 : bid;
    const int sj = split_wg ? bid - g.full : 0;
    const int sk = split_wg ? sj / g.rem : 0;                          // split of this workgroup
    const int logical = split_wg ? g.full + sj % g.rem : ((T % 8 == 0) ? (w & 7) * (T >> 3) + (w >> 3) : w);
    int tm, tn;
    tile_coords(g, logical, tm, tn);
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
    // K-steps of this workgroup: main steps [kb, ke) of P Q^T, then (last split, or no
    // split) the kt2 LoRA steps; step k of the loop is global step kb + k while k < ke - kb
    const int kb = split_wg ? sk * g.kper : 0;
    const int ke = split_wg ? min(kb + g.kper, g.kt1) : g.kt1;
    const bool lora = !split_wg || sk == g.splits - 1;
    const int KT = (ke - kb) + (lora ? g.kt2 : 0);
    const int kshift = kb;                      // global main step = local + kshift
    const int kmain = ke - kb;

#define QN_ISSUE(KTV, ST)                                                                         \
    {                                                                                             \
        const int kl_ = (KTV);                                                                    \
        uint4* sp_ = (ST) + wave * (64 * SEG);                                                    \
        uint4* sq_ = sp_ + kChunks;                                                               \
        if (kl_ < kmain) {                                                                        \
            const int so_ = (kl_ + kshift) * (BK * 2);                                            \
            _Pragma("unroll") for (int j = 0; j < SEG; ++j) {                                     \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP, (lds_ptr_t)(sp_ + 64 * j), 16, voP[j], so_, 0, 0); \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQ, (lds_ptr_t)(sq_ + 64 * j), 16, voQ[j], so_, 0, 0); \
            }                                                                                     \
        } else {                                                                                  \
            const int so_ = (kl_ - kmain) * (BK * 2);                                             \
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
    // A wave runs its first three sub-steps at raised issue priority and drops it for
    // the barrier, the next step's loads and the sub-step after the barrier, so the
    // waves of a SIMD that are still in their MFMA run go first (2-4 % faster on the
    // 4096^2 layer than equal priority; the results do not change).
#define QN_STEP(KTV, CUR, NXT)                                                 \
    {                                                                          \
        const int k_ = (KTV);                                                  \
        if (k_ + 1 < KT) QN_ISSUE(k_ + 1, NXT)                                 \
        QN_FRAGS(CUR, chs[1], fb)                                              \
        __builtin_amdgcn_s_setprio(1);                                         \
        QN_MFMAS(fa)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
        QN_FRAGS(CUR, chs[2], fa)                                              \
        QN_MFMAS(fb)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
        QN_FRAGS(CUR, chs[3], fb)                                              \
        QN_MFMAS(fa)                                                           \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                      \
        __builtin_amdgcn_s_setprio(0);                                         \
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

    if (split_wg) {
        // fp32 partial tile of this split, compact 256 x 256: the lane's 4 consecutive n
        // of tile row ml as 16 bytes
        float* pt = g.part + (static_cast<int64_t>(sk) * g.rem + sj % g.rem) * (BM * BN);
#pragma unroll
        for (int b = 0; b < TM; ++b) {
            const int ml = wm * (TM * 32) + b * 32 + static_cast<int>(frow);
#pragma unroll
            for (int a = 0; a < TN; ++a) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int nl = wn * (TN * 32) + a * 32 + 8 * gq + 4 * (lane >> 5);
                    *reinterpret_cast<float4*>(pt + ml * BN + nl) =
                        float4{acc[a][b][4 * gq], acc[a][b][4 * gq + 1], acc[a][b][4 * gq + 2], acc[a][b][4 * gq + 3]};
                }
            }
        }
        return;
    }
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
    gemm_nt_body<kGemmWM, kGemmWN, false>(g);
}

__global__ __launch_bounds__(64 * kGemmWM * kGemmWN, 1)
void gemm_nt_split(GemmArgs g) {
    gemm_nt_body<kGemmWM, kGemmWN, true>(g);
}

// Split tiles: C[m, n..n+3] = bf16(sum of the tile's partials in split order), 4 outputs
// per thread; 64 workgroups per tile (4 rows each). SP = the split count (2..4): that
// many partial loads per thread.
template <int SP>
__global__ __launch_bounds__(256)
void gemm_split_reduce(GemmArgs g) {
    const int j = static_cast<int>(blockIdx.x) / 64;                  // split tile
    const int ml = (static_cast<int>(blockIdx.x) % 64) * 4 + (threadIdx.x >> 6);
    const int nl = (threadIdx.x & 63) * 4;
    int tm, tn;
    tile_coords(g, g.full + j, tm, tn);
    const int m = tm * BM + ml, n = tn * BN + nl;
    if (m >= g.M || n >= g.N) return;
    const float* p = g.part + static_cast<int64_t>(j) * (BM * BN) + ml * BN + nl;
    const int64_t stride = static_cast<int64_t>(g.rem) * (BM * BN);
    float4 v[SP];
#pragma unroll
    for (int s = 0; s < SP; ++s) v[s] = *reinterpret_cast<const float4*>(p + s * stride);
    float4 t = v[0];
#pragma unroll
    for (int s = 1; s < SP; ++s) { t.x += v[s].x; t.y += v[s].y; t.z += v[s].z; t.w += v[s].w; }
    *reinterpret_cast<uint2*>(g.C + static_cast<int64_t>(m) * g.ldc + n) =
        uint2{pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w)};
}

}  // namespace

GemmSplit gemm_split(int64_t M, int64_t N, int64_t K1) {
    const int64_t T = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t rem = T % 256;
    GemmSplit gs{1, static_cast<int>(T), 0};
    if (rem == 0 || rem > 128) return gs;
    const int64_t s = std::min<int64_t>({4, 256 / rem, K1 / BK / 8});    // at least 8 K-steps per split
    if (s < 2) return gs;
    gs.splits = static_cast<int>(s);
    gs.full = static_cast<int>(T - rem);
    gs.rem = static_cast<int>(rem);
    return gs;
}

int64_t gemm_split_part_floats(int64_t M, int64_t N, int64_t K1) {
    const GemmSplit gs = gemm_split(M, N, K1);
    return gs.splits > 1 ? static_cast<int64_t>(gs.splits) * gs.rem * BM * BN : 0;
}

hipError_t launch_gemm_nt(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, int64_t K1,
                          const uint16_t* P2, int64_t ldp2, const uint16_t* Q2, int64_t ldq2,
                          int64_t K2, uint16_t* C, int64_t ldc, int64_t M, int64_t N, float* part,
                          hipStream_t st, const uint8_t* codes, const BlockConsts* bc) {
    GemmArgs g;
    const bool deq = codes != nullptr;              // Q = W_hat formed from the codes in the kernel
    g.codes = codes;
    g.bc = deq ? *bc : BlockConsts{nullptr, nullptr, nullptr, 0, 0};
    {
        const NF4Tables& tab = tables();
        for (int i = 0; i < 16; ++i) g.code[i] = tab.code[i];
    }
    const int64_t nblk = deq ? N * (K1 / BK) : 0;   // NF4 blocks of the weight (K1 % 64 == 0)
    g.bytesC = static_cast<uint32_t>(nblk * 32);
    g.bytesBq = static_cast<uint32_t>(nblk);
    g.bytesBs = static_cast<uint32_t>(deq ? 4 * (((nblk - 1) >> g.bc.gshift) + 1) : 0);
    if (deq) { Q = P; ldq = ldp; }                  // no bf16 weight operand
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
    const GemmSplit gs = gemm_split(M, N, K1);
    g.splits = gs.splits;
    g.full = gs.full;
    g.rem = gs.rem;
    g.kper = (g.kt1 + g.splits - 1) / g.splits;
    g.part = part;
    if (g.splits <= 1 || part == nullptr) {
        g.splits = 1;
        if (deq) return launch_gemm_nf4_body(g, false, st);
        QN_LAUNCH("gemm_nt_kernel", st, gemm_nt_kernel, dim3(g.tiles_m * g.tiles_n), dim3(64 * kGemmWM * kGemmWN), 0,
                  st, g);
        return hipGetLastError();
    }
    if (deq) {
        const hipError_t e = launch_gemm_nf4_body(g, true, st);
        if (e != hipSuccess) return e;
    } else {
        QN_LAUNCH("gemm_nt_split", st, gemm_nt_split, dim3(g.full + g.rem * g.splits), dim3(64 * kGemmWM * kGemmWN),
                  0, st, g);
    }
    const dim3 rgrid(static_cast<unsigned>(g.rem * 64));
    if (g.splits == 2) QN_LAUNCH("gemm_split_reduce", st, gemm_split_reduce<2>, rgrid, dim3(256), 0, st, g);
    else if (g.splits == 3) QN_LAUNCH("gemm_split_reduce", st, gemm_split_reduce<3>, rgrid, dim3(256), 0, st, g);
    else QN_LAUNCH("gemm_split_reduce", st, gemm_split_reduce<4>, rgrid, dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace qn
