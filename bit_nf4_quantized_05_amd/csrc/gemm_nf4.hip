// Forward product with the NF4 weight dequantised inside the GEMM (learn.ifs.name deck,
// card 1: the stored 4-bit weights are turned into BF16 each time they are used in a
// matrix product; QLoRA's doubleDequant gives the values). C[M, N] = X[M, K] W_hat[N, K]^T
// + s (X A^T)[M, r] B[N, r]^T, with M = tokens, as gemm_nt does for operands that are
// already in memory, except that W_hat is never written: each K-step's 256 x 64 weight
// tile is formed in LDS from the 8 KB of codes it comes from.
//
// Same tile (256 x 256, 8 waves of 128 x 64, v_mfma_f32_32x32x16_bf16, K-steps of 64,
// double-buffered, X tiles by buffer_load ... lds) and the same raster and split rules
// as gemm_nt. Differences:
//   - LDS (160 KB): the P (X) and Q (W_hat) tiles of the two stages are four distinct
//     objects, so the direct loads into a stage's P tile and the dequantised writes into
//     its Q tile never have to wait for one another; two code areas; the lanes' tables.
//   - Thread t owns weights 32 h .. 32 h + 31 (h = t % 2) of tile row t / 2 of every Q
//     tile. The 16 bytes of codes it needs for main K-step j go straight to code area
//     stage(j) two steps ahead, the block's 8-bit constant and group scale to registers.
//     After step j - 2's barrier it forms the block's 16 values bf16(code[e] * a_hat)
//     (a_hat = mu + scale * r_hat, the dequantiser's float32 operations) in a table of
//     its own, entry e of lane l at halfword 64 e + l of its wave's 2 KB, so two lanes
//     can only collide when they share a bank pair. During step j - 1 it looks its 32
//     weights up there, 8 per sub-step, and stores them into stage(j)'s Q tile as 16-byte
//     chunks (chunk c of tile row r at c ^ ((r >> 1) & 7), the layout the direct loads
//     give), between the MFMAs of that sub-step.
//   - The last main step and the LoRA steps (B by direct loads into the Q tile) run
//     after the dequantising steps, so that stores into a Q tile never meet direct loads
//     into it. Step 0 starts on stage (kmain - 1) % 2, which puts these on stage 0.
#include <hip/hip_runtime.h>

#include "gemm_common.h"
#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

namespace qn {
namespace {

__shared__ uint4 g_fp0[kChunks];
__shared__ uint4 g_fp1[kChunks];
__shared__ uint4 g_fq0[kChunks];
__shared__ uint4 g_fq1[kChunks];
__shared__ uint4 g_fc0[512];
__shared__ uint4 g_fc1[512];
__shared__ uint16_t g_ft[8 * 1024];

#define FP(S) ((S) ? g_fp1 : g_fp0)
#define FQ(S) ((S) ? g_fq1 : g_fq0)
#define FC(S) ((S) ? g_fc1 : g_fc0)

template <int WM, int WN, bool kSplit>
__device__ __forceinline__ void gemm_nf4_body(const GemmArgs& g) {
    constexpr int NW = WM * WN;                 // waves
    constexpr int NT = 64 * NW;                 // threads
    constexpr int TM = BM / WM / 32;            // m sub-tiles per wave
    constexpr int TN = BN / WN / 32;            // n sub-tiles per wave
    constexpr int SEG = BM / NW / 8;            // 8-row load segments per wave and operand
    static_assert(NT == 2 * BN, "two threads per Q tile row");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int M = g.M, N = g.N;

    // ---- tile assignment (as gemm_nt)
    const int bid = static_cast<int>(blockIdx.x);
    const bool split_wg = kSplit && bid >= g.full;
    const int T = kSplit ? g.full : g.tiles_m * g.tiles_n;
    const int w = split_wg ? 0 : bid;
    const int sj = split_wg ? bid - g.full : 0;
    const int sk = split_wg ? sj / g.rem : 0;
    const int logical = split_wg ? g.full + sj % g.rem : ((T % 8 == 0) ? (w & 7) * (T >> 3) + (w >> 3) : w);
    int tm, tn;
    tile_coords(g, logical, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- direct loads (as gemm_nt): lane i of a 1 KB segment lands at row i / 8,
    // position i % 8, and fetches chunk (i % 8) ^ ((r >> 1) & 7) of its row
    const uint32_t kcE = static_cast<uint32_t>((lane & 7) ^ (lane >> 4)) * 16u;
    const uint32_t kcO = static_cast<uint32_t>((lane & 7) ^ (4 | (lane >> 4))) * 16u;
    uint32_t voP[SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        const int rr = 8 * SEG * wave + 8 * j + (lane >> 3);
        const uint32_t kc16 = (((SEG * wave + j) & 1) ? kcO : kcE);
        voP[j] = static_cast<uint32_t>(min(m0 + rr, M - 1)) * static_cast<uint32_t>(g.ldp * 2) + kc16;
    }
    const __amdgpu_buffer_rsrc_t rsP = make_rsrc(g.P, g.bytesP);
    const __amdgpu_buffer_rsrc_t rsP2 = make_rsrc(g.P2, g.bytesP2);
    const __amdgpu_buffer_rsrc_t rsQ2 = make_rsrc(g.Q2, g.bytesQ2);
    const int kb = split_wg ? sk * g.kper : 0;
    const int ke = split_wg ? min(kb + g.kper, g.kt1) : g.kt1;
    const bool lora = !split_wg || sk == g.splits - 1;
    const int KT = (ke - kb) + (lora ? g.kt2 : 0);
    const int kshift = kb;                      // global main step = local + kshift
    const int kmain = ke - kb;                  // >= 1 on every path

    // main step KL's X tile into stage S
#define NF_ISSUE_MAIN(KL, S)                                                                      \
    {                                                                                             \
        uint4* sp_ = FP(S) + wave * (64 * SEG);                                                   \
        const int so_ = ((KL) + kshift) * (BK * 2);                                               \
        _Pragma("unroll") for (int j = 0; j < SEG; ++j)                                           \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP, (lds_ptr_t)(sp_ + 64 * j), 16, voP[j], so_, 0, 0); \
    }
    // LoRA step KL (>= kmain): (s X A^T) into P, B into Q. The offsets are formed here from
    // an opaque copy of the lane index, so they hold no registers through the main steps.
#define NF_ISSUE_LORA(KL, S)                                                                      \
    {                                                                                             \
        uint4* sp_ = FP(S) + wave * (64 * SEG);                                                   \
        uint4* sq_ = FQ(S) + wave * (64 * SEG);                                                   \
        const int so_ = ((KL) - kmain) * (BK * 2);                                                \
        int ln_ = lane;                                                                           \
        asm volatile("" : "+v"(ln_));                                                             \
        const uint32_t e_ = static_cast<uint32_t>((ln_ & 7) ^ (ln_ >> 4)) * 16u;                  \
        const uint32_t o_ = static_cast<uint32_t>((ln_ & 7) ^ (4 | (ln_ >> 4))) * 16u;            \
        _Pragma("unroll") for (int j = 0; j < SEG; ++j) {                                         \
            const int rr_ = 8 * SEG * wave + 8 * j + (ln_ >> 3);                                  \
            const uint32_t kc_ = ((SEG * wave + j) & 1) ? o_ : e_;                                \
            const uint32_t p_ = static_cast<uint32_t>(min(m0 + rr_, M - 1)) * static_cast<uint32_t>(g.ldp2 * 2) + kc_; \
            const uint32_t q_ = static_cast<uint32_t>(min(n0 + rr_, N - 1)) * static_cast<uint32_t>(g.ldq2 * 2) + kc_; \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsP2, (lds_ptr_t)(sp_ + 64 * j), 16, p_, so_, 0, 0); \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsQ2, (lds_ptr_t)(sq_ + 64 * j), 16, q_, so_, 0, 0); \
        }                                                                                         \
    }

    // ---- dequantisation state
    const int drow = tid >> 1, dh = tid & 1;
    const uint32_t dblk0 = static_cast<uint32_t>(min(n0 + drow, N - 1)) * static_cast<uint32_t>(g.kt1);
    const uint32_t dq_vo = dblk0 * 32u + 16u * static_cast<uint32_t>(dh);
    const __amdgpu_buffer_rsrc_t rsC = make_rsrc(g.codes, g.bytesC);
    const __amdgpu_buffer_rsrc_t rsBq = make_rsrc(g.bc.q, g.bytesBq);
    const __amdgpu_buffer_rsrc_t rsBs = make_rsrc(g.bc.scale, g.bytesBs);
    const float dq_mu = g.bc.mean[0];
    uint16_t* const dq_tp = g_ft + wave * 1024 + lane;      // the lane's entry 0
    // tile row r's chunk c sits at 8 r + ((4 h + c) ^ ((r >> 1) & 7)) = dq_qi ^ c
    const uint32_t dq_qi = static_cast<uint32_t>(drow * 8 + ((4 * dh) ^ ((drow >> 1) & 7)));
    uint32_t dq_q = 0, dq_s = 0;          // constants of the block whose table comes next
    uint32_t dq_a[8];                     // code indices, then table entries, of one chunk
    // codes of global main step KG into code area CB, its constants into QV, SV
#define NF_DQ_LOADS(KG, CB, QV, SV)                                                               \
    {                                                                                             \
        const uint32_t kg_ = static_cast<uint32_t>(KG);                                          \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsC, (lds_ptr_t)((CB) + 64 * wave), 16, dq_vo,   \
                                                 kg_ * 32u, 0, 0);                                \
        QV = __builtin_amdgcn_raw_buffer_load_b8(rsBq, dblk0 + kg_, 0, 0);                        \
        SV = __builtin_amdgcn_raw_buffer_load_b32(rsBs, ((dblk0 + kg_) >> g.bc.gshift) * 4u, 0, 0); \
    }
    // the lane's table for the block whose constants are QV, SV
#define NF_DQ_TABLE(QV, SV)                                                                       \
    {                                                                                             \
        const float ah_ = block_constant_nb(g.bc.fmt, static_cast<int8_t>(QV), __uint_as_float(SV), dq_mu); \
        _Pragma("unroll") for (int e = 0; e < 16; e += 2) {                                       \
            const uint32_t p_ = pack_bf16x2(g.code[e] * ah_, g.code[e + 1] * ah_);                \
            dq_tp[e * 64] = static_cast<uint16_t>(p_);                                            \
            dq_tp[(e + 1) * 64] = static_cast<uint16_t>(p_ >> 16);                                \
        }                                                                                         \
    }
#define NF_DQ_WORD(CB, C) reinterpret_cast<const uint32_t*>(CB)[4 * tid + (C)]
    // the 8 code indices of code word W (low nibble first), then their table entries
#define NF_DQ_ADDR(W) _Pragma("unroll") for (int i = 0; i < 8; ++i) dq_a[i] = __builtin_amdgcn_ubfe((W), 4 * i, 4);
#define NF_DQ_LOOKUP() _Pragma("unroll") for (int i = 0; i < 8; ++i) dq_a[i] = dq_tp[dq_a[i] << 6];
    // the looked-up chunk C into the Q tile of stage S
#define NF_DQ_STORE(S, C)                                                                         \
    {                                                                                             \
        uint32_t qi_ = dq_qi;                                                                     \
        asm volatile("" : "+v"(qi_));                                                             \
        FQ(S)[qi_ ^ (C)] = uint4{dq_a[0] | (dq_a[1] << 16), dq_a[2] | (dq_a[3] << 16),            \
                                 dq_a[4] | (dq_a[5] << 16), dq_a[6] | (dq_a[7] << 16)};           \
    }

    // ---- fragments: 32-row x 16-K reads per k16 sub-step kk (0..3); the row indices
    // come from an opaque copy each sub-step (chunk kk of a row is chs0 ^ 2 kk), two VALU
    // per base instead of address registers held through the loop
    const uint32_t frow = lane & 31;
    const uint32_t fsw = (frow >> 1) & 7;
    const uint32_t chs0 = (lane >> 5) ^ fsw;
    const uint32_t prow = (wm * (TM * 32) + frow) * 8 + chs0;
    const uint32_t qrow = (wn * (TN * 32) + frow) * 8 + chs0;
#define NF_FRAGS(S, KK, F)                                                                        \
    {                                                                                             \
        uint32_t ip_ = prow, iq_ = qrow;                                                          \
        asm volatile("" : "+v"(ip_), "+v"(iq_));                                                  \
        ip_ ^= 2u * (KK);                                                                         \
        iq_ ^= 2u * (KK);                                                                         \
        F[0] = FQ(S)[iq_];                                                                        \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) F[TN + i] = FP(S)[ip_ + i * 256];          \
        _Pragma("unroll") for (int i = 1; i < TN; ++i) F[i] = FQ(S)[iq_ + i * 256];               \
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = f32x16{};
#define NF_MFMAS(F)                                                                               \
    _Pragma("unroll") for (int a = 0; a < TN; ++a)                                                \
        _Pragma("unroll") for (int b = 0; b < TM; ++b)                                            \
            acc[a][b] = mfma32(F[a], F[TN + b], acc[a][b]);

    uint4 fa[TM + TN], fb[TM + TN];
    // One pre-barrier sub-step of a dequantising step on stage S: MFMAs on FO while the
    // next fragments go to FN; chunk C (its indices formed before) is looked up and
    // stored into stage 1 - S, and chunk C + 1's indices formed.
#define NF_SUB_DQ(S, KK, FN, FO, C)                                                               \
    {                                                                                             \
        const uint32_t w_ = NF_DQ_WORD(FC(1 - (S)), (C) + 1);                                     \
        NF_FRAGS(S, KK, FN)                                                                       \
        NF_DQ_LOOKUP()                                                                            \
        NF_MFMAS(FO)                                                                              \
        NF_DQ_STORE(1 - (S), C)                                                                   \
        NF_DQ_ADDR(w_)                                                                            \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                                         \
        __builtin_amdgcn_sched_barrier(0);                                                        \
    }
    // Dequantising step k (< kmain - 1) on stage S: step k + 1's X tile and step k + 2's
    // codes and constants are fetched, step k + 1's Q tile formed in stage 1 - S; after
    // the barrier the table for step k + 2 and its chunk-0 indices.
#define NF_STEP_DQ(KTV, S)                                                                        \
    {                                                                                             \
        const int k_ = (KTV);                                                                     \
        NF_ISSUE_MAIN(k_ + 1, 1 - (S))                                                            \
        NF_DQ_LOADS(kshift + min(k_ + 2, kmain - 1), FC(S), dq_q, dq_s)                           \
        __builtin_amdgcn_sched_barrier(0);                                                        \
        __builtin_amdgcn_s_setprio(1);                                                            \
        NF_SUB_DQ(S, 1, fb, fa, 0)                                                                \
        NF_SUB_DQ(S, 2, fa, fb, 1)                                                                \
        NF_SUB_DQ(S, 3, fb, fa, 2)                                                                \
        NF_DQ_LOOKUP()                                                                            \
        NF_DQ_STORE(1 - (S), 3)                                                                   \
        __builtin_amdgcn_s_setprio(0);                                                            \
        __builtin_amdgcn_s_waitcnt(0);                                                            \
        QN_BARRIER();                                                                             \
        NF_FRAGS(1 - (S), 0, fa)                                                                  \
        {                                                                                         \
            const uint32_t w0_ = NF_DQ_WORD(FC(S), 0);                                            \
            NF_MFMAS(fb)                                                                          \
            NF_DQ_TABLE(dq_q, dq_s)                                                               \
            NF_DQ_ADDR(w0_)                                                                       \
        }                                                                                         \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                                         \
    }
    // Step k (the last main step, or a LoRA step) on stage S, as in gemm_nt. Both kinds of
    // step raise the wave's issue priority for their pre-barrier sub-steps, as gemm_nt does.
#define NF_STEP(KTV, S)                                                                           \
    {                                                                                             \
        const int k_ = (KTV);                                                                     \
        if (k_ + 1 < KT) NF_ISSUE_LORA(k_ + 1, 1 - (S))                                           \
        NF_FRAGS(S, 1, fb)                                                                        \
        __builtin_amdgcn_s_setprio(1);                                                            \
        NF_MFMAS(fa)                                                                              \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                                         \
        NF_FRAGS(S, 2, fa)                                                                        \
        NF_MFMAS(fb)                                                                              \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                                         \
        NF_FRAGS(S, 3, fb)                                                                        \
        NF_MFMAS(fa)                                                                              \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                                         \
        __builtin_amdgcn_s_setprio(0);                                                            \
        __builtin_amdgcn_s_waitcnt(0);                                                            \
        QN_BARRIER();                                                                             \
        if (k_ + 1 < KT) NF_FRAGS(1 - (S), 0, fa)                                                 \
        NF_MFMAS(fb)                                                                              \
        QN_INTERLEAVE_DS_MFMA((TM + TN));                                                         \
    }
    // Stage S receives step 0: its X tile, codes and table, and chunk-0 indices of step 1.
#define NF_PROLOGUE(S)                                                                            \
    {                                                                                             \
        uint32_t q0_, s0_;                                                                        \
        NF_DQ_LOADS(kshift, FC(S), q0_, s0_)                                                      \
        NF_ISSUE_MAIN(0, S)                                                                       \
        NF_DQ_LOADS(kshift + min(1, kmain - 1), FC(1 - (S)), dq_q, dq_s)                          \
        QN_WAIT_VM(0);                                                                            \
        NF_DQ_TABLE(q0_, s0_)                                                                     \
        _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                           \
            NF_DQ_ADDR(NF_DQ_WORD(FC(S), c))                                                      \
            NF_DQ_LOOKUP()                                                                        \
            NF_DQ_STORE(S, c)                                                                     \
        }                                                                                         \
        NF_DQ_TABLE(dq_q, dq_s)                                                                   \
        NF_DQ_ADDR(NF_DQ_WORD(FC(1 - (S)), 0))                                                    \
        __builtin_amdgcn_s_waitcnt(0);                                                            \
        QN_BARRIER();                                                                             \
        NF_FRAGS(S, 0, fa)                                                                        \
    }

    const int D = kmain - 1;                    // dequantising steps
    int kt = 0;
    if (D & 1) {
        NF_PROLOGUE(1)
        NF_STEP_DQ(0, 1)
        kt = 1;
    } else {
        NF_PROLOGUE(0)
    }
    for (; kt + 2 <= D; kt += 2) {
        NF_STEP_DQ(kt, 0)
        NF_STEP_DQ(kt + 1, 1)
    }
    for (; kt + 2 <= KT; kt += 2) {
        NF_STEP(kt, 0)
        NF_STEP(kt + 1, 1)
    }
    if (kt < KT) NF_STEP(kt, 0)
#undef NF_PROLOGUE
#undef NF_STEP
#undef NF_STEP_DQ
#undef NF_SUB_DQ
#undef NF_MFMAS
#undef NF_FRAGS
#undef NF_DQ_STORE
#undef NF_DQ_LOOKUP
#undef NF_DQ_ADDR
#undef NF_DQ_WORD
#undef NF_DQ_TABLE
#undef NF_DQ_LOADS
#undef NF_ISSUE_LORA
#undef NF_ISSUE_MAIN

    // Tile row rl of the 256 x 256 output, staged in LDS for the epilogue: rows
    // 64 q .. 64 q + 63 in the q-th of the four 32 KB tiles
    auto stage_row = [](int rl) -> char* {
        uint4* arr = (rl >> 7) ? ((rl >> 6) & 1 ? g_fq1 : g_fq0) : ((rl >> 6) & 1 ? g_fp1 : g_fp0);
        return reinterpret_cast<char*>(arr) + (rl & 63) * 512;
    };
    if (split_wg) {
        // fp32 partial tile of this split, compact 256 x 256 (as gemm_nt)
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
    // ---- epilogue (as gemm_nt): every wave is past the last barrier and no load is in
    // flight, so the LDS tiles are free; the bf16 C tile goes to LDS with 16-byte chunk j
    // of row r at j ^ (r & 31), then each row leaves as 512 contiguous bytes
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const int rl = wm * (TM * 32) + b * 32 + static_cast<int>(frow);
        char* rowp = stage_row(rl);
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
    const int cj = tid & 31;
    constexpr int kRowsPerPass = NT / 32;
#pragma unroll
    for (int i = 0; i < BM / kRowsPerPass; ++i) {
        const int r = i * kRowsPerPass + (tid >> 5);
        const uint4 v = *reinterpret_cast<const uint4*>(stage_row(r) + ((cj ^ (r & 31)) << 4));
        const int m = m0 + r;
        const int n = n0 + cj * 8;
        if (m < M && n < N) *reinterpret_cast<uint4*>(g.C + static_cast<int64_t>(m) * g.ldc + n) = v;
    }
}

#undef FP
#undef FQ
#undef FC

constexpr int kNfWM = 2, kNfWN = 4;

__global__ __launch_bounds__(64 * kNfWM * kNfWN, 1)
void gemm_nf4_kernel(GemmArgs g) {
    gemm_nf4_body<kNfWM, kNfWN, false>(g);
}

__global__ __launch_bounds__(64 * kNfWM * kNfWN, 1)
void gemm_nf4_split(GemmArgs g) {
    gemm_nf4_body<kNfWM, kNfWN, true>(g);
}

}  // namespace

hipError_t launch_gemm_nf4_body(const GemmArgs& g, bool split, hipStream_t st) {
    if (split)
        QN_LAUNCH("gemm_nf4_split", st, gemm_nf4_split, dim3(g.full + g.rem * g.splits), dim3(64 * kNfWM * kNfWN), 0,
                  st, g);
    else
        QN_LAUNCH("gemm_nf4_kernel", st, gemm_nf4_kernel, dim3(g.tiles_m * g.tiles_n), dim3(64 * kNfWM * kNfWN), 0,
                  st, g);
    return hipGetLastError();
}

}  // namespace qn
