// d_seq = 1 forward (decode) of the QLoRA linear layer on gfx950: a streaming GEMV
// over the packed NF4 codes with the rank-r LoRA term.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

#include <algorithm>
#include <atomic>

namespace qn {
namespace {

// ---------------------------------------------------------------------------
// d_seq = 1 (decode), and 2 or 3 tokens. When all of A fits one 4096-column segment
// with r <= 16 (A <= 128 KB, read from L2 by every workgroup), one launch: each
// gemv_nf4 workgroup forms s A x itself, wave j the dot product of row j of A with the
// x segment (of each token) it has staged in LDS anyway. Otherwise the 64-column
// blocks of x are split into nparts contiguous slices (nparts * tokens * r <= 1024),
// and the slice partial of every token t and rank row j (the dot product of A[j] and
// x_t over the slice, fixed summation order) is formed
//   - for one token on the persistent GEMV: inside the same launch, slice p by its
//     workgroup p, published as 64-bit (value, tag) words that the other workgroups
//     wait for (bounded, then forming the slices themselves);
//   - otherwise by lora_ax_partial, launched first, into part[w][t][j].
// gemv_nf4 / gemv_nf4_persist stream the packed codes once and add B (s A x), summing
// the slice partials in slice order: y = W_hat x + B (s A x). Every path is
// deterministic and forms the same s A x bits.
// ---------------------------------------------------------------------------
constexpr int kAxMaxParts = 16;

// The A x slice of 64-column blocks [b_lo, b_hi): thread tid < 256 (of a workgroup of
// 256 or more) accumulates, for rank row j = tid % r, the blocks b_lo + tid / r,
// + 256 / r, ... of every token (x rows at stride ldx) in a fixed order; the slice sum
// of row j is then ax_slice_sum over the 256 / r threads of row j, in thread order.
// The slice kernel and the persistent GEMV's in-launch slices both run these two
// functions, so they form the same bits.
template <int T>
__device__ __forceinline__ void ax_slice_acc(const uint16_t* __restrict__ A, int d_in, const uint16_t* __restrict__ x,
                                             int64_t ldx, int r, int b_lo, int b_hi, int tid, float (&acc)[T]) {
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0f;
    const int groups = 256 / r;                   // threads per rank row
    if (tid < groups * r) {
        const int j = tid % r;
        for (int b = b_lo + tid / r; b < b_hi; b += groups) {
            const uint4* ar = reinterpret_cast<const uint4*>(A + static_cast<int64_t>(j) * d_in + b * 64);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint4* xr = reinterpret_cast<const uint4*>(x + t * ldx + static_cast<int64_t>(b) * 64);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint4 av = ar[e], xv = xr[e];
                    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
                    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[q]),
                                                                 __builtin_bit_cast(bf16x2, xw[q]), acc[t], false);
                }
            }
        }
    }
}

// red = the 256 accumulators of one token (LDS); rank row j < r
__device__ __forceinline__ float ax_slice_sum(const float* red, int r, int j) {
    float v = 0.0f;
    for (int g = 0; g < 256 / r; ++g) v += red[g * r + j];
    return v;
}

// T tokens (rows of x at stride ldx): part[(w T + t) r + j] (the one-token layout for T = 1)
template <int T>
__global__ __launch_bounds__(256)
void lora_ax_partial_kernel(const uint16_t* __restrict__ A, int d_in, const uint16_t* __restrict__ x,
                            int64_t ldx, int r, int blocks_per_part, float* __restrict__ part) {
    __shared__ float red[T][256];
    const int tid = threadIdx.x;
    const int nb64 = d_in / 64;
    const int b_lo = blockIdx.x * blocks_per_part;
    const int b_hi = min(b_lo + blocks_per_part, nb64);
    float acc[T];
    ax_slice_acc<T>(A, d_in, x, ldx, r, b_lo, b_hi, tid, acc);
#pragma unroll
    for (int t = 0; t < T; ++t) red[t][tid] = acc[t];
    __syncthreads();
    if (tid < r) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            part[(static_cast<int64_t>(blockIdx.x) * T + t) * r + tid] = ax_slice_sum(red[t], r, tid);
    }
}

// gemv_nf4: a workgroup of 16 waves takes 16 consecutive rows, one per wave (four
// waves per SIMD hide each other's latencies). A row is walked in segments of 4096
// weights = 64 blocks; in a segment, lane l of a wave owns block l's constant and
// two chunks of 2048 weights, in each the weights [32 l, 32 l + 32) = 16 code bytes
// (one 16-byte load; the wave reads 1 KB contiguous), half of block 32 h + l/2.
// The vector-memory address unit takes about as long for a 1-byte load as for a
// 16-byte one, so what all 16 rows share is loaded once per workgroup with wide
// loads by one wave each and passed through LDS: the x segment (waves 0..7), the
// A x slice partials (waves 10..13) and the 16 rows of B (wave 14). The block
// constants are per row: lane l loads block l's 8-bit code (or a_j) and scale with
// its code words. In the one-launch form the first segment's code loads go out only
// after the first barrier (x, B and the tables in LDS): issued at once with x they
// filled the memory queues ahead of it and every wave started later (one-launch decode
// on a 4096 x 4096 layer: 7.3 -> 6.7 us median); the two-launch form, which fetches no
// A rows, issues them right behind x. The next segment's loads go out before the
// current one is computed.
// A lane forms a_hat of block l and hands it to the two lanes owning the block's
// halves by a cross-lane read. Each code byte (two weights) is looked up as a pair
// of bf16 code values and dotted with the bf16 x pair (v_dot2_f32_bf16); a_hat
// multiplies each half-block partial once (the constant factors out of the sum
// over its block). The pair table holds one copy per lane (64 KB), so a wave's
// lookups never share a bank, and the LDS address of a lookup, byte << 8 | lane << 2,
// is one v_perm_b32 of the code word and the lane offset (two ALU operations per byte
// before: extract, then shift and merge; 6.3 -> 6.0 us per 4096 x 4096 call). The x
// chunks are XOR-swizzled so the 16-byte reads of 16 lanes hit 16 distinct bank groups. s (A x) is formed before
// the weight loop, so each wave finishes on its own (formed after it, the A loads
// would have longer to land, but the call measured 7.6 against 6.9 us).
constexpr int kGvWaves = 16;
constexpr int kGvSeg = 4096;
constexpr int kLutCopies = 64;

struct GvRowSeg {
    uint4 cw[2];            // code words of the two chunks
    int8_t qv;              // second-level code of block l
    float sv;               // its group scale (a_j without a second level)
};

// LDS byte address (within the table) of the bf16 pair of byte i of code word w for
// the lane whose byte offset is lane4 = 4 lane: [0, 0, byte, lane4] by one v_perm_b32
// (selector bytes 0..3 pick bytes of w, 4 picks lane4's low byte, 12 gives zero).
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, uint32_t lane4, uint32_t i) {
    return __builtin_amdgcn_perm(lane4, w, 0x0C0C0004u | (i << 8));
}

__device__ __forceinline__ uint32_t lut_pair(const char* lut, uint32_t w, uint32_t lane4, uint32_t i) {
    return *reinterpret_cast<const uint32_t*>(lut + lut_addr(w, lane4, i));
}

__device__ __forceinline__ float gemv_half_block(const uint4 c, const uint4* xv, const char* lut, uint32_t lane4) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float part = 0.0f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        const uint32_t xw[4] = {xv[w4].x, xv[w4].y, xv[w4].z, xv[w4].w};
#pragma unroll
        for (int b = 0; b < 4; ++b)
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lut_pair(lut, cw[w4], lane4, b)),
                                                   __builtin_bit_cast(bf16x2, xw[b]), part, false);
    }
    return part;
}

// position of 16-byte x chunk c of a segment in LDS: lane l = (c >> 2) & 63 reads
// chunks 4 l .. 4 l + 3; their order is XORed with bits 2..3 of l
__device__ __forceinline__ int gv_xpos(int c) { return (c & ~3) | ((c & 3) ^ ((c >> 4) & 3)); }

// T tokens (1, 2 or 3; the ntok <= T real ones first, x rows past ntok read as zero and
// their outputs not stored): each code-pair lookup serves all T tokens. T > 1 only with
// the one-launch form (kAx); 4 tokens would need more than the 128 registers a lane has
// at 16 waves per CU.
template <int T, bool kAx>
__global__ __launch_bounds__(1024)
void gemv_nf4_kernel(const uint4* __restrict__ codes, BlockConsts bc,
                     int d_out, int d_in, const uint16_t* __restrict__ x, int ldx, int ntok,
                     const uint16_t* __restrict__ B, int r, float s, const float* __restrict__ part,
                     int nparts, const uint16_t* __restrict__ A, uint16_t* __restrict__ y, int ldy, NF4Tables tab) {
    static_assert(T == 1 || kAx, "several tokens only in the one-launch form");
    __shared__ uint4 lut4[256 * kLutCopies / 4];
    __shared__ uint4 xs[2][T][kGvSeg / 8];
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
    const int nseg = kAx ? 1 : (d_in + kGvSeg - 1) / kGvSeg;   // the one-launch form takes d_in <= kGvSeg
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    const int64_t row_u = static_cast<int64_t>(row) * upr;

    // the x segment of each token: waves 0..7, one 16-byte chunk per lane and token
    auto stage_issue = [&](uint4 (&g)[T], int S) {
        if (wave < 8) {
            const int col = S * kGvSeg + 8 * tid;
#pragma unroll
            for (int k = 0; k < T; ++k)
                g[k] = x4[(static_cast<int64_t>(min(k, ntok - 1)) * ldx + min(col, d_in - 8)) / 8];
        }
    };
    auto stage_store = [&](const uint4 (&g)[T], int S) {
        if (wave < 8) {
#pragma unroll
            for (int k = 0; k < T; ++k)
                xs[S & 1][k][gv_xpos(tid)] = S * kGvSeg + 8 * tid < d_in && k < ntok ? g[k] : uint4{0, 0, 0, 0};
        }
    };
    auto seg_issue = [&](GvRowSeg& k, int S) {
        {
            const int64_t b = static_cast<int64_t>(row) * nbpr + min(S * 64 + lane, nbpr - 1);
            k.qv = bc.q[b];
            k.sv = bc.scale[b >> bc.gshift];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = S * kGvSeg + h * 2048 + lane * 32;
            k.cw[h] = codes[row_u + (col < d_in ? col / 32 : 0)];
        }
    };

    // ---- loads: staged data first (the codes follow the first barrier)
    uint4 st[T];
#pragma unroll
    for (int k = 0; k < T; ++k) st[k] = uint4{0, 0, 0, 0};
    stage_issue(st, 0);
    const int nval = nparts * r;                  // <= 1024
    uint4 tst = uint4{0, 0, 0, 0};
    // one-launch form: wave j loads row j of A (rows past r repeat row r - 1 and are not
    // used), lane l the 16-byte chunks l + 64 e, so each load is 1 KB contiguous
    const int nch = d_in / 8;                     // 16-byte chunks of a row (d_in <= 4096)
    uint4 av[8];
    if constexpr (kAx) {
        const uint4* ar = reinterpret_cast<const uint4*>(A) + static_cast<int64_t>(min(wave, r - 1)) * nch;
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = ar[min(lane + 64 * e, nch - 1)];
    } else {
        if (wave >= 10 && wave < 14)
            tst = reinterpret_cast<const uint4*>(part)[min(tid - 640, (nval + 3) / 4 - 1)];
    }
    const int nbv = 2 * r;                        // 16-byte pieces of the 16 rows of B
    const uint4* b4 = reinterpret_cast<const uint4*>(B + static_cast<int64_t>(row0) * r);
    constexpr int kBst = kAx ? 1 : 8;             // r <= 16 in the one-launch form: one piece per lane
    uint4 bst[kBst];
#pragma unroll
    for (int i = 0; i < kBst; ++i) bst[i] = uint4{0, 0, 0, 0};
    if (wave == 14) {
#pragma unroll
        for (int i = 0; i < kBst; ++i)
            if (64 * i < nbv) bst[i] = b4[min(lane + 64 * i, nbv - 1)];
    }
    GvRowSeg g0, g1;
    // without A rows to fetch, the first segment's code loads go out right behind x (the
    // two-launch form: 4096 x 11008 16.5 -> 15.5 us per call); with them they wait for
    // the first barrier (issued behind the 128 KB of A they made the 4096 x 4096 call
    // 6.35 -> 6.94 us)
    if constexpr (!kAx) {
        seg_issue(g0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- tables and staged data to LDS; the barriers wait for LDS writes only
    {
        // code-book pairs picked from the (scalar) kernel arguments by selects (an
        // indexed read would be a memory load); thread t fills pair t / 4, copies
        // 16 (t % 4) .. + 15
        const int pr = tid >> 2;
        float lo = tab.code[0], hi = tab.code[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            lo = (pr & 15) == i ? tab.code[i] : lo;
            hi = (pr >> 4) == i ? tab.code[i] : hi;
        }
        const uint32_t v = pack_bf16x2(lo, hi);
#pragma unroll
        for (int c = 0; c < 4; ++c) lut4[pr * (kLutCopies / 4) + (tid & 3) * 4 + c] = uint4{v, v, v, v};
        if (tid < 256) qlut[tid] = dq_step(bc.fmt, static_cast<int8_t>(tid - 128));      // T[q] at q + 128
    }
    stage_store(st, 0);
    if (!kAx && wave >= 10 && wave < 14) reinterpret_cast<uint4*>(tvs)[tid - 640] = tst;
    if (wave == 14) {
#pragma unroll
        for (int i = 0; i < kBst; ++i)
            if (lane + 64 * i < nbv) bs[lane + 64 * i] = bst[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (kAx) {
        seg_issue(g0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kAx) {
        // s (A x) of rank row `wave` for each token: 8 chunk dot products per lane, then
        // a fixed xor tree; token k's entries at s_t[16 k + rank]
        // (one token at a time: the scheduling barrier keeps the x reads of the next
        // token from being hoisted, which would need 32 registers per token)
#pragma unroll
        for (int k = 0; k < T; ++k) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = lane + 64 * e;
                if (c < nch) {
                    const uint4 xv = xs[0][k][gv_xpos(c)];
                    const uint32_t aw[4] = {av[e].x, av[e].y, av[e].z, av[e].w};
                    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[q]),
                                                            __builtin_bit_cast(bf16x2, xw[q]), t, false);
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
            if (lane == 0 && wave < r) s_t[16 * k + wave] = s * t;
            if constexpr (T > 1) __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // s (A x), summed per rank row in slice order
        if (tid < r) {
            float t = 0.0f;
            for (int p = 0; p < nparts; ++p) t += tvs[p * r + tid];
            s_t[tid] = s * t;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const char* lut = reinterpret_cast<const char*>(lut4);
    const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
    const float mu = bc.mean[0];
    float acc[T];
#pragma unroll
    for (int k = 0; k < T; ++k) acc[k] = 0.0f;
    auto compute = [&](const GvRowSeg& g, int S) {
        const int kb = S & 1;
        const bool bok = S * 64 + lane < nbpr;
        const float ah = !bok ? 0.0f : bc.fmt == kDqNone ? g.sv : mu + g.sv * qlut[g.qv + 128];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float a = __shfl(ah, h * 32 + (lane >> 1));
            if constexpr (T == 1) {
                uint4 xv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[e] = xs[kb][0][h * 256 + 4 * lane + (e ^ ((lane >> 2) & 3))];
                acc[0] += a * gemv_half_block(g.cw[h], xv, lut, lane4);
            } else {
                // one code-pair lookup per byte for all tokens; per token the same dot
                // order as the single-token form
                const uint32_t cw[4] = {g.cw[h].x, g.cw[h].y, g.cw[h].z, g.cw[h].w};
                float part[T];
#pragma unroll
                for (int k = 0; k < T; ++k) part[k] = 0.0f;
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    uint4 xv[T];
#pragma unroll
                    for (int k = 0; k < T; ++k) xv[k] = xs[kb][k][h * 256 + 4 * lane + (w4 ^ ((lane >> 2) & 3))];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const bf16x2 lv = __builtin_bit_cast(bf16x2, lut_pair(lut, cw[w4], lane4, b));
#pragma unroll
                        for (int k = 0; k < T; ++k) {
                            const uint32_t xw[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
                            part[k] = __builtin_amdgcn_fdot2_f32_bf16(lv, __builtin_bit_cast(bf16x2, xw[b]), part[k],
                                                                      false);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int k = 0; k < T; ++k) acc[k] += a * part[k];
            }
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
#pragma unroll
    for (int k = 0; k < T; ++k) {
        float v = acc[k];
        for (int j = lane; j < r; j += 64) v += bf16_to_f32(brow[j]) * s_t[16 * k + j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && row0 + wave < d_out && k < ntok) y[static_cast<int64_t>(k) * ldy + row0 + wave] = bf16_bits(v);
    }
}

// ---------------------------------------------------------------------------
// gemv_nf4_persist (layers of more than 4096 rows, and one token on rows of several
// 4096-weight segments whatever their number): the same per-row work
// as gemv_nf4_kernel<1, kAx>, but one workgroup per CU walks many rows. Wave w of
// workgroup b takes rows g * 16 + w for the row groups g = b, b + grid, ...; a row is
// one unit per 4096-weight segment, and the loads of a wave's next unit (its code
// words, block constants and its row of B) go out before the current unit is computed,
// so a wave keeps two units in flight without any barrier. Every unit issues the same
// loads (B on every segment, the unit past the last one re-issued clamped, the
// block-constant select without a branch, mu by a scalar load), so the compiler waits
// for the current unit's loads only: with a load count that depended on the path, it
// had waited for all loads in flight (the next unit's too) before computing.
// x (d_in <= kGvXMax) is staged in LDS whole, once, with the tables and s (A x), which
// the one-launch form (r <= 16, d_in <= 4096) forms once per workgroup. With one token
// and larger A (kPub) the A x slices are formed in this launch: workgroup p < nparts
// starts slice p before its staging barrier and stores each sum with its word's tag + 1
// in one 64-bit agent-scope store; every thread notes at its start the tag of the word it
// gathers, and at the first row end (the same unit for every wave of a workgroup) polls
// it until the tag has advanced by one, which only this launch's producer does, so any
// prior content of the words is harmless. A wait that runs out (a producer not yet
// resident, or a word published before the tag was noted) makes the workgroup form every
// slice itself, with the same arithmetic: the outputs are the same bits in every case.
// (Against the slice kernel launched first: 11008 x 4096 and 4096 x 11008 at r = 64
// 5-7 % faster per call, 28672 x 8192 within 1 %.) Each row's
// sums run in the order of gemv_nf4_kernel, so the outputs are the same bits. With one
// workgroup of 16 rows per CU and round, the kernel above waits out a full load
// latency per round (28672 x 8192: 7 rounds, 54 us for 126 MB).
// ---------------------------------------------------------------------------
constexpr int kGvXMax = 16384;            // x held whole in LDS (32 KB), one token
constexpr int kGvXMaxT = 8192;            // the same with 2 or 3 tokens (16 KB each)
constexpr int kGvPersistWgs = 256;        // one workgroup per CU
constexpr int kAxSpin = 64;               // default polls of a published A x word before forming the slices locally
std::atomic<int> g_ax_polls{kAxSpin};

struct GvUnit {
    uint4 cw[2];            // code words of the two chunks
    int8_t qv;              // second-level code of block l
    float sv;               // its group scale (a_j without a second level)
    uint16_t bw[4];         // B[row, lane + 64 i] (clamped; used on a row's last segment, masked)
};

// T = 1, 2 or 3 tokens (x and y rows at strides ldx, ldy): each code-pair lookup serves
// every token, with per token the dot order of the one-token form; s (A x) per token
// at s_t[16 t + j] (one-launch form) or s_t[t r + j] (from the T-token slice partials).
template <int T, bool kAx, bool kPub>
__global__ __launch_bounds__(1024)
void gemv_nf4_persist(const uint4* __restrict__ codes, BlockConsts bc, int d_out, int d_in,
                      const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ B, int r, float s,
                      float* __restrict__ part, int nparts, int per, int ax_polls, const uint16_t* __restrict__ A,
                      uint16_t* __restrict__ y, int64_t ldy, NF4Tables tab) {
    constexpr int kBw = kAx ? 1 : 4;              // 64-entry pieces of a row of B (r <= 16 in the one-launch form)
    constexpr int kX = T == 1 ? kGvXMax : kGvXMaxT;
    constexpr int kXPer = kX / 8 / 1024;          // 16-byte x chunks per thread and token
    __shared__ uint4 lut4[256 * kLutCopies / 4];
    __shared__ uint4 xs[T][kX / 8];
    __shared__ float tvs[1024];
    __shared__ float qlut[256];
    __shared__ float s_t[T * 256];
    __shared__ float red[kPub ? T : 1][256];
    __shared__ int ax_late;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbpr = d_in / 64;
    const int upr = d_in / 32;
    const int nseg = (d_in + kGvSeg - 1) / kGvSeg;
    const int nch = d_in / 8;
    const int ngroups = (d_out + kGvWaves - 1) / kGvWaves;
    const int grid = static_cast<int>(gridDim.x);
    const int my_groups = (ngroups - static_cast<int>(blockIdx.x) + grid - 1) / grid;
    const int nunits = my_groups * nseg;
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    // two-launch form: the slice partials of A x are formed in this launch (workgroup p <
    // nparts forms slice p) and published as 64-bit words (value bits, tag) in part; each
    // thread notes, at its start, the tag of the word it will gather (nw <= 1024 words)
    // and waits for that tag + 1, which only this launch's producer writes (so any prior
    // content of part is harmless)
    uint64_t* words = reinterpret_cast<uint64_t*>(part);
    const int nw = kPub ? nparts * T * r : 0;
    const bool producer = kPub && static_cast<int>(blockIdx.x) < nparts;
    uint32_t gtag = 0;
    uint32_t ptag[T];
    if constexpr (kPub) {
        if (tid < nw)
            gtag = static_cast<uint32_t>(__hip_atomic_load(words + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            ptag[t] = 0;
            if (producer && tid < r)
                ptag[t] = static_cast<uint32_t>(__hip_atomic_load(words + (blockIdx.x * T + t) * r + tid,
                                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
        }
    }

    // ---- x whole (chunk c of segment c / 512 at its swizzled place; zero past d_in),
    // A rows or the A x slice partials, tables
    uint4 xr[T][kXPer];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < kXPer; ++i) xr[t][i] = x4[t * (ldx / 8) + min(tid + 1024 * i, nch - 1)];
    uint4 av[8];
    uint4 tst = uint4{0, 0, 0, 0};
    if constexpr (kAx) {
        const uint4* ar = reinterpret_cast<const uint4*>(A) + static_cast<int64_t>(min(wave, r - 1)) * nch;
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = ar[min(lane + 64 * e, nch - 1)];
    } else if constexpr (!kPub) {
        // the slice partials of the slice kernel (launched before this one)
        if (wave >= 10 && wave < 14)
            tst = reinterpret_cast<const uint4*>(part)[min(tid - 640, (nparts * T * r + 3) / 4 - 1)];
    }
    auto unit_issue = [&](GvUnit& k, int u) {
        const int gi = u / nseg;
        const int S = u - gi * nseg;
        const int row = min((static_cast<int>(blockIdx.x) + gi * grid) * kGvWaves + wave, d_out - 1);
        {
            const int64_t b = static_cast<int64_t>(row) * nbpr + min(S * 64 + lane, nbpr - 1);
            k.qv = bc.q[b];
            k.sv = bc.scale[b >> bc.gshift];
        }
        const int64_t row_u = static_cast<int64_t>(row) * upr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = S * kGvSeg + h * 2048 + lane * 32;
            k.cw[h] = codes[row_u + (col < d_in ? col / 32 : 0)];
        }
#pragma unroll
        for (int i = 0; i < kBw; ++i) k.bw[i] = B[static_cast<int64_t>(row) * r + min(lane + 64 * i, r - 1)];
    };
    // the first unit's loads: right behind x in the two-launch form, after the first
    // barrier when the workgroup also fetches the rows of A (as in gemv_nf4_kernel)
    GvUnit g0, g1;
    if constexpr (!kAx) {
        unit_issue(g0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPub) {
        // slice p = blockIdx.x of A x from A and x in memory (the slice kernel's
        // arithmetic), started before the staging barrier, which also orders red
        if (producer) {
            float pacc[T];
            const int b_lo = static_cast<int>(blockIdx.x) * per;
            ax_slice_acc<T>(A, d_in, x, ldx, r, b_lo, min(b_lo + per, nbpr), tid, pacc);
            if (tid < 256) {
#pragma unroll
                for (int k = 0; k < T; ++k) red[k][tid] = pacc[k];
            }
        }
    }
    {
        const int pr = tid >> 2;
        float lo = tab.code[0], hi = tab.code[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            lo = (pr & 15) == i ? tab.code[i] : lo;
            hi = (pr >> 4) == i ? tab.code[i] : hi;
        }
        const uint32_t v = pack_bf16x2(lo, hi);
#pragma unroll
        for (int c = 0; c < 4; ++c) lut4[pr * (kLutCopies / 4) + (tid & 3) * 4 + c] = uint4{v, v, v, v};
        if (tid < 256) qlut[tid] = dq_step(bc.fmt, static_cast<int8_t>(tid - 128));
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < kXPer; ++i) {
            const int c = tid + 1024 * i;
            if (c < nseg * (kGvSeg / 8)) xs[t][(c & ~511) + gv_xpos(c & 511)] = c < nch ? xr[t][i] : uint4{0, 0, 0, 0};
        }
    if (!kAx && !kPub && wave >= 10 && wave < 14) reinterpret_cast<uint4*>(tvs)[tid - 640] = tst;
    if (tid == 0) ax_late = 0;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    if constexpr (kAx) {
        unit_issue(g0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kAx) {
        // one token at a time (the scheduling barrier keeps the next token's x reads from
        // being hoisted)
#pragma unroll
        for (int k = 0; k < T; ++k) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = lane + 64 * e;
                if (c < nch) {
                    const uint4 xv = xs[k][gv_xpos(c)];
                    const uint32_t aw[4] = {av[e].x, av[e].y, av[e].z, av[e].w};
                    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[q]),
                                                            __builtin_bit_cast(bf16x2, xw[q]), t, false);
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
            if (lane == 0 && wave < r) s_t[16 * k + wave] = s * t;
            if constexpr (T > 1) __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (!kPub) {
        if (tid < r) {
#pragma unroll
            for (int k = 0; k < T; ++k) {
                float t = 0.0f;
                for (int p = 0; p < nparts; ++p) t += tvs[(p * T + k) * r + tid];
                s_t[k * r + tid] = s * t;
            }
        }
    } else if (producer) {
        // the slice sums, published with their words' tags + 1 in one 64-bit store each
        if (tid < r) {
#pragma unroll
            for (int k = 0; k < T; ++k) {
                const float v = ax_slice_sum(red[k], r, tid);
                const uint64_t w = (static_cast<uint64_t>(ptag[k] + 1u) << 32) | __float_as_uint(v);
                __hip_atomic_store(words + (blockIdx.x * T + k) * r + tid, w, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const char* lut = reinterpret_cast<const char*>(lut4);
    const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
    typedef const __attribute__((address_space(4))) float cfloat;   // a scalar load
    const float mu = *(cfloat*)(bc.mean);
    float acc[T];
#pragma unroll
    for (int k = 0; k < T; ++k) acc[k] = 0.0f;
    // two-launch form, at the first row end of the workgroup's waves (the same unit for
    // all of them): gather the published slice words into LDS, each with a bounded wait;
    // if any wait ran out (a producer not yet resident, or its word published before this
    // workgroup noted the tag), the workgroup forms every slice itself. Then s (A x) as
    // the slice partials' sum in slice order.
    auto ax_gather = [&]() {
        if (tid < nw) {
            uint64_t w = 0;
            for (int it = 0;; ++it) {
                w = __hip_atomic_load(words + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (static_cast<uint32_t>(w >> 32) == gtag + 1u) break;
                if (it >= ax_polls) {
                    ax_late = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(4);
            }
            tvs[tid] = __uint_as_float(static_cast<uint32_t>(w));
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (__builtin_amdgcn_readfirstlane(ax_late)) {
            for (int p = 0; p < nparts; ++p) {
                // token by token (each token's sum runs in the same order as in the
                // producers' all-token pass)
                for (int k = 0; k < T; ++k) {
                    float pacc[1];
                    ax_slice_acc<1>(A, d_in, x + k * ldx, ldx, r, p * per, min(p * per + per, nbpr), tid, pacc);
                    if (tid < 256) red[k][tid] = pacc[0];
                }
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (tid < r) {
#pragma unroll
                    for (int k = 0; k < T; ++k) tvs[(p * T + k) * r + tid] = ax_slice_sum(red[k], r, tid);
                }
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
        }
        if (tid < r) {
#pragma unroll
            for (int k = 0; k < T; ++k) {
                float t = 0.0f;
                for (int p = 0; p < nparts; ++p) t += tvs[(p * T + k) * r + tid];
                s_t[k * r + tid] = s * t;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // rank-r term of a row, row sum, store (the order of gemv_nf4_kernel)
    auto finish_row = [&](float v, const uint16_t (&bw)[4], int row, int k) {
#pragma unroll
        for (int i = 0; i < kBw; ++i) {
            const int j = lane + 64 * i;
            if (j < r) v += bf16_to_f32(bw[i]) * s_t[(kAx ? 16 : r) * k + j];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && row < d_out) y[k * ldy + row] = bf16_bits(v);
    };
    auto unit = [&](const GvUnit& cur, GvUnit& nxt, int u, bool issue) {
        if (issue) {
            unit_issue(nxt, min(u + 1, nunits - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        const int gi = u / nseg;
        const int S = u - gi * nseg;
        const bool bok = S * 64 + lane < nbpr;
        const float qstep = qlut[cur.qv + 128];
        const float ah_dq = mu + cur.sv * qstep;
        const float ah = !bok ? 0.0f : bc.fmt == kDqNone ? cur.sv : ah_dq;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float a = __shfl(ah, h * 32 + (lane >> 1));
            if constexpr (T == 1) {
                uint4 xv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[e] = xs[0][S * 512 + h * 256 + 4 * lane + (e ^ ((lane >> 2) & 3))];
                acc[0] += a * gemv_half_block(cur.cw[h], xv, lut, lane4);
            } else {
                const uint32_t cw[4] = {cur.cw[h].x, cur.cw[h].y, cur.cw[h].z, cur.cw[h].w};
                float pt[T];
#pragma unroll
                for (int k = 0; k < T; ++k) pt[k] = 0.0f;
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    uint4 xv[T];
#pragma unroll
                    for (int k = 0; k < T; ++k) xv[k] = xs[k][S * 512 + h * 256 + 4 * lane + (w4 ^ ((lane >> 2) & 3))];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const bf16x2 lv = __builtin_bit_cast(bf16x2, lut_pair(lut, cw[w4], lane4, b));
#pragma unroll
                        for (int k = 0; k < T; ++k) {
                            const uint32_t xw[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
                            pt[k] = __builtin_amdgcn_fdot2_f32_bf16(lv, __builtin_bit_cast(bf16x2, xw[b]), pt[k], false);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int k = 0; k < T; ++k) acc[k] += a * pt[k];
            }
        }
        if (S == nseg - 1) {
            const int row = (static_cast<int>(blockIdx.x) + gi * grid) * kGvWaves + wave;
            if constexpr (kPub) {
                if (gi == 0) ax_gather();
            }
            finish_row(acc[0], cur.bw, row, 0);
            acc[0] = 0.0f;
#pragma unroll
            for (int k = 1; k < T; ++k) {
                finish_row(acc[k], cur.bw, row, k);
                acc[k] = 0.0f;
            }
        }
    };
    // three tokens keep the loop with path-dependent issue (two units' registers in
    // flight there would exceed the 128 a lane has at 16 waves per CU)
    if constexpr (T <= 2) {
        int u = 0;
        for (; u + 1 < nunits; u += 2) {
            unit(g0, g1, u, true);
            unit(g1, g0, u + 1, true);
        }
        if (u < nunits) unit(g0, g1, u, false);
    } else {
        for (int u = 0; u < nunits; u += 2) {
            unit(g0, g1, u, u + 1 < nunits);
            if (u + 1 < nunits) unit(g1, g0, u + 1, u + 2 < nunits);
        }
    }
}

}  // namespace

int set_ax_polls(int polls) { return g_ax_polls.exchange(polls); }

bool gemv_takes_tokens(int64_t d_seq, int64_t d_out, int64_t d_in, int r) {
    if (d_seq == 1) return true;
    if (d_seq > kGemvMaxTokens) return false;
    if (r <= kGvWaves && d_in <= kGvSeg) return true;              // one launch, s A x per workgroup
    // persistent, after the A x slice kernel: 2 tokens (28672 x 8192, r = 64: 45.6 us per
    // call against 61 us in the small-batch kernels; 11008 x 4096: 17.2 against 19.4); a
    // third token costs more than it saves there (21.7 against 19.4 us on 11008 x 4096)
    return d_seq == 2 && (d_out + kGvWaves - 1) / kGvWaves > kGvPersistWgs && d_in <= kGvXMaxT;
}

int64_t gemv_part_floats(int64_t d_seq, int64_t d_in, int r) {
    // up to 1024 slice partials: floats for the slice kernel, 64-bit words (value, tag)
    // for the persistent GEMV's in-launch slices
    return 2 * std::min<int64_t>(1024, std::max<int64_t>(1, d_in / 64) * r * d_seq);
}

hipError_t launch_gemv_nf4(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                           const uint16_t* A, const uint16_t* B, int r, float s,
                           const uint16_t* x, int64_t ldx, int64_t d_seq, uint16_t* y, int64_t ldy, float* ws_part,
                           hipStream_t st) {
    if (!gemv_takes_tokens(d_seq, d_out, d_in, r)) return hipErrorInvalidValue;
    const int64_t ngroups = (d_out + kGvWaves - 1) / kGvWaves;
    const dim3 grid(static_cast<unsigned>(ngroups));
    const int nt = static_cast<int>(d_seq);
    // more row groups than CUs, or one token on rows of several segments (its loads of
    // the next segment stay in flight while one is computed: 4096 x 11008, r = 64, 15.6 ->
    // 14.8 us per call, the same bits), with x small enough to keep whole: the persistent form
    const bool one_launch = r <= kGvWaves && d_in <= kGvSeg;
    const bool persist = (ngroups > kGvPersistWgs || (nt == 1 && d_in > kGvSeg)) &&
                         d_in <= (nt == 1 ? kGvXMax : kGvXMaxT);
    // (at least one workgroup per A x slice in the two-launch form: a workgroup past the
    // row groups only forms its slice)
    const int64_t want_wgs = std::min<int64_t>(ngroups, kGvPersistWgs);
    const uint4* c4 = reinterpret_cast<const uint4*>(codes);
    const int dout = static_cast<int>(d_out), din = static_cast<int>(d_in);
    // slices of A x: at most 16, and nparts * d_seq * r <= 1024 partials in all
    // (gemv_part_floats); two tokens only in the persistent form
    const int nb64 = static_cast<int>(d_in / 64);
    const int want = std::max(1, std::min({kAxMaxParts, nb64, 1024 / (r * nt)}));
    const int per = (nb64 + want - 1) / want;
    const int nparts = (nb64 + per - 1) / per;   // <= want
    const dim3 pgrid(static_cast<unsigned>(one_launch || nt != 1 ? want_wgs : std::max<int64_t>(want_wgs, nparts)));
#define QN_GVP_LAUNCH(TT, AX, PUB, NP, PER) \
    QN_LAUNCH("gemv_nf4_persist", st, (gemv_nf4_persist<TT, AX, PUB>), pgrid, dim3(64 * kGvWaves), 0, st, c4, bc, dout, \
              din, x, ldx, B, r, s, ws_part, NP, PER, g_ax_polls.load(std::memory_order_relaxed), A, y, ldy, tables())
    if (persist && one_launch) {
        if (nt == 1) QN_GVP_LAUNCH(1, true, false, 0, 0);
        else if (nt == 2) QN_GVP_LAUNCH(2, true, false, 0, 0);
        else QN_GVP_LAUNCH(3, true, false, 0, 0);
        return hipGetLastError();
    }
    if (one_launch) {
        // one launch: every workgroup forms s A x from A (r x d_in <= 16 x 4096 bf16)
#define QN_GV_LAUNCH(TT) \
        QN_LAUNCH("gemv_nf4_kernel", st, (gemv_nf4_kernel<TT, true>), grid, dim3(64 * kGvWaves), 0, st, \
                  c4, bc, dout, din, x, static_cast<int>(ldx), nt, B, r, s, ws_part, 0, A, y, static_cast<int>(ldy), \
                  tables())
        if (nt == 1) QN_GV_LAUNCH(1);
        else if (nt == 2) QN_GV_LAUNCH(2);
        else QN_GV_LAUNCH(3);
#undef QN_GV_LAUNCH
        return hipGetLastError();
    }
    if (nt > 2) return hipErrorInvalidValue;
    if (persist && nt == 1) {
        // one token: the slices are formed inside the persistent launch (workgroups
        // 0 .. nparts - 1)
        QN_GVP_LAUNCH(1, false, true, nparts, per);
        return hipGetLastError();
    }
#define QN_AX_LAUNCH(TT) \
    QN_LAUNCH("lora_ax_partial_kernel", st, lora_ax_partial_kernel<TT>, dim3(nparts), dim3(256), 0, st, A, din, x, \
              ldx, r, per, ws_part)
    if (nt == 1) QN_AX_LAUNCH(1);
    else QN_AX_LAUNCH(2);
#undef QN_AX_LAUNCH
    if (persist) {
        QN_GVP_LAUNCH(2, false, false, nparts, per);
        return hipGetLastError();
    }
#undef QN_GVP_LAUNCH
    if (nt != 1) return hipErrorInvalidValue;
    QN_LAUNCH("gemv_nf4_kernel", st, (gemv_nf4_kernel<1, false>), grid, dim3(64 * kGvWaves), 0, st, c4, bc, dout, din,
              x, static_cast<int>(ldx), 1, B, r, s, ws_part, nparts, A, y, static_cast<int>(ldy), tables());
    return hipGetLastError();
}

}  // namespace qn
