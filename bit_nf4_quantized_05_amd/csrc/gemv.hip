// d_seq = 1 forward (decode) of the QLoRA linear layer on gfx950: a streaming GEMV
// over the packed NF4 codes with the rank-r LoRA term.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

#include <algorithm>

namespace qn {
namespace {

// ---------------------------------------------------------------------------
// d_seq = 1 (decode), and 2 or 3 tokens. When all of A fits one 4096-column segment
// with r <= 16 (A <= 128 KB, read from L2 by every workgroup), one launch: each
// gemv_nf4 workgroup forms s A x itself, wave j the dot product of row j of A with the
// x segment (of each token) it has staged in LDS anyway. Otherwise (one token only)
// two launches:
//   lora_ax_partial: the 64-column blocks of x are split into nparts contiguous
//     slices (nparts * r <= 1024); workgroup w writes, for every rank row j, the dot
//     product of A[j] and x over slice w to part[w][j] (fixed summation order).
//   gemv_nf4: streams the packed codes once and adds B (s A x), summing the slice
//     partials in a fixed order: y = W_hat x + B (s A x).
// Both are deterministic, and every workgroup forms the same s A x bits.
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
// 16-byte one, so what all 16 rows share is loaded once per workgroup with wide
// loads by one wave each and passed through LDS: the x segment (waves 0..7), the
// A x slice partials (waves 10..13) and the 16 rows of B (wave 14). The block
// constants are per row: lane l loads block l's 8-bit code (or a_j) and scale with
// its code words. The first segment's code loads go out only after the first
// barrier (x, B and the tables in LDS): issued at once with x they filled the
// memory queues ahead of it and every wave started later (one-launch decode on a
// 4096 x 4096 layer: 7.3 -> 6.7 us median). The next segment's loads go out before
// the current one is computed.
// A lane forms a_hat of block l and hands it to the two lanes owning the block's
// halves by a cross-lane read. Each code byte (two weights) is looked up as a pair
// of bf16 code values and dotted with the bf16 x pair (v_dot2_f32_bf16); a_hat
// multiplies each half-block partial once (the constant factors out of the sum
// over its block). The lookup table is replicated kLutCopies times with copy c in
// bank c, so a half-wave never collides, and the x chunks are XOR-swizzled so the
// 16-byte reads of 16 lanes hit 16 distinct bank groups. s (A x) is formed before
// the weight loop, so each wave finishes on its own (formed after it, the A loads
// would have longer to land, but the call measured 7.6 against 6.9 us).
constexpr int kGvWaves = 16;
constexpr int kGvSeg = 4096;
constexpr int kLutCopies = 32;

struct GvRowSeg {
    uint4 cw[2];            // code words of the two chunks
    int8_t qv;              // second-level code of block l
    float sv;               // its group scale (a_j without a second level)
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

// T tokens (1, 2 or 3; the ntok <= T real ones first, x rows past ntok read as zero and
// their outputs not stored): each code-pair lookup serves all T tokens. T > 1 only with
// the one-launch form (kAx); 4 tokens would need more than the 128 registers a lane has
// at 16 waves per CU.
template <int T, bool kAx>
__global__ __launch_bounds__(1024)
void gemv_nf4_kernel(const uint4* __restrict__ codes, BlockConsts bc,
                     int d_out, int d_in, const uint16_t* __restrict__ x, int ntok,
                     const uint16_t* __restrict__ B, int r, float s, const float* __restrict__ part,
                     int nparts, const uint16_t* __restrict__ A, uint16_t* __restrict__ y, NF4Tables tab) {
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
                g[k] = x4[(static_cast<int64_t>(min(k, ntok - 1)) * d_in + min(col, d_in - 8)) / 8];
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
    uint4 bst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) bst[i] = uint4{0, 0, 0, 0};
    if (wave == 14) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (64 * i < nbv) bst[i] = b4[min(lane + 64 * i, nbv - 1)];
    }
    GvRowSeg g0, g1;

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
        qlut[tid] = dq_step(bc.fmt, static_cast<int8_t>(tid - 128));      // T[q] at q + 128
    }
    stage_store(st, 0);
    if (!kAx && wave >= 10 && wave < 14) reinterpret_cast<uint4*>(tvs)[tid - 640] = tst;
    if (wave == 14) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (lane + 64 * i < nbv) bs[lane + 64 * i] = bst[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    seg_issue(g0, 0);
    __builtin_amdgcn_sched_barrier(0);
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

    const uint32_t* lut = reinterpret_cast<const uint32_t*>(lut4);
    const uint32_t lane_off = static_cast<uint32_t>(lane & (kLutCopies - 1));
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
                acc[0] += a * gemv_half_block(g.cw[h], xv, lut, lane_off);
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
                        const uint32_t byte = (cw[w4] >> (8 * b)) & 0xFFu;
                        const bf16x2 lv = __builtin_bit_cast(bf16x2, lut[byte * kLutCopies + lane_off]);
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
        if (lane == 0 && row0 + wave < d_out && k < ntok) y[static_cast<int64_t>(k) * d_out + row0 + wave] = bf16_bits(v);
    }
}

}  // namespace

bool gemv_takes_tokens(int64_t d_seq, int64_t d_in, int r) {
    return d_seq == 1 || (d_seq <= kGemvMaxTokens && r <= kGvWaves && d_in <= kGvSeg);
}

hipError_t launch_gemv_nf4(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                           const uint16_t* A, const uint16_t* B, int r, float s,
                           const uint16_t* x, int64_t d_seq, uint16_t* y, float* ws_part, hipStream_t st) {
    if (!gemv_takes_tokens(d_seq, d_in, r)) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>((d_out + kGvWaves - 1) / kGvWaves));
    const int nt = static_cast<int>(d_seq);
    if (r <= kGvWaves && d_in <= kGvSeg) {
        // one launch: every workgroup forms s A x from A (r x d_in <= 16 x 4096 bf16)
#define QN_GV_LAUNCH(TT) \
        QN_LAUNCH("gemv_nf4_kernel", st, (gemv_nf4_kernel<TT, true>), grid, dim3(64 * kGvWaves), 0, st, \
                  reinterpret_cast<const uint4*>(codes), bc, static_cast<int>(d_out), static_cast<int>(d_in), x, nt, \
                  B, r, s, ws_part, 0, A, y, tables())
        if (nt == 1) QN_GV_LAUNCH(1);
        else if (nt == 2) QN_GV_LAUNCH(2);
        else QN_GV_LAUNCH(3);
#undef QN_GV_LAUNCH
        return hipGetLastError();
    }
    // slices of A x: at most 16, and nparts * r <= 1024 partials in all
    const int nb64 = static_cast<int>(d_in / 64);
    const int want = std::max(1, std::min({kAxMaxParts, nb64, 1024 / r}));
    const int per = (nb64 + want - 1) / want;
    const int nparts = (nb64 + per - 1) / per;   // <= want
    QN_LAUNCH("lora_ax_partial_kernel", st, lora_ax_partial_kernel, dim3(nparts), dim3(256), 0, st, A,
              static_cast<int>(d_in), x, r, per, ws_part);
    QN_LAUNCH("gemv_nf4_kernel", st, (gemv_nf4_kernel<1, false>), grid, dim3(64 * kGvWaves), 0, st,
              reinterpret_cast<const uint4*>(codes), bc, static_cast<int>(d_out), static_cast<int>(d_in), x, 1, B,
              r, s, ws_part, nparts, A, y, tables());
    return hipGetLastError();
}

}  // namespace qn
