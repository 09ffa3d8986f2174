// Small-batch forward of the QLoRA linear layer on gfx950 (2 <= d_seq <= 64 tokens).
//
// Y = dequant(W) X + s B (A X) (whoami-wesleyyou.top "LoRA"; "1. NF4": the 4-bit
// weight is dequantised to BF16 for the product) with few tokens: the weight stream
// (0.516 B per weight) dominates, so the packed codes are read once and dequantised
// in registers straight into MFMA operands; nothing is written back but Y.
//
// skinny_nf4: a workgroup takes 64 rows of W and K-slices of 8 blocks (512 weights)
// s = split, split + splits, ...; the splits are summed by the second kernel.
// ceil(r / 64) more row blocks take the rows of A instead (bf16, loaded as they are),
// so the same launch also forms the K-split partials of A x. The 64 rows are 4 groups
// of 16, each taken by two waves: of a slice's four 128-weight block pairs, wave kq of
// the group takes pairs kq and kq + 2 (two waves per SIMD where one workgroup fills a
// CU); at the end the second wave's accumulators are added to the first's through LDS.
// Per slice, the x slice of every token (zero past d_seq) is staged in LDS with its
// 16-byte chunks XOR-swizzled by the token index, and a_hat of the 64 rows x 8 blocks
// is formed once into LDS. Per block pair p, lane l of a wave (row i = l % 16, k-group
// g = l / 16) loads 16 code bytes = weights [128 p + 32 g, +32) of its row (one 16-byte
// load; the k order inside the pair is permuted, and the x fragments follow the same
// permutation), forms bf16(c[code] * a_hat) exactly as the dequantiser does, and feeds
// v_mfma_f32_16x16x32_bf16 with one 16-token tile of x as the other operand (up to 4
// tiles).
// skinny_reduce: per 16 rows, adds the split partials in order; forms T' = bf16(s A x)
// from the A x partials (in split order, as the large-batch pre-pass rounds it) and
// adds the rank-r term T' B^T (both staged in LDS); rounds to bf16.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

#include <algorithm>

namespace qn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSkRows = 64;         // rows of W per workgroup (4 groups of 16)
constexpr int kSkKq = 2;            // waves per 16-row group (they split each slice's block pairs)
constexpr int kSkThreads = 64 * 4 * kSkKq;
constexpr int kSkBlk = 8;           // 64-weight blocks per K-slice
constexpr int kSkTok = 64;          // tokens at most
constexpr int kSkSplits = 8;        // K-split partials at most
constexpr int kSkSplitTokens = 32;  // above this many tokens, at most 4 K-splits

struct SkArgs {
    const uint8_t* codes; BlockConsts bc;
    int d_out, d_in, d_seq, splits, r, r_pad;
    int64_t ldx;                    // row stride of X (elements)
    const uint16_t* X;              // [d_seq, d_in]
    const uint16_t* A;              // [r, d_in]
    float* part;                    // [splits][d_seq][d_out]
    float* part_a;                  // [splits][d_seq][r_pad]
};

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// one MFMA per token tile: the lane's 8 weights (x chunk c) of row i against token i
// of each tile
template <int TT>
__device__ __forceinline__ void mma(f32x4 (&acc)[TT], const uint4* xs, const uint4& af, int c, int i) {
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = mfma16(af, xs[(t * 16 + i) * 64 + (c ^ i)], acc[t]);
}

template <int TT>   // 16-token tiles
__global__ __launch_bounds__(kSkThreads)
void skinny_nf4(SkArgs a, NF4Tables tab) {
    constexpr int KQ = kSkKq;
    constexpr int NW = 4 * KQ;                     // waves
    constexpr int NT = 64 * NW;                    // threads
    constexpr int PP = kSkBlk / 2 / KQ;            // block pairs per wave and slice
    __shared__ uint4 xs[TT * 16 * kSkBlk * 8];     // [token][64 chunks of 8 weights], swizzled
    __shared__ float s_code[16 * 64];              // code book, copy per lane (conflict-free lookups)
    __shared__ float s_ahat[kSkRows * kSkBlk];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave & 3;                       // 16-row group
    const int kq = wave >> 2;                      // block pairs kq, kq + KQ, ... of each slice
    const int row_blocks = a.d_out / kSkRows;
    const int all_blocks = row_blocks + (a.r + kSkRows - 1) / kSkRows;
    const int rb = static_cast<int>(blockIdx.x) % all_blocks;
    const int sp = static_cast<int>(blockIdx.x) / all_blocks;
    const bool lora = rb >= row_blocks;            // workgroup-uniform: rows of A
    const int ra = (rb - row_blocks) * kSkRows + rg * 16 + (threadIdx.x & 15);
    const int nb = a.d_in / 64;
    const int nslices = (nb + kSkBlk - 1) / kSkBlk;
    const int i = lane & 15;                       // row within the group / token within a tile
    const int g = lane >> 4;                       // k-group
    const int o = lora ? 0 : rb * kSkRows + rg * 16 + i;
    const int64_t row_u = static_cast<int64_t>(o) * (a.d_in / 32);   // 16-byte code words per row
    const uint4* arow = reinterpret_cast<const uint4*>(a.A + static_cast<int64_t>(lora ? min(ra, a.r - 1) : 0) * a.d_in);
    const bool aok = lora && ra < a.r;
    const uint4* codes4 = reinterpret_cast<const uint4*>(a.codes);
    const uint4* x4 = reinterpret_cast<const uint4*>(a.X);
    const float mu = a.bc.mean[0];
    const char* code_lds = reinterpret_cast<const char*>(s_code);
    const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
    {
        // code book from the (scalar) kernel arguments by selects
        for (int e = tid; e < 16 * 64; e += NT) {
            const int c = e >> 6;
            float v = tab.code[0];
#pragma unroll
            for (int q = 1; q < 16; ++q) v = c == q ? tab.code[q] : v;
            s_code[e] = v;
        }
    }
    f32x4 acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // x of a K-slice into LDS as [token][64 chunks of 8 weights], the chunk index
    // XOR-swizzled by the token: straight from global memory (no registers), one token
    // row of 1 KB per wave instruction, lane l writing slot l = chunk l ^ (token % 16).
    // The addresses are clamped into X: a token past d_seq only feeds an output column
    // that is never stored, a chunk past the row meets zero weights.
    constexpr int kXRows = TT * 16 / NW;           // token rows per wave
    static_assert(kXRows * NW == TT * 16, "token rows split evenly over the waves");
    auto stage_x = [&](int b0, int nbk) {
#pragma unroll
        for (int j = 0; j < kXRows; ++j) {
            const int tok = wave + NW * j;
            const int c = min(lane ^ (tok & 15), nbk * 8 - 1);
            load_lds16(x4 + (static_cast<int64_t>(min(tok, a.d_seq - 1)) * a.ldx + b0 * 64) / 8 + c, xs + tok * 64);
        }
        __builtin_amdgcn_sched_barrier(0);         // the row loads go out before the loads that follow
    };
    if (lora) {
        // rows of A (workgroup-uniform branch): the 32 k of a lane as 4 x 8 bf16
        for (int sl = sp; sl < nslices; sl += a.splits) {
            const int b0 = sl * kSkBlk;
            const int nbk = min(kSkBlk, nb - b0);
            __syncthreads();                         // the previous slice's readers are done
            stage_x(b0, nbk);
            uint4 aw[PP][4];
#pragma unroll
            for (int pp = 0; pp < PP; ++pp) {
                const int p = kq + KQ * pp;
                const int bl = 2 * p + (g >> 1);
                const int64_t e0 = static_cast<int64_t>(b0 + min(bl, nbk - 1)) * 64 + 32 * (g & 1);   // clamped
#pragma unroll
                for (int st = 0; st < 4; ++st) aw[pp][st] = arow[e0 / 8 + st];
            }
            QN_WAIT_VM(PP * 4);                      // this wave's x rows have landed (A words may be in flight)
            __syncthreads();
#pragma unroll
            for (int pp = 0; pp < PP; ++pp) {
                const int p = kq + KQ * pp;
                if (2 * p >= nbk) break;
                const bool ok = aok && 2 * p + (g >> 1) < nbk;
#pragma unroll
                for (int st = 0; st < 4; ++st) mma<TT>(acc, xs, ok ? aw[pp][st] : uint4{0, 0, 0, 0}, 16 * p + 4 * g + st, i);
            }
        }
    } else {
        for (int sl = sp; sl < nslices; sl += a.splits) {
            const int b0 = sl * kSkBlk;
            const int nbk = min(kSkBlk, nb - b0);
            // x rows and block constants first, then this wave's code words
            __syncthreads();                         // the previous slice's readers are done
            stage_x(b0, nbk);
            constexpr int kCq = (kSkRows * kSkBlk + NT - 1) / NT;
            int8_t qv[kCq];
            float sv[kCq];
#pragma unroll
            for (int q = 0; q < kCq; ++q) {
                const int e = min(tid + NT * q, kSkRows * kSkBlk - 1);   // (row e / 8, block e % 8) of the rows
                const int64_t blk = static_cast<int64_t>(rb * kSkRows + (e >> 3)) * nb + b0 + min(e & 7, nbk - 1);
                qv[q] = a.bc.q[blk];
                sv[q] = a.bc.scale[blk >> a.bc.gshift];
            }
            uint4 cw[PP];
#pragma unroll
            for (int pp = 0; pp < PP; ++pp) {
                const int p = kq + KQ * pp;
                const int bl = 2 * p + (g >> 1);
                const int word = (b0 + min(bl, nbk - 1)) * 2 + (g & 1);   // clamped into the row
                cw[pp] = codes4[row_u + word];
            }
            QN_WAIT_VM(PP);                          // x rows and block constants in (code words may not be)
#pragma unroll
            for (int q = 0; q < kCq; ++q)
                if (tid + NT * q < kSkRows * kSkBlk) s_ahat[tid + NT * q] = block_constant(a.bc.fmt, qv[q], sv[q], mu);
            __syncthreads();
#pragma unroll
            for (int pp = 0; pp < PP; ++pp) {
                const int p = kq + KQ * pp;
                const int bl = 2 * p + (g >> 1);
                if (2 * p >= nbk) break;              // uniform: no block of this pair exists
                const float ah = bl < nbk ? s_ahat[(rg * 16 + i) * kSkBlk + bl] : 0.0f;
                const uint32_t words[4] = {cw[pp].x, cw[pp].y, cw[pp].z, cw[pp].w};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    // weight 2b + h of the word is nibble h of byte b: the lane's copy of code
                    // value c sits at byte offset c << 8 | lane << 2, one v_perm_b32 of the byte
                    // of low (high) nibbles and the lane offset
                    const uint32_t nib[2] = {words[st] & 0x0F0F0F0Fu, (words[st] >> 4) & 0x0F0F0F0Fu};
                    float w[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        w[e] = *reinterpret_cast<const float*>(
                                   code_lds + __builtin_amdgcn_perm(lane4, nib[e & 1], 0x0C0C0004u | ((e >> 1) << 8))) *
                               ah;
                    mma<TT>(acc, xs,
                            uint4{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                                  pack_bf16x2(w[6], w[7])},
                            16 * p + 4 * g + st, i);
                }
            }
        }
    }
    {
        // the KQ waves of a row group add their accumulators in kq order through LDS
        // (the x buffer, free once every wave is past its last MFMA)
        static_assert((KQ - 1) * 4 * TT * 64 <= TT * 16 * kSkBlk * 8, "reduction fits the x buffer");
        f32x4* red = reinterpret_cast<f32x4*>(xs);
        __syncthreads();
        if (kq > 0) {
#pragma unroll
            for (int t = 0; t < TT; ++t) red[(((kq - 1) * 4 + rg) * TT + t) * 64 + lane] = acc[t];
        }
        __syncthreads();
        if (kq > 0) return;
#pragma unroll
        for (int q = 1; q < KQ; ++q)
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const f32x4 v = red[(((q - 1) * 4 + rg) * TT + t) * 64 + lane];
                acc[t] = acc[t] + v;
            }
    }
    // D of a 16x16 tile: lane l holds rows 4 (l / 16) + v of column l % 16
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int tok = t * 16 + i;
        if (tok < a.d_seq) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if (lora) {
                    const int j = (rb - row_blocks) * kSkRows + rg * 16 + 4 * g + v;
                    if (j < a.r_pad) a.part_a[(static_cast<int64_t>(sp) * a.d_seq + tok) * a.r_pad + j] = acc[t][v];
                } else {
                    const int orow = rb * kSkRows + rg * 16 + 4 * g + v;
                    a.part[(static_cast<int64_t>(sp) * a.d_seq + tok) * a.d_out + orow] = acc[t][v];
                }
            }
        }
    }
}

// Y[t, o] = bf16( sum_split part + sum_j T'[t, j] B[o, j] ) for kRdRows rows o per
// workgroup, T'[t, j] = bf16(s * sum_split part_a). Thread tid takes the (token, row)
// pairs tid + 256 q; the rank sums go through LDS in chunks of 64 rank entries (rows
// of odd pitch, so a row of B and a row of T' fall in different banks), added chunk by
// chunk, and the ordered split sum is added to them last. Every load of a chunk is
// issued before any of them is used (split indices past `splits` re-read the last
// split and are masked out), and the split partials' loads go out first and are not
// waited for before the first chunk's, so r <= 64 costs one memory round trip.
constexpr int kRdRows = 16;

// SPL >= splits loads per output issued at once (clamped); kOne: r <= 64 (one chunk)
template <int SPL, bool kOne>
__global__ __launch_bounds__(256)
void skinny_reduce(const float* __restrict__ part, const float* __restrict__ part_a, int splits, float s,
                   int r_pad, const uint16_t* __restrict__ B, int r, int d_out, int d_seq, uint16_t* __restrict__ Y,
                   int64_t ldy) {
    constexpr int kJ = 64, kP = kJ + 1;
    constexpr int kPairs = kSkTok * kRdRows / 256;   // pairs per thread at most
    constexpr int kBPer = kRdRows * kJ / 256;        // B entries per thread and chunk
    __shared__ float s_b[kRdRows * kP];
    __shared__ float s_t[kSkTok * kP];
    const int tid = threadIdx.x;
    const int o0 = static_cast<int>(blockIdx.x) * kRdRows;
    const int npairs = d_seq * kRdRows;
    float pv[kPairs][SPL];
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
        const int e = min(tid + 256 * q, npairs - 1);
        const int64_t idx = static_cast<int64_t>(e / kRdRows) * d_out + o0 + e % kRdRows;
#pragma unroll
        for (int sp = 0; sp < SPL; ++sp)
            pv[q][sp] = part[static_cast<int64_t>(min(sp, splits - 1)) * d_seq * d_out + idx];
    }
    // the rank term of each output, chunk by chunk; the split partials are added after
    // it, so that no wait for them stands between their loads and the chunks' loads
    float lacc[kPairs];
#pragma unroll
    for (int q = 0; q < kPairs; ++q) lacc[q] = 0.0f;
    // one chunk (r <= 64) runs as straight-line code (its own instantiation): in a loop the
    // compiler waits for every load in flight (the split partials too) where the loop starts,
    // since the chunk's B loads write the same registers on each pass
    auto chunk = [&](int j0) {
        const int nj = min(kJ, r - j0);
        // this chunk's loads: kBPer entries of B, then one (token, rank) entry of T' per
        // pass (all splits); the sums follow once they are in flight
        uint16_t bv[kBPer];
#pragma unroll
        for (int i = 0; i < kBPer; ++i) {
            const int e = min(tid + 256 * i, kRdRows * nj - 1);
            bv[i] = B[static_cast<int64_t>(o0 + e / nj) * r + j0 + e % nj];
        }
        const int nt = d_seq * nj;
        __syncthreads();                                  // the previous chunk's LDS reads are done
        for (int e0 = 0; e0 < nt; e0 += 256) {
            const int e = min(e0 + tid, nt - 1);
            const int t = e / nj, j = e % nj;
            float av[SPL];
#pragma unroll
            for (int sp = 0; sp < SPL; ++sp)
                av[sp] = part_a[(static_cast<int64_t>(min(sp, splits - 1)) * d_seq + t) * r_pad + j0 + j];
            if (e0 + tid < nt) {
                float v = 0.0f;
#pragma unroll
                for (int sp = 0; sp < SPL; ++sp) v += sp < splits ? av[sp] : 0.0f;
                s_t[t * kP + j] = __uint_as_float(static_cast<uint32_t>(bf16_bits(s * v)) << 16);
            }
        }
#pragma unroll
        for (int i = 0; i < kBPer; ++i) {
            const int e = tid + 256 * i;
            if (e < kRdRows * nj) s_b[(e / nj) * kP + e % nj] = __uint_as_float(static_cast<uint32_t>(bv[i]) << 16);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPairs; ++q) {
            const int e = tid + 256 * q;
            if (e < npairs) {
                const int t = e / kRdRows, ro = e % kRdRows;
                float l = 0.0f;
                for (int j = 0; j < nj; ++j) l += s_t[t * kP + j] * s_b[ro * kP + j];
                lacc[q] = j0 == 0 ? l : lacc[q] + l;
            }
        }
    };
    if constexpr (kOne) {
        chunk(0);
    } else {
        for (int j0 = 0; j0 < r; j0 += kJ) chunk(j0);
    }
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
        const int e = tid + 256 * q;
        if (e < npairs) {
            float d = 0.0f;
#pragma unroll
            for (int sp = 0; sp < SPL; ++sp) d += sp < splits ? pv[q][sp] : 0.0f;
            Y[static_cast<int64_t>(e / kRdRows) * ldy + o0 + e % kRdRows] = bf16_bits(d + lacc[q]);
        }
    }
}

}  // namespace

int skinny_splits(int64_t d_in, int64_t d_seq) {
    // up to 8 K-splits; with more than 32 tokens the fp32 partials (splits x d_seq x d_out)
    // cost more than the extra workgroups gain, so at most 4
    const int64_t nslices = (d_in / 64 + kSkBlk - 1) / kSkBlk;
    const int64_t cap = d_seq > kSkSplitTokens ? 4 : kSkSplits;
    return static_cast<int>(std::min<int64_t>(cap, nslices));
}

hipError_t launch_skinny_nf4(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                             const uint16_t* X, int64_t ldx, int64_t d_seq,
                             const uint16_t* A, const uint16_t* B, int r, int r_pad, float s, float* part,
                             float* part_a, uint16_t* Y, int64_t ldy, hipStream_t st) {
    SkArgs a;
    a.codes = codes; a.bc = bc;
    a.d_out = static_cast<int>(d_out); a.d_in = static_cast<int>(d_in); a.d_seq = static_cast<int>(d_seq);
    a.splits = skinny_splits(d_in, d_seq);
    a.r = r; a.r_pad = r_pad;
    a.X = X; a.ldx = ldx; a.A = A; a.part = part; a.part_a = part_a;
    const int blocks = static_cast<int>(d_out / kSkRows) + (r + kSkRows - 1) / kSkRows;
    const dim3 grid(static_cast<unsigned>(blocks * a.splits));
    const NF4Tables& tab = tables();
    switch ((d_seq + 15) / 16) {
        case 1: QN_LAUNCH("skinny_nf4", st, skinny_nf4<1>, grid, dim3(kSkThreads), 0, st, a, tab); break;
        case 2: QN_LAUNCH("skinny_nf4", st, skinny_nf4<2>, grid, dim3(kSkThreads), 0, st, a, tab); break;
        case 3: QN_LAUNCH("skinny_nf4", st, skinny_nf4<3>, grid, dim3(kSkThreads), 0, st, a, tab); break;
        case 4: QN_LAUNCH("skinny_nf4", st, skinny_nf4<4>, grid, dim3(kSkThreads), 0, st, a, tab); break;
        default: return hipErrorInvalidValue;
    }
    // as many partial loads per output as there are splits (4 or 8), not 8 at clamped addresses
    const dim3 rgrid(static_cast<unsigned>(d_out / kRdRows));
    const int o = static_cast<int>(d_out), t = static_cast<int>(d_seq);
#define QN_RED(SPL, ONE) \
    QN_LAUNCH("skinny_reduce", st, (skinny_reduce<SPL, ONE>), rgrid, dim3(256), 0, st, part, part_a, a.splits, s, \
              r_pad, B, r, o, t, Y, ldy)
    if (a.splits <= 4) {
        if (r <= 64) QN_RED(4, true); else QN_RED(4, false);
    } else {
        if (r <= 64) QN_RED(kSkSplits, true); else QN_RED(kSkSplits, false);
    }
#undef QN_RED
    return hipGetLastError();
}

}  // namespace qn
