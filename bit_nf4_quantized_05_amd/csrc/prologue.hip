// Prologue of a QLoRA linear call on gfx950: the LoRA pre-pass (rank-r product of
// the activations with A or B^T; up to two such products per launch), the adapter
// layouts and the double dequantisation of the NF4 weight to bf16 W_hat or W_hat^T,
// in one launch; the reduction of K-split pre-pass partials; and the small transpose
// of B that the input gradient uses when the pre-pass cannot read B itself.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

#include <algorithm>

namespace qn {
namespace {

// ---------------------------------------------------------------------------
// Prologue of a linear call: one launch whose workgroups take three independent
// jobs, all memory-bound, so they overlap on the chip:
//   [0, n_pre)            LoRA pre-pass  OUT[M, r_pad] = bf16(s * P[M,K] R[r,K]^T):
//                         128 tokens (32 per wave) and one K-slice per workgroup;
//                         with one slice it writes OUT (columns r..r_pad-1 as 0);
//                         with several, either each slice writes bf16(s partial) to
//                         its own r columns of OUT (when the adapter is laid out in
//                         the same launch and the slices fit in r_pad: the adapter
//                         repeats once per slice, so the GEMM adds the partials), or
//                         fp32 partials that prepass_reduce adds in slice order.
//   [n_pre, +n_adapt)     adapter layout: B padded to r_pad columns (forward) or
//                         A^T padded to r_pad columns (input gradient).
//   [.., +n_deq)          double dequantisation to bf16: W_hat row-major
//                         (forward) or W_hat^T through 64x64 LDS tiles (dX).
// ---------------------------------------------------------------------------
// One LoRA pre-pass OUT = bf16(s P R^T); a launch takes up to two (the adapter
// gradients need X A^T and dY B together; M, r, s and r_pad are shared).
struct PreJob {
    const uint16_t* P; int64_t ldp; int K;
    const uint16_t* R; int64_t ldr;  // R [r, K] row stride ldr, or k-major [K, r]
    uint16_t* OUT;
    float* ppart;                    // [psplits][M][32 NT] fp32 partials when psplits > 1 and !cat
    int psplits, kper;               // K-slices and 64-wide K-chunks per slice
    int cat;                         // slice sp writes its own bf16 partial to OUT columns sp r .. sp r + r - 1
    int n;                           // workgroups of this job
};

struct PrologueArgs {
    const uint8_t* codes; BlockConsts bc;
    int64_t d_out, d_in;
    int transposed;                 // dequant to W_hat^T [d_in, d_out] instead of W_hat
    uint16_t* what;
    PreJob pre[2];
    int M, r, r_pad; float s;
    int adapt_mode;                 // 0 none, 1 pad columns, 2 transpose + pad
    int reps;                       // copies of the adapter's r columns side by side (one per slice of a cat job)
    const uint16_t* asrc; uint16_t* adst; int64_t arows, acols;
    int n_pre, n_adapt, n_deq;      // n_pre = pre[0].n + pre[1].n
    int trans_tiles;                // 64 x 64 tiles per transposed-dequant workgroup (1..4)
};

constexpr int kDeqPerWG = 8192;                  // weights per row-major dequant workgroup (128 blocks)
constexpr int kTP = 64 + 8;                      // LDS pitch (bf16) of the transpose tile

// LoRA pre-pass. A workgroup takes 128 tokens (wave w: tokens 32 w .. 32 w + 31) and a
// slice of K; per 64-wide K chunk, the 128 rows of P and the 32 NT rows of R are fetched
// straight into LDS (direct loads, two stages that are distinct LDS objects), so every
// wave reuses the same R chunk (R is read once per 128 tokens, not once per 32). A row
// is 128 B = 8 chunks of 16 B; chunk c of row r sits at c ^ ((r >> 1) & 7), which keeps
// the 32-row MFMA fragment reads free of bank conflicts. D = R P^T per 32x32 tile:
// rank rows, token columns. Rows of R past r and tokens past M are clamped into the
// arrays; their results are not stored (ranks past r are written as 0).
// With R given k-major (R^T = B [K, r] of the input gradient, r % 8 == 0, r <= 32),
// the chunk is fetched as 64 k-rows of 32 NT ranks (pieces past r repeat a valid
// address; their ranks are not stored) and each lane's fragment of 8 consecutive k is
// gathered by ds_read_b64_tr_b16, which hands lane p of a 16-lane group column p of
// a 4 x 16 block: two reads give rows k .. k + 7. This replaces a separate transpose
// of B before the launch.
template <int NT>
struct PreStage {
    uint4 x[128 * 8];               // 128 token rows
    uint4 r[32 * NT * 8];           // 32 NT rank rows
};

template <int NT, bool KM>
__device__ __forceinline__ void pre_issue(PreStage<NT>& st, const PreJob& j, const PrologueArgs& a, int wave,
                                          int lane, int m0, int kc) {
    const int64_t k0 = static_cast<int64_t>(kc) * 64;
#pragma unroll
    for (int u = 0; u < 4; ++u) {                      // P rows 32 w + 8 u .. +7
        const int row = 32 * wave + 8 * u + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        const int64_t m = min(m0 + row, a.M - 1);
        __builtin_amdgcn_global_load_lds((global_ptr)(j.P + m * j.ldp + k0 + 8 * c),
                                         (lds_ptr)(&st.x[(32 * wave + 8 * u) * 8]), 16, 0, 0);
    }
    if constexpr (KM) {
        // piece q = 64 (4 i + w) + lane of the [64 k][32 NT ranks] chunk: k-row q / (4 NT),
        // ranks 8 (q % (4 NT)) .. +7 (pieces past r re-read the last valid one)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int q = 64 * (4 * i + wave) + lane;
            const int64_t k = k0 + q / (4 * NT);
            const int pj = min(q % (4 * NT), a.r / 8 - 1);
            __builtin_amdgcn_global_load_lds((global_ptr)(j.R + k * a.r + 8 * pj),
                                             (lds_ptr)(&st.r[64 * (4 * i + wave)]), 16, 0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NT; ++i) {                 // R rows 8 (4 i + w) .. +7
            const int row = 8 * (4 * i + wave) + (lane >> 3);
            const int c = (lane & 7) ^ ((row >> 1) & 7);
            const int64_t jr = min(row, a.r - 1);
            __builtin_amdgcn_global_load_lds((global_ptr)(j.R + jr * j.ldr + k0 + 8 * c),
                                             (lds_ptr)(&st.r[8 * (4 * i + wave) * 8]), 16, 0, 0);
        }
    }
}

#define QN_TR(d, a, off) "ds_read_b64_tr_b16 %" #d ", %" #a " offset:" #off "\n\t"

// k-major R (one rank tile): the lane's fragments for the four k16 steps u, rows
// k = 16 u + 8 (g4 / 2) + 4 h .. +3 (h = 0, 1) of ranks 16 (g4 % 2) + 4 (lane % 4) .. +3 per
// address, all eight reads in one asm block ending with its own wait. The row pitch is
// 32 ranks = 64 bytes, so the offsets are (16 u + 4 h) 64 bytes.
__device__ __forceinline__ void pre_r_fragments(const PreStage<1>& st, int lane, uint4 (&rf)[4]) {
    const int g4 = lane >> 4;
    const uint32_t base = lds_addr(st.r) +
        2 * ((8 * (g4 >> 1) + ((lane >> 2) & 3)) * 32 + 16 * (g4 & 1) + 4 * (lane & 3));
    unsigned long long v[8];
    asm volatile(QN_TR(0, 8, 0) QN_TR(1, 8, 256) QN_TR(2, 8, 1024) QN_TR(3, 8, 1280)
                 QN_TR(4, 8, 2048) QN_TR(5, 8, 2304) QN_TR(6, 8, 3072) QN_TR(7, 8, 3328)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
                   "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
                 : "v"(base)
                 : "memory");
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const unsigned long long lo = v[2 * u], hi = v[2 * u + 1];
        rf[u] = uint4{static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                      static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32)};
    }
}
#undef QN_TR

template <int NT, bool KM>
__device__ __forceinline__ void pre_compute(const PreStage<NT>& st, int wave, int lane, f32x16 (&acc)[NT]) {
    const int frow = lane & 31;
    const int sw = (frow >> 1) & 7;                    // rows 32 w + frow and 32 t + frow share it
    uint4 rf[4];
    if constexpr (KM) {
        static_assert(NT == 1, "k-major R: at most 32 ranks");
        pre_r_fragments(st, lane, rf);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = (2 * u + (lane >> 5)) ^ sw;
        const uint4 xf = st.x[(32 * wave + frow) * 8 + c];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma32(KM ? rf[u] : st.r[(32 * t + frow) * 8 + c], xf, acc[t]);
    }
}

#define QN_PRE_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

template <int NT, bool KM>
__device__ __forceinline__ void prepass_job(const PreJob& j, const PrologueArgs& a, int b, PreStage<NT>& s0,
                                            PreStage<NT>& s1) {
    constexpr int kLoads = 4 + NT;                     // direct loads per wave and stage
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles = (a.M + 127) / 128;
    const int tile = b % tiles, sp = b / tiles;
    const int m0 = tile * 128;
    const int kb = sp * j.kper;
    const int ke = min(kb + j.kper, j.K / 64);
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    // The barriers wait for LDS traffic only; each wave first waits for its own loads
    // of the stage about to be read (loads complete in issue order).
    pre_issue<NT, KM>(s0, j, a, wave, lane, m0, kb);
    for (int kc = kb; kc < ke; kc += 2) {
        if (kc + 1 < ke) { pre_issue<NT, KM>(s1, j, a, wave, lane, m0, kc + 1); QN_WAIT_VM(kLoads); }
        else QN_WAIT_VM(0);
        QN_PRE_BARRIER();
        pre_compute<NT, KM>(s0, wave, lane, acc);
        QN_PRE_BARRIER();
        if (kc + 1 >= ke) break;
        if (kc + 2 < ke) { pre_issue<NT, KM>(s0, j, a, wave, lane, m0, kc + 2); QN_WAIT_VM(kLoads); }
        else QN_WAIT_VM(0);
        QN_PRE_BARRIER();
        pre_compute<NT, KM>(s1, wave, lane, acc);
        QN_PRE_BARRIER();
    }
    // D of tile t: lane l holds ranks 32 t + 8 (v / 4) + 4 (l / 32) + v % 4 of token l % 32
    const int m = m0 + 32 * wave + (lane & 31);
    if (m >= a.M) return;
    if (j.cat) {
        // r % 4 == 0: each group of 4 ranks is wholly below r or wholly past it
        uint16_t* orow = j.OUT + static_cast<int64_t>(m) * a.r_pad;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int n = t * 32 + 8 * gq + 4 * (lane >> 5);
                if (n < a.r)
                    *reinterpret_cast<uint2*>(orow + sp * a.r + n) =
                        uint2{pack_bf16x2(a.s * acc[t][4 * gq], a.s * acc[t][4 * gq + 1]),
                              pack_bf16x2(a.s * acc[t][4 * gq + 2], a.s * acc[t][4 * gq + 3])};
            }
        }
        if (sp == j.psplits - 1)
            for (int n = j.psplits * a.r + 4 * (lane >> 5); n < a.r_pad; n += 8)   // padding columns
                *reinterpret_cast<uint2*>(orow + n) = uint2{0u, 0u};
        return;
    }
    if (j.psplits == 1) {
        uint16_t* orow = j.OUT + static_cast<int64_t>(m) * a.r_pad;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int n = t * 32 + 8 * gq + 4 * (lane >> 5);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = n + e < a.r ? a.s * acc[t][4 * gq + e] : 0.0f;
                *reinterpret_cast<uint2*>(orow + n) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
        }
        for (int n = NT * 32 + 4 * (lane >> 5); n < a.r_pad; n += 8)      // padding columns
            *reinterpret_cast<uint2*>(orow + n) = uint2{0u, 0u};
        return;
    }
    float* prow = j.ppart + (static_cast<int64_t>(sp) * a.M + m) * (32 * NT);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int n = t * 32 + 8 * gq + 4 * (lane >> 5);
            *reinterpret_cast<float4*>(prow + n) =
                float4{acc[t][4 * gq], acc[t][4 * gq + 1], acc[t][4 * gq + 2], acc[t][4 * gq + 3]};
        }
    }
}
#undef QN_PRE_BARRIER

// OUT[m, j] = bf16(s * sum of the slice partials in slice order) for j < r, 0 for
// r <= j < r_pad; a thread takes 4 consecutive columns. The first `blocks0` workgroups
// reduce job 0, the rest job 1.
struct ReduceJob { const float* part; uint16_t* OUT; int splits; };

__global__ __launch_bounds__(256)
void prepass_reduce(ReduceJob j0, ReduceJob j1, int blocks0, int M, int ncols, int r, int r_pad, float s) {
    const bool second = static_cast<int>(blockIdx.x) >= blocks0;
    const ReduceJob& jb = second ? j1 : j0;
    const int64_t idx = static_cast<int64_t>(second ? blockIdx.x - blocks0 : blockIdx.x) * 256 + threadIdx.x;
    const int q4 = r_pad / 4;
    if (idx >= static_cast<int64_t>(M) * q4) return;
    const int64_t m = idx / q4;
    const int j = static_cast<int>(idx % q4) * 4;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (j < ncols) {
        const float4 t = ordered_sum4<8>(jb.part + m * ncols + j, static_cast<int64_t>(M) * ncols, jb.splits);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = j + e < r ? s * v[e] : 0.0f;
    *reinterpret_cast<uint2*>(jb.OUT + m * r_pad + j) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
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
        const int r = static_cast<int>(a.acols), span = r * a.reps;
        if (j0 + 8 <= span && (r & 7) == 0) {
            const uint4 w = *reinterpret_cast<const uint4*>(a.asrc + i * r + j0 % r);
            *reinterpret_cast<uint4*>(a.adst + c * 8) = w;
            return;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = j0 + e < span ? a.asrc[i * r + (j0 + e) % r] : uint16_t{0};
    } else {                                                       // A [r, acols] -> A^T [acols, r_pad]
        const int r = static_cast<int>(a.arows), span = r * a.reps;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = j0 + e < span ? a.asrc[static_cast<int64_t>((j0 + e) % r) * a.acols + i] : uint16_t{0};
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
        s_ahat[tid] = block_constant(a.bc.fmt, a.bc.q[blk], a.bc.scale[blk >> a.bc.gshift], a.bc.mean[0]);
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

// Transposed dequantisation of a region of 64 (o) x 64 nt (i), nt = trans_tiles <= 4
// tiles of 64 x 64 (more tiles per workgroup for larger weights, so that there are
// about 2048 workgroups): thread (o, q4) loads the code words of its 16 columns in
// every tile at once, and thread t forms a_hat of block (o = t / 4, tile t % 4) into
// LDS, so the region costs one memory round trip. Then tile by tile, each row o
// dequantises into an LDS tile that is written out transposed as W_hat^T rows.
constexpr int kTransTiles = 4;

__device__ __forceinline__ void dequant_transposed_job(const PrologueArgs& a, int b, const float* s_code,
                                                       float* s_ahat, uint16_t* tile) {
    const int tid = threadIdx.x;
    const int tiles_i = static_cast<int>(a.d_in / 64);
    const int regions_i = (tiles_i + a.trans_tiles - 1) / a.trans_tiles;
    const int t0 = (b % regions_i) * a.trans_tiles;          // first tile of the region
    const int nt = min(a.trans_tiles, tiles_i - t0);
    const int64_t o0 = static_cast<int64_t>(b / regions_i) * 64;
    const int ol = tid >> 2;             // local row o (becomes the output column)
    const int q4 = tid & 3;              // which 16 of a tile's 64 columns
    const int64_t o = min(o0 + ol, a.d_out - 1);
    uint2 cw[kTransTiles];
#pragma unroll
    for (int k = 0; k < kTransTiles; ++k) {
        const int64_t e0 = o * a.d_in + static_cast<int64_t>(t0 + min(k, nt - 1)) * 64 + q4 * 16;
        cw[k] = *reinterpret_cast<const uint2*>(a.codes + (e0 >> 1));
    }
    {
        const int64_t ob = min(o0 + (tid >> 2), a.d_out - 1);
        const int64_t blk = (ob * a.d_in + static_cast<int64_t>(t0 + min(tid & 3, nt - 1)) * 64) >> 6;
        s_ahat[tid] = block_constant(a.bc.fmt, a.bc.q[blk], a.bc.scale[blk >> a.bc.gshift], a.bc.mean[0]);
    }
    __syncthreads();
    // write-out: the tile is 64 rows of 128 B = 512 chunks of 16 B; store u of thread t
    // takes chunk 256 u + t, so 8 consecutive lanes write one whole 128-byte row.
    // The loop runs to the constant kTransTiles so that cw[k] has a constant index
    // (a runtime index would put cw in scratch memory); nt is uniform per workgroup.
#pragma unroll
    for (int k = 0; k < kTransTiles; ++k) {
        if (k >= nt) break;
        if (k > 0) __syncthreads();      // the previous tile has been written out
        const float ahat = s_ahat[ol * kTransTiles + k];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t word = e < 8 ? cw[k].x : cw[k].y;
            tile[(q4 * 16 + e) * kTP + ol] = bf16_bits(s_code[(word >> (4 * (e & 7))) & 0xFu] * ahat);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = 256 * u + tid;
            const int il = c >> 3;           // tile row = output row i - 64 (t0 + k)
            const int cc = c & 7;            // 16-byte chunk: output columns o0 + 8 cc .. + 7
            const int64_t i = static_cast<int64_t>(t0 + k) * 64 + il;
            if (o0 + 8 * cc < a.d_out)       // d_out % 64 == 0 on this path: whole chunks
                *reinterpret_cast<uint4*>(a.what + i * a.d_out + o0 + 8 * cc) =
                    *reinterpret_cast<const uint4*>(&tile[il * kTP + 8 * cc]);
        }
    }
}

// KM0, KM1: whether pre-pass job 0 / 1 takes its R k-major
template <int NT, bool KM0, bool KM1>
__global__ __launch_bounds__(256)
void prologue_kernel(PrologueArgs a, NF4Tables tab) {
    __shared__ PreStage<NT> s0, s1;
    char* lds = reinterpret_cast<char*>(s1.x);             // 16 KB of scratch for the other jobs
    const int b = blockIdx.x;
    if (b < a.pre[0].n) {
        prepass_job<NT, KM0>(a.pre[0], a, b, s0, s1);
        return;
    }
    if (b < a.n_pre) {
        prepass_job<NT, KM1>(a.pre[1], a, b - a.pre[0].n, s0, s1);
        return;
    }
    if (b < a.n_pre + a.n_adapt) {
        adapt_job(a, b - a.n_pre);
        return;
    }
    float* s_code = reinterpret_cast<float*>(lds);             // 16 floats
    float* s_ahat = reinterpret_cast<float*>(lds + 64);        // up to 256 floats
    if (threadIdx.x < 16) s_code[threadIdx.x] = tab.code[threadIdx.x];
    const int bd = b - a.n_pre - a.n_adapt;
    if (a.transposed) {
        // Workgroups go to the 8 XCDs in turn; a code row's 128-byte line spans several
        // neighbouring regions, so each XCD takes a contiguous range of regions and a
        // line is fetched into one XCD's L2 rather than into several.
        const int bl = (a.n_deq & 7) == 0 ? (bd & 7) * (a.n_deq >> 3) + (bd >> 3) : bd;
        dequant_transposed_job(a, bl, s_code, s_ahat, reinterpret_cast<uint16_t*>(lds + 64 + 1024));
    } else {
        dequant_rows_job(a, bd, s_code, s_ahat);
    }
}

// ---------------------------------------------------------------------------
// Small layout helpers for the adapter matrices.
// ---------------------------------------------------------------------------
// src [rows, cols] -> dst [cols, ld_dst] = src^T, zero in columns rows..ld_dst-1
// (cols <= 256, ld_dst % 8 == 0, src 16-byte aligned). A workgroup takes 64 source rows,
// one contiguous span of 64 cols elements starting 128 cols bytes into src, so 16-byte
// aligned: it is read with 16-byte loads (all issued before any is used) into LDS, then
// written as cols destination segments of 64 elements, 16 bytes per thread. When cols is
// a multiple of 8, a 16-byte piece lies within one source row and goes to LDS as it is
// (row pitch cols + 8 elements keeps the pieces 16-byte aligned); otherwise element by
// element.
constexpr int kTpRows = 64;
constexpr int kTpMaxCols = 256;
constexpr int kTpPer = kTpRows * kTpMaxCols / 8 / 256;      // 16-byte pieces per thread at most

__global__ __launch_bounds__(256)
void transpose_pad_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                          uint16_t* __restrict__ dst, int64_t ld_dst) {
    __shared__ __align__(16) uint16_t t[kTpRows * (kTpMaxCols + 8)];
    const int tid = threadIdx.x;
    const int nc = static_cast<int>(cols);
    const int pitch = nc + 2;
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kTpRows;
    const int nrow = static_cast<int>(std::min<int64_t>(kTpRows, std::max<int64_t>(0, rows - i0)));
    const int total = nrow * nc;                                  // elements of the span
    const uint16_t* sp = src + i0 * cols;
    if (nc % 8 == 0) {
        const int cpr = nc / 8;                                   // pieces per source row
        const int tpitch = nc + 8;
        uint4 v[kTpPer];
#pragma unroll
        for (int k = 0; k < kTpPer; ++k) {
            const int e0 = 8 * (tid + 256 * k);
            v[k] = e0 < total ? *reinterpret_cast<const uint4*>(sp + e0) : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < kTpPer; ++k) {
            const int p = tid + 256 * k;
            if (8 * p < total) {
                const int row = p / cpr, c8 = p - row * cpr;
                *reinterpret_cast<uint4*>(&t[row * tpitch + 8 * c8]) = v[k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kTpPer; ++k) {
            const int p = tid + 256 * k;
            const int j = p >> 3, q8 = 8 * (p & 7);
            if (j < nc && i0 + q8 < ld_dst) {
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const int a = q8 + 2 * h, b = a + 1;
                    const uint32_t lo = a < nrow ? t[a * tpitch + j] : 0u;
                    const uint32_t hi = b < nrow ? t[b * tpitch + j] : 0u;
                    w[h] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(j) * ld_dst + i0 + q8) =
                    uint4{w[0], w[1], w[2], w[3]};
            }
        }
        return;
    }
    uint4 v[kTpPer];
#pragma unroll
    for (int k = 0; k < kTpPer; ++k) {
        const int e0 = 8 * (tid + 256 * k);
        v[k] = uint4{0, 0, 0, 0};
        if (e0 + 8 <= total) {
            v[k] = *reinterpret_cast<const uint4*>(sp + e0);
        } else if (e0 < total) {                                  // the span's last, partial piece
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (e0 + q < total) w[q >> 1] |= static_cast<uint32_t>(sp[e0 + q]) << (16 * (q & 1));
            v[k] = uint4{w[0], w[1], w[2], w[3]};
        }
    }
#pragma unroll
    for (int k = 0; k < kTpPer; ++k) {
        const int e0 = 8 * (tid + 256 * k);
        if (e0 < total) {
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int e = e0 + q;
                if (e < total) t[(e / nc) * pitch + e % nc] = static_cast<uint16_t>(w[q >> 1] >> (16 * (q & 1)));
            }
        }
    }
    __syncthreads();
    // destination piece p: row j = p / 8 of dst, elements i0 + 8 (p % 8) .. + 7
#pragma unroll
    for (int k = 0; k < kTpPer; ++k) {
        const int p = tid + 256 * k;
        const int j = p >> 3, q8 = 8 * (p & 7);
        if (j < nc && i0 + q8 < ld_dst) {
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int a = q8 + 2 * h, b = a + 1;
                const uint32_t lo = a < nrow ? t[a * pitch + j] : 0u;
                const uint32_t hi = b < nrow ? t[b * pitch + j] : 0u;
                w[h] = lo | (hi << 16);
            }
            *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(j) * ld_dst + i0 + q8) = uint4{w[0], w[1], w[2], w[3]};
        }
    }
}

}  // namespace

PrepassSplit prepass_split(int64_t M, int64_t K) {
    // about one pre-pass workgroup per CU: 128-token tiles times K-slices of at least
    // 4 chunks of 64
    const int64_t tiles = (M + 127) / 128;
    const int64_t nk = K / 64;
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>((256 + tiles - 1) / tiles, nk / 4));
    PrepassSplit ps;
    ps.kper = static_cast<int>((nk + want - 1) / want);
    ps.splits = static_cast<int>((nk + ps.kper - 1) / ps.kper);
    return ps;
}

namespace {

// cat_max > 1: up to cat_max K-slices, each writing its bf16 partial into its own
// column block of OUT (no reduction), unless that makes a slice much longer than the
// split it replaces (more than max(16, that split's) 64-wide K-chunks: the pre-pass
// would outlast the rest of the launch); otherwise fp32 partials in ppart (if given).
PreJob make_job(const uint16_t* P, int64_t ldp, int64_t M, int64_t K, const uint16_t* R, int64_t ldr,
                uint16_t* OUT, float* ppart, int cat_max = 0) {
    PreJob j;
    j.P = P; j.ldp = ldp; j.K = static_cast<int>(K); j.R = R; j.ldr = ldr; j.OUT = OUT; j.ppart = ppart;
    const PrepassSplit ps = prepass_split(M, K);
    const int64_t nk = K / 64;
    const int64_t cat_kper = cat_max > 1 ? (nk + std::min<int64_t>(ps.splits, cat_max) - 1) /
                                               std::min<int64_t>(ps.splits, cat_max)
                                         : 0;
    j.cat = 0;
    if (cat_max > 1 && ps.splits > 1 && cat_kper <= std::max(16, ps.kper)) {
        j.kper = static_cast<int>(cat_kper);
        j.psplits = static_cast<int>((nk + j.kper - 1) / j.kper);
        j.cat = j.psplits > 1 ? 1 : 0;
    } else {
        j.psplits = ppart == nullptr ? 1 : ps.splits;
        j.kper = j.psplits == 1 ? static_cast<int>(K / 64) : ps.kper;
    }
    j.n = static_cast<int>((M + 127) / 128) * j.psplits;
    return j;
}

// Launch the prologue for a (pre[0].n, pre[1].n set; the dequant and adapter fields
// set by the caller), then one reduction of the split pre-pass jobs.
hipError_t launch_prologue_args(PrologueArgs& a, bool km0, bool km1, hipStream_t st) {
    a.n_pre = a.pre[0].n + a.pre[1].n;
    const int NT = (a.r + 31) / 32;
    const dim3 grid(static_cast<unsigned>(a.n_pre + a.n_adapt + a.n_deq));
    const NF4Tables& tab = tables();
    if (km0 || km1) {
        if (!prepass_takes_kmajor(a.r) || (km0 && km1)) return hipErrorInvalidValue;
        if (km0) QN_LAUNCH("prologue_kernel", st, (prologue_kernel<1, true, false>), grid, dim3(256), 0, st, a, tab);
        else QN_LAUNCH("prologue_kernel", st, (prologue_kernel<1, false, true>), grid, dim3(256), 0, st, a, tab);
    } else {
        switch (NT) {
#define QN_PRO_CASE(T) \
            case T: QN_LAUNCH("prologue_kernel", st, (prologue_kernel<T, false, false>), grid, dim3(256), 0, st, \
                              a, tab); break;
            QN_PRO_CASE(1) QN_PRO_CASE(2) QN_PRO_CASE(3) QN_PRO_CASE(4)
            QN_PRO_CASE(5) QN_PRO_CASE(6) QN_PRO_CASE(7) QN_PRO_CASE(8)
#undef QN_PRO_CASE
            default: return hipErrorInvalidValue;
        }
    }
    const int64_t per_job = (static_cast<int64_t>(a.M) * (a.r_pad / 4) + 255) / 256;
    const int blocks0 = a.pre[0].n > 0 && a.pre[0].psplits > 1 && !a.pre[0].cat ? static_cast<int>(per_job) : 0;
    const int blocks1 = a.pre[1].n > 0 && a.pre[1].psplits > 1 && !a.pre[1].cat ? static_cast<int>(per_job) : 0;
    if (blocks0 + blocks1 > 0) {
        const ReduceJob r0{a.pre[0].ppart, a.pre[0].OUT, a.pre[0].psplits};
        const ReduceJob r1{a.pre[1].ppart, a.pre[1].OUT, a.pre[1].psplits};
        QN_LAUNCH("prepass_reduce", st, prepass_reduce, dim3(static_cast<unsigned>(blocks0 + blocks1)), dim3(256), 0,
                  st, r0, r1, blocks0, a.M, 32 * NT, a.r, a.r_pad, a.s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                           bool transposed,
                           uint16_t* what, const uint16_t* P, int64_t ldp, int64_t M, int64_t K,
                           const uint16_t* R, int64_t ldr, bool r_kmajor, int r, float s, uint16_t* OUT,
                           int r_pad, int adapt_mode, const uint16_t* asrc, uint16_t* adst, int64_t arows,
                           int64_t acols, float* ppart, hipStream_t st) {
    PrologueArgs a{};
    a.codes = codes; a.bc = bc;
    a.d_out = d_out; a.d_in = d_in; a.transposed = transposed ? 1 : 0; a.what = what;
    // With the adapter laid out here (r < r_pad), the K-slices of the pre-pass can each
    // take r of the r_pad columns and the adapter repeat once per slice: the GEMM's
    // LoRA K-steps then add the slice partials, and no reduction pass is needed.
    const int cat_max = adapt_mode != 0 && r % 4 == 0 ? r_pad / r : 0;
    a.pre[0] = make_job(P, ldp, M, K, R, ldr, OUT, ppart, cat_max);
    a.pre[1] = PreJob{};
    a.M = static_cast<int>(M); a.r = r; a.s = s; a.r_pad = r_pad;
    a.adapt_mode = adapt_mode; a.asrc = asrc; a.adst = adst; a.arows = arows; a.acols = acols;
    a.reps = a.pre[0].cat ? a.pre[0].psplits : 1;
    const int64_t adapt_elems = adapt_mode == 0 ? 0 : (adapt_mode == 1 ? arows : acols) * r_pad;
    a.n_adapt = static_cast<int>((adapt_elems / 8 + 255) / 256);    // one 8-entry chunk per thread
    const int64_t n = d_out * d_in;
    a.trans_tiles = static_cast<int>(std::min<int64_t>(kTransTiles, std::max<int64_t>(1, (n / 4096) / 2048)));
    a.n_deq = what == nullptr ? 0   // pre-pass (and adapter layout) only
                              : static_cast<int>(transposed ? (d_in / 64 + a.trans_tiles - 1) / a.trans_tiles *
                                                                  ((d_out + 63) / 64)
                                                            : (n + kDeqPerWG - 1) / kDeqPerWG);
    static_assert(64 + 1024 + 64 * kTP * sizeof(uint16_t) <= sizeof(PreStage<1>::x), "dequant scratch fits a stage");
    return launch_prologue_args(a, r_kmajor, false, st);
}

hipError_t launch_prepass_pair(const uint16_t* P0, int64_t ldp0, int64_t K0, const uint16_t* R0, int64_t ldr0,
                               uint16_t* OUT0, float* ppart0, const uint16_t* P1, int64_t ldp1, int64_t K1,
                               const uint16_t* R1, int64_t ldr1, bool r1_kmajor, uint16_t* OUT1, float* ppart1,
                               int64_t M, int r, float s, int r_pad, hipStream_t st) {
    PrologueArgs a{};
    a.pre[0] = make_job(P0, ldp0, M, K0, R0, ldr0, OUT0, ppart0);
    a.pre[1] = make_job(P1, ldp1, M, K1, R1, ldr1, OUT1, ppart1);
    a.M = static_cast<int>(M); a.r = r; a.s = s; a.r_pad = r_pad;
    a.n_adapt = 0; a.n_deq = 0; a.trans_tiles = 1; a.reps = 1;
    return launch_prologue_args(a, false, r1_kmajor, st);
}

hipError_t launch_transpose_pad(const uint16_t* src, int64_t rows, int64_t cols,
                                uint16_t* dst, int64_t ld_dst, hipStream_t st) {
    if (cols < 1 || cols > kTpMaxCols || ld_dst % 8 != 0 || ld_dst < rows) return hipErrorInvalidValue;
    QN_LAUNCH("transpose_pad_kernel", st, transpose_pad_kernel,
              dim3(static_cast<unsigned>((ld_dst + kTpRows - 1) / kTpRows)), dim3(256), 0, st, src, rows, cols, dst,
              ld_dst);
    return hipGetLastError();
}

}  // namespace qn
