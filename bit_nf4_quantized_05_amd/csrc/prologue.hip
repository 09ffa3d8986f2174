// Prologue of a QLoRA linear call on gfx950: the LoRA pre-pass (rank-r product of
// the activations with A or B^T), the adapter layouts and the double dequantisation
// of the NF4 weight to bf16 W_hat or W_hat^T, in one launch; plus the small
// transpose of B used by the input gradient.
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
//   [0, n_pre)            LoRA pre-pass  OUT[M, r_pad] = bf16(s * P[M,K] R[r,K]^T),
//                         32 tokens per workgroup, the 4 waves on K-quarters,
//                         summed through LDS; columns r..r_pad-1 come out 0.
//   [n_pre, +n_adapt)     adapter layout: B padded to r_pad columns (forward) or
//                         A^T padded to r_pad columns (input gradient).
//   [.., +n_deq)          double dequantisation to bf16: W_hat row-major
//                         (forward) or W_hat^T through a 64x64 LDS tile (dX).
// ---------------------------------------------------------------------------
struct PrologueArgs {
    const uint8_t* codes; BlockConsts bc;
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
        s_ahat[tid] = block_constant(a.bc.fmt, a.bc.q[blk], a.bc.scale[blk >> a.bc.gshift], a.bc.mean[0]);
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

}  // namespace

hipError_t launch_prologue(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                           bool transposed,
                           uint16_t* what, const uint16_t* P, int64_t ldp, int64_t M, int64_t K,
                           const uint16_t* R, int64_t ldr, int r, float s, uint16_t* OUT, int r_pad,
                           int adapt_mode, const uint16_t* asrc, uint16_t* adst, int64_t arows,
                           int64_t acols, hipStream_t st) {
    PrologueArgs a;
    a.codes = codes; a.bc = bc;
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

}  // namespace qn
