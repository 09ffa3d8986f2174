// Gradients of the adapter factors of the QLoRA linear layer on gfx950.
//
// Only A and B are trained; the quantised weight stays frozen (learn.ifs.name
// deck card 1; whoami-wesleyyou.top "LoRA"). For Y = X W_hat^T + s (X A^T) B^T and
// the loss gradient dY (torch layout, one token per row):
//     dB [d_out, r] = s dY^T (X A^T) = dY^T T',   T' = bf16(s X A^T)
//     dA [r, d_in]  = s (dY B)^T X   = U'^T X,    U' = bf16(s dY B)
// T' and U' come from the LoRA pre-pass of the linear calls (here with its K-slice
// partials added before the rounding to bf16). What remains is a reduction over the
// d_seq tokens, out[n, j] = sum_m P[m, n] T[m, j] with P = dY or X: tall and skinny
// (N = 4096 columns, r = 16 rank entries, K = d_seq), bound by the single read of P.
//
// lora_grad_mfma: the reduction over tokens on BF16 MFMAs. A workgroup takes 128
// columns n (32 per wave), 64 (or 32) rank entries j and a slice of tokens; per step
// of 32 tokens, P [32 x 128] and T [32 x 64] are fetched straight into LDS (direct
// loads, two stages that are distinct LDS objects), and each wave reads its MFMA
// fragments with ds_read_b64_tr_b16: P and T are token-major, the MFMA wants 8
// consecutive tokens per lane, and the transposing read gives a lane 4 consecutive
// rows of one column. v_mfma_f32_32x32x16_bf16 accumulates C[n, j] over the slice;
// tokens past the slice are zeroed in the A fragment. Chunks of 16 bytes in a row m
// sit at position chunk ^ 2 (m % 4), so the 4 rows a 16-lane group reads in one
// transposing read fall in different LDS banks. Each workgroup writes one partial
// per (slice, n, j).
// lora_grad_reduce: adds the slice partials in slice order. Deterministic.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mfma_device.h"
#include "nf4_device.h"

#include <algorithm>

namespace qn {
namespace {

constexpr int kGCols = 128;       // columns n per workgroup, 32 per wave
constexpr int kGJ = 64;           // rank entries per workgroup (two 32-wide MFMA blocks)
constexpr int kGK = 32;           // tokens per LDS stage
constexpr int kGSlices = 512;     // target workgroups per gradient

struct GradJob {
    const uint16_t* P; int64_t N;    // [d_seq, N]
    int64_t ldp;                     // row stride of P (elements)
    const uint16_t* T;               // [d_seq, r_pad]
    float* part;                     // [S][N][r]
    int tiles, S, L;                 // column tiles, token slices, slice length (multiple of kGK)
};

struct GradArgs {
    GradJob job[2];                  // 0: dB (P = dY), 1: dA (P = X)
    int d_seq, r, r_pad, jchunks;
};

__device__ __forceinline__ int swz(int m) { return 2 * (m & 3); }

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 r + b gives the address of row r,
// columns 4 b .. 4 b + 3 of a 4 x 16 block; lane p of the group receives column p's 4 rows.

struct GradTile {
    uint4 P[kGK * 16];               // 32 token rows x 16 chunks of 8 columns
    uint4 T[kGK * 8];                // 32 token rows x 8 chunks of 8 rank entries
};

// the step's loads, 3 per wave: P rows 4 (2 w + q) .. +3 (q = 0, 1), T rows 8 w .. +7;
// lane L of an instruction fills chunk position L % 16 (P) or L % 8 (T) of its row
__device__ __forceinline__ void grad_issue(GradTile& t, const GradJob& jb, const GradArgs& g, int wave, int lane,
                                           int64_t n0, int j0, int m) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = 4 * (2 * wave + q) + (lane >> 4);
        const int64_t mg = min(m + row, g.d_seq - 1);
        const int64_t ng = min(n0 + 8 * ((lane & 15) ^ swz(row)), jb.N - 8);
        load_lds16(jb.P + mg * jb.ldp + ng, &t.P[(2 * wave + q) * 64]);
    }
    const int row = 8 * wave + (lane >> 3);
    const int64_t mg = min(m + row, g.d_seq - 1);
    load_lds16(jb.T + mg * g.r_pad + j0 + 8 * ((lane & 7) ^ swz(row)), &t.T[wave * 64]);
}

// All transposing reads of one 32-token step in one asm block that ends with its own
// wait (so no read is in flight when the block ends). The swizzle depends on the row
// only through row % 4, so the reads of a lane differ by constant row offsets: 4 rows
// (h) and 16 rows (sub), i.e. 1 KB / 4 KB in P and 512 B / 2 KB in T.
#define QN_TR(d, a, off) "ds_read_b64_tr_b16 %" #d ", %" #a " offset:" #off "\n\t"

template <int JB>
__device__ __forceinline__ void grad_compute(const GradTile& t, int wave, int lane, int valid, f32x16 (&acc)[JB]) {
    const int g4 = lane >> 4, r = (lane >> 2) & 3, bq = lane & 3;
    const int m = 8 * (g4 >> 1) + r;                                   // row of read (sub 0, h 0)
    const int n = 32 * wave + 16 * (g4 & 1) + 4 * bq;
    const uint32_t pa = lds_addr(t.P) + 2 * (m * 128 + ((((n >> 3) ^ swz(m)) << 3) | (n & 7)));
    uint32_t ta[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
        const int j = 32 * jb + 16 * (g4 & 1) + 4 * bq;
        ta[jb] = lds_addr(t.T) + 2 * (m * 64 + ((((j >> 3) ^ swz(m)) << 3) | (j & 7)));
    }
    unsigned long long a[4], b[JB][4];                                 // [2 sub + h]
    if constexpr (JB == 1) {
        asm volatile(QN_TR(0, 8, 0) QN_TR(1, 8, 1024) QN_TR(2, 8, 4096) QN_TR(3, 8, 5120)
                     QN_TR(4, 9, 0) QN_TR(5, 9, 512) QN_TR(6, 9, 2048) QN_TR(7, 9, 2560)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
                       "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[0][2]), "=&v"(b[0][3])
                     : "v"(pa), "v"(ta[0])
                     : "memory");
    } else {
        asm volatile(QN_TR(0, 12, 0) QN_TR(1, 12, 1024) QN_TR(2, 12, 4096) QN_TR(3, 12, 5120)
                     QN_TR(4, 13, 0) QN_TR(5, 13, 512) QN_TR(6, 13, 2048) QN_TR(7, 13, 2560)
                     QN_TR(8, 14, 0) QN_TR(9, 14, 512) QN_TR(10, 14, 2048) QN_TR(11, 14, 2560)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
                       "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[0][2]), "=&v"(b[0][3]),
                       "=&v"(b[1][0]), "=&v"(b[1][1]), "=&v"(b[1][2]), "=&v"(b[1][3])
                     : "v"(pa), "v"(ta[0]), "v"(ta[1])
                     : "memory");
    }
#pragma unroll
    for (int sub = 0; sub < kGK / 16; ++sub) {
        const int mb = 16 * sub + 8 * (g4 >> 1);                       // first token of this lane's 8
        uint32_t aw[4] = {static_cast<uint32_t>(a[2 * sub]), static_cast<uint32_t>(a[2 * sub] >> 32),
                          static_cast<uint32_t>(a[2 * sub + 1]), static_cast<uint32_t>(a[2 * sub + 1] >> 32)};
        if (valid < kGK) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t keep = (mb + 2 * i < valid ? 0xFFFFu : 0u) | (mb + 2 * i + 1 < valid ? 0xFFFF0000u : 0u);
                aw[i] &= keep;
            }
        }
        const uint4 A = uint4{aw[0], aw[1], aw[2], aw[3]};
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            const unsigned long long b0 = b[jb][2 * sub], b1 = b[jb][2 * sub + 1];
            acc[jb] = mfma32(A, uint4{static_cast<uint32_t>(b0), static_cast<uint32_t>(b0 >> 32),
                                      static_cast<uint32_t>(b1), static_cast<uint32_t>(b1 >> 32)}, acc[jb]);
        }
    }
}
#undef QN_TR

template <int JB>   // 32-wide rank blocks per workgroup: 1 (r <= 32) or 2
__global__ __launch_bounds__(256)
void lora_grad_mfma(GradArgs g) {
    __shared__ GradTile s0, s1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int b = static_cast<int>(blockIdx.x);
    const int nb0 = g.job[0].tiles * g.job[0].S * g.jchunks;
    const bool second = b >= nb0;
    const GradJob jb = second ? g.job[1] : g.job[0];       // selects on kernel arguments
    b -= second ? nb0 : 0;
    const int tile = b % jb.tiles;
    b /= jb.tiles;
    const int slice = b % jb.S;
    const int j0 = (b / jb.S) * kGJ;
    const int64_t n0 = static_cast<int64_t>(tile) * kGCols;
    const int m_lo = slice * jb.L;
    const int m_hi = min(m_lo + jb.L, g.d_seq);
    const int steps = (m_hi - m_lo + kGK - 1) / kGK;

    f32x16 acc[JB];
#pragma unroll
    for (int k = 0; k < JB; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[k][v] = 0.0f;

    // The barriers wait for LDS reads and writes only (a __syncthreads fence would also
    // wait for the next stage's loads); each wave first waits for its own loads of the
    // stage about to be read, which complete in issue order.
#define QN_GRAD_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
    grad_issue(s0, jb, g, wave, lane, n0, j0, m_lo);
    for (int s = 0; s < steps; s += 2) {
        // stage 0 holds step s; step s + 1 goes to stage 1 while stage 0 is read
        if (s + 1 < steps) { grad_issue(s1, jb, g, wave, lane, n0, j0, m_lo + (s + 1) * kGK); QN_WAIT_VM(3); }
        else QN_WAIT_VM(0);
        QN_GRAD_BARRIER();
        grad_compute<JB>(s0, wave, lane, min(kGK, m_hi - (m_lo + s * kGK)), acc);
        QN_GRAD_BARRIER();
        if (s + 1 >= steps) break;
        if (s + 2 < steps) { grad_issue(s0, jb, g, wave, lane, n0, j0, m_lo + (s + 2) * kGK); QN_WAIT_VM(3); }
        else QN_WAIT_VM(0);
        QN_GRAD_BARRIER();
        grad_compute<JB>(s1, wave, lane, min(kGK, m_hi - (m_lo + (s + 1) * kGK)), acc);
        QN_GRAD_BARRIER();
    }
#undef QN_GRAD_BARRIER
    // D of a 32 x 32 tile: lane l holds rows 8 (v / 4) + 4 (l / 32) + v % 4 of column l % 32
#pragma unroll
    for (int k = 0; k < JB; ++k) {
        const int j = j0 + 32 * k + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t n = n0 + 32 * wave + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (n < jb.N && j < g.r) jb.part[(static_cast<int64_t>(slice) * jb.N + n) * g.r + j] = acc[k][v];
        }
    }
}

// dB: one output per thread, dB[n, j] at idx = n r + j, its slice partials idx + s d_out r.
// dA [r, d_in] (n fastest) from partials [S][d_in][r] (j fastest): workgroup b - nbB sums
// the contiguous partials of c = rd_cols(r) columns n (c r <= 256 floats per slice, read
// in order; one output per thread, so every thread's slice loads go out together),
// keeps them in LDS (row pitch r + 1) and writes c contiguous columns of each of the r
// rows of dA. Each output is the same ordered sum over the slices either way.
int rd_cols(int r) { return std::max(1, std::min(32, 256 / r)); }

// the ordered slice sum with as many loads in flight as there are slices (up to 16): the
// loads past the last slice would re-read it for nothing
__device__ __forceinline__ float slice_sum(const float* p, int64_t stride, int n) {
    if (n <= 4) return ordered_sum<4>(p, stride, n);
    if (n <= 8) return ordered_sum<8>(p, stride, n);
    return ordered_sum<16>(p, stride, n);
}

__global__ __launch_bounds__(256)
void lora_grad_reduce(const float* __restrict__ partB, int SB, const float* __restrict__ partA, int SA,
                      int64_t d_out, int64_t d_in, int r, int cols, int nbB, float* __restrict__ dA,
                      float* __restrict__ dB) {
    extern __shared__ float tile[];                    // cols x (r + 1)
    const int tid = threadIdx.x;
    if (static_cast<int>(blockIdx.x) < nbB) {
        const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + tid;
        const int64_t nB = d_out * r;
        if (idx < nB) dB[idx] = slice_sum(partB + idx, nB, SB);
        return;
    }
    const int64_t n0 = static_cast<int64_t>(static_cast<int>(blockIdx.x) - nbB) * cols;
    const int ncol = static_cast<int>(min<int64_t>(cols, d_in - n0));
    const int64_t nA = d_in * r;
    const int cnt = ncol * r;
    for (int e = tid; e < cnt; e += 256) {
        const int nn = e / r, j = e - nn * r;
        tile[nn * (r + 1) + j] = slice_sum(partA + n0 * r + e, nA, SA);
    }
    __syncthreads();
    for (int e = tid; e < r * cols; e += 256) {
        const int j = e / cols, nn = e % cols;
        if (nn < ncol) dA[static_cast<int64_t>(j) * d_in + n0 + nn] = tile[nn * (r + 1) + j];
    }
}

// token slices (multiples of kGK) for N columns: about kGSlices workgroups in all
void slicing(int64_t N, int64_t d_seq, int jchunks, int* tiles, int* S, int* L) {
    *tiles = static_cast<int>((N + kGCols - 1) / kGCols);
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>((d_seq + kGK - 1) / kGK,
                                                                kGSlices / (*tiles * jchunks)));
    const int64_t len = ((d_seq + want - 1) / want + kGK - 1) / kGK * kGK;
    *L = static_cast<int>(len);
    *S = static_cast<int>((d_seq + len - 1) / len);
}

int jchunks_of(int r) { return r <= 32 ? 1 : (r + kGJ - 1) / kGJ; }

}  // namespace

int64_t lora_grads_partials(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    int t, S, L;
    slicing(d_out, d_seq, jchunks_of(r), &t, &S, &L);
    const int64_t nb = static_cast<int64_t>(S) * d_out * r;
    slicing(d_in, d_seq, jchunks_of(r), &t, &S, &L);
    return nb + static_cast<int64_t>(S) * d_in * r;
}

hipError_t launch_lora_grads(const uint16_t* X, int64_t ldx, const uint16_t* dY, int64_t lddy, const uint16_t* Tp,
                             const uint16_t* Up,
                             int64_t d_out, int64_t d_in, int64_t d_seq, int r, int r_pad,
                             float* part, float* dA, float* dB, hipStream_t st) {
    GradArgs g;
    g.d_seq = static_cast<int>(d_seq);
    g.r = r;
    g.r_pad = r_pad;
    g.jchunks = jchunks_of(r);
    GradJob& jB = g.job[0];
    GradJob& jA = g.job[1];
    jB.P = dY; jB.N = d_out; jB.ldp = lddy; jB.T = Tp; jB.part = part;
    slicing(d_out, d_seq, g.jchunks, &jB.tiles, &jB.S, &jB.L);
    jA.P = X; jA.N = d_in; jA.ldp = ldx; jA.T = Up; jA.part = part + static_cast<int64_t>(jB.S) * d_out * r;
    slicing(d_in, d_seq, g.jchunks, &jA.tiles, &jA.S, &jA.L);
    const dim3 grid(static_cast<unsigned>((jB.tiles * jB.S + jA.tiles * jA.S) * g.jchunks));
    if (r <= 32) {
        QN_LAUNCH("lora_grad_mfma", st, lora_grad_mfma<1>, grid, dim3(256), 0, st, g);
    } else {
        QN_LAUNCH("lora_grad_mfma", st, lora_grad_mfma<2>, grid, dim3(256), 0, st, g);
    }
    const int nbB = static_cast<int>((d_out * r + 255) / 256);
    const int cols = rd_cols(r);
    const int nbA = static_cast<int>((d_in + cols - 1) / cols);
    QN_LAUNCH("lora_grad_reduce", st, lora_grad_reduce, dim3(static_cast<unsigned>(nbB + nbA)), dim3(256),
              static_cast<unsigned>(4 * cols * (r + 1)), st, jB.part, jB.S, jA.part, jA.S, d_out, d_in, r, cols, nbB,
              dA, dB);
    return hipGetLastError();
}

}  // namespace qn
