// Gradients of the adapter factors of the QLoRA linear layer on gfx950.
//
// Only A and B are trained; the quantised weight stays frozen (learn.ifs.name
// deck card 1; whoami-wesleyyou.top "LoRA"). For Y = X W_hat^T + s (X A^T) B^T and
// the loss gradient dY (torch layout, one token per row):
//     dB [d_out, r] = s dY^T (X A^T) = dY^T T',   T' = bf16(s X A^T)
//     dA [r, d_in]  = s (dY B)^T X   = U'^T X,    U' = bf16(s dY B)
// T' and U' come from the linear layer's LoRA pre-pass (the same bf16 operands the
// forward and input-gradient GEMMs use). What remains is a reduction over the
// d_seq tokens, out[n, j] = sum_m P[m, n] T[m, j] with P = dY or X: tall and skinny
// (N = 4096 columns, r = 16 rank entries, K = d_seq), bound by the single read of P.
//
// lora_grad_partials: a workgroup takes 128 columns and a slice of tokens; lane l
// owns columns 2l, 2l+1 (one 4-byte load per token), the 4 waves take quarters of
// the slice. Two tokens at a time, each column's bf16 pair (P[m, c], P[m+1, c]) is
// dotted with the pair (T[m, j], T[m+1, j]) by v_dot2_f32_bf16; the T rows are
// wave-uniform (scalar loads). The 4 waves are summed through LDS in a fixed order
// and the workgroup writes one partial per (slice, column, j).
// lora_grad_reduce: adds the slice partials in slice order. Deterministic.
#include <hip/hip_runtime.h>

#include "internal.h"

#include <algorithm>

namespace qn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGCols = 128;       // columns per workgroup
constexpr int kGSlices = 512;     // target partial workgroups per gradient

struct GradJob {
    const uint16_t* P; int64_t N;    // [d_seq, N]
    const uint16_t* T;               // [d_seq, r_pad]
    float* part;                     // [S][N][r]
    int tiles, S, L;                 // column tiles, token slices, slice length (multiple of 8)
};

struct GradArgs {
    GradJob job[2];                  // 0: dB (P = dY), 1: dA (P = X)
    int d_seq, r, r_pad;
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int J>
__global__ __launch_bounds__(256)
void lora_grad_partials(GradArgs g) {
    __shared__ float red[4][kGCols][16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb0 = g.job[0].tiles * g.job[0].S;
    const int which = static_cast<int>(blockIdx.x) < nb0 ? 0 : 1;
    const GradJob& jb = g.job[which];
    const int b = static_cast<int>(blockIdx.x) - (which ? nb0 : 0);
    const int tile = b % jb.tiles;
    const int slice = b / jb.tiles;
    const int64_t n0 = static_cast<int64_t>(tile) * kGCols;
    const int c0 = 2 * lane;
    const bool cok = n0 + c0 < jb.N;                 // N is even: both columns or neither
    const int m_lo = slice * jb.L;
    const int m_hi = min(m_lo + jb.L, g.d_seq);
    const int q = jb.L / 4;
    const int wm_lo = min(m_lo + wave * q, m_hi);
    const int wm_hi = min(wm_lo + q, m_hi);
    const uint32_t* pcol = reinterpret_cast<const uint32_t*>(jb.P + (cok ? n0 + c0 : 0));
    const int64_t pstride = jb.N / 2;                // in 32-bit words

    for (int j0 = 0; j0 < g.r; j0 += J) {
        float acc[2][J];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < J; ++j) acc[c][j] = 0.0f;
        // the P words of the next token pair are loaded before the current pair is used
        uint32_t n0w = wm_lo < wm_hi ? pcol[static_cast<int64_t>(wm_lo) * pstride] : 0u;
        uint32_t n1w = wm_lo + 1 < wm_hi ? pcol[static_cast<int64_t>(wm_lo + 1) * pstride] : 0u;
        for (int m = wm_lo; m < wm_hi; m += 2) {
            const bool two = m + 1 < wm_hi;
            const int m1 = two ? m + 1 : m;
            const uint32_t p0 = n0w;
            const uint32_t p1 = two ? n1w : 0u;
            n0w = m + 2 < wm_hi ? pcol[static_cast<int64_t>(m + 2) * pstride] : 0u;
            n1w = m + 3 < wm_hi ? pcol[static_cast<int64_t>(m + 3) * pstride] : 0u;
            const uint32_t pc0 = (p0 & 0xFFFFu) | (p1 << 16);          // (P[m, c0], P[m+1, c0])
            const uint32_t pc1 = (p0 >> 16) | (p1 & 0xFFFF0000u);      // (P[m, c1], P[m+1, c1])
            const uint32_t* t0 = reinterpret_cast<const uint32_t*>(jb.T + static_cast<int64_t>(m) * g.r_pad + j0);
            const uint32_t* t1 = reinterpret_cast<const uint32_t*>(jb.T + static_cast<int64_t>(m1) * g.r_pad + j0);
#pragma unroll
            for (int w = 0; w < J / 2; ++w) {
                const uint32_t a = t0[w];
                const uint32_t bb = t1[w];                               // a second copy of row m if !two
                const uint32_t te = (a & 0xFFFFu) | (bb << 16);          // (T[m, 2w], T[m+1, 2w])
                const uint32_t to = (a >> 16) | (bb & 0xFFFF0000u);      // (T[m, 2w+1], T[m+1, 2w+1])
                acc[0][2 * w] = dot2(pc0, te, acc[0][2 * w]);
                acc[1][2 * w] = dot2(pc1, te, acc[1][2 * w]);
                acc[0][2 * w + 1] = dot2(pc0, to, acc[0][2 * w + 1]);
                acc[1][2 * w + 1] = dot2(pc1, to, acc[1][2 * w + 1]);
            }
        }
        // the 4 waves' partials, 16 rank entries at a time, summed in wave order
#pragma unroll
        for (int jc = 0; jc < J / 16; ++jc) {
            __syncthreads();
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) red[wave][c0 + c][jj] = acc[c][jc * 16 + jj];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kGCols * 16 / 256; ++k) {
                const int idx = tid + 256 * k;
                const int col = idx >> 4, jj = idx & 15;
                const int j = j0 + jc * 16 + jj;
                const float v = ((red[0][col][jj] + red[1][col][jj]) + red[2][col][jj]) + red[3][col][jj];
                if (n0 + col < jb.N && j < g.r)
                    jb.part[(static_cast<int64_t>(slice) * jb.N + n0 + col) * g.r + j] = v;
            }
        }
    }
}

__global__ __launch_bounds__(256)
void lora_grad_reduce(const float* __restrict__ partB, int SB, const float* __restrict__ partA, int SA,
                      int64_t d_out, int64_t d_in, int r, float* __restrict__ dA, float* __restrict__ dB) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nB = d_out * r;
    if (idx < nB) {                                   // dB[n, j], n = idx / r
        float v = 0.0f;
#pragma unroll 8
        for (int s = 0; s < SB; ++s) v += partB[static_cast<int64_t>(s) * nB + idx];
        dB[idx] = v;
        return;
    }
    const int64_t k = idx - nB;                       // dA[j, n], n fastest
    if (k >= d_in * r) return;
    const int64_t j = k / d_in, n = k % d_in;
    const int64_t nA = d_in * r;
    float v = 0.0f;
#pragma unroll 8
    for (int s = 0; s < SA; ++s) v += partA[static_cast<int64_t>(s) * nA + n * r + j];
    dA[k] = v;
}

// token slices for N columns: about kGSlices workgroups in all
void slicing(int64_t N, int64_t d_seq, int* tiles, int* S, int* L) {
    *tiles = static_cast<int>((N + kGCols - 1) / kGCols);
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>((d_seq + 7) / 8, kGSlices / *tiles));
    const int64_t len = ((d_seq + want - 1) / want + 7) / 8 * 8;
    *L = static_cast<int>(len);
    *S = static_cast<int>((d_seq + len - 1) / len);
}

}  // namespace

int64_t lora_grads_partials(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    int t, S, L;
    slicing(d_out, d_seq, &t, &S, &L);
    const int64_t nb = static_cast<int64_t>(S) * d_out * r;
    slicing(d_in, d_seq, &t, &S, &L);
    return nb + static_cast<int64_t>(S) * d_in * r;
}

hipError_t launch_lora_grads(const uint16_t* X, const uint16_t* dY, const uint16_t* Tp, const uint16_t* Up,
                             int64_t d_out, int64_t d_in, int64_t d_seq, int r, int r_pad,
                             float* part, float* dA, float* dB, hipStream_t st) {
    GradArgs g;
    g.d_seq = static_cast<int>(d_seq);
    g.r = r;
    g.r_pad = r_pad;
    GradJob& jB = g.job[0];
    GradJob& jA = g.job[1];
    jB.P = dY; jB.N = d_out; jB.T = Tp; jB.part = part;
    slicing(d_out, d_seq, &jB.tiles, &jB.S, &jB.L);
    jA.P = X; jA.N = d_in; jA.T = Up; jA.part = part + static_cast<int64_t>(jB.S) * d_out * r;
    slicing(d_in, d_seq, &jA.tiles, &jA.S, &jA.L);
    const dim3 grid(static_cast<unsigned>(jB.tiles * jB.S + jA.tiles * jA.S));
    if (r <= 16) {
        QN_LAUNCH("lora_grad_partials", st, lora_grad_partials<16>, grid, dim3(256), 0, st, g);
    } else if (r <= 32) {
        QN_LAUNCH("lora_grad_partials", st, lora_grad_partials<32>, grid, dim3(256), 0, st, g);
    } else {
        QN_LAUNCH("lora_grad_partials", st, lora_grad_partials<64>, grid, dim3(256), 0, st, g);
    }
    const int64_t total = (d_out + d_in) * r;
    QN_LAUNCH("lora_grad_reduce", st, lora_grad_reduce, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
              st, jB.part, jB.S, jA.part, jA.S, d_out, d_in, r, dA, dB);
    return hipGetLastError();
}

}  // namespace qn
