// Internal declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qn {

constexpr int kBlock = 64;        // weights per NF4 block
constexpr int kGroup = 256;       // block constants per double-quantisation group
constexpr int kInt8Step = 127;    // symmetric INT8 code range [-127, 127]
constexpr int kE4m3Max = 448;     // largest finite OCP FP8 E4M3 magnitude
constexpr int kLimbs = 10;        // 32-bit limbs of the exact constant sum (covers 2^320)

// Second-level (block constant) formats, the values of the C ABI's QN_DQ_* codes.
constexpr int kDqInt8 = 0;        // q = round(r * 127), a_hat = mu + b (q / 127)
constexpr int kDqFp8 = 1;         // q = E4M3 code of r * 448, a_hat = mu + b (e4m3(q) / 448)
constexpr int kDqNone = 2;        // no second level: the float32 a_j per block

// Where a kernel finds a_hat_j: from q[j], scale[j >> gshift] and mean[0]. For
// kDqNone, scale holds a_j (gshift 0) and q, mean point at readable stand-ins whose
// values are not used, so kernels may load them unconditionally.
struct BlockConsts {
    const int8_t* q;
    const float* scale;
    const float* mean;
    int fmt;
    int gshift;
};
constexpr int kCells = 32;        // [-1, 1] split into 32 equal cells for the code search

// Constant tables, built once on the host and passed to kernels by value.
struct NF4Tables {
    float code[16];                 // code book, ascending, code[7] == +0
    float cell_thr[kCells];         // the single code threshold inside cell c, or +inf
    uint32_t cell_base[kCells];     // number of thresholds below the cell's lower edge
};

// Returns the process-wide tables (built on first use, thread-safe).
const NF4Tables& tables();

// Optional kernel timing (see qn_profile_enable): a launch is wrapped as
//   void* t = prof_begin(st); launch...; prof_end(t, "name", st);
// Both are no-ops (nullptr token) while timing is off.
void* prof_begin(hipStream_t st);
void prof_end(void* token, const char* name, hipStream_t st);

#define QN_LAUNCH(NAME, ST, ...)                         \
    do {                                                 \
        void* qn_tok_ = ::qn::prof_begin(ST);            \
        hipLaunchKernelGGL(__VA_ARGS__);                 \
        ::qn::prof_end(qn_tok_, NAME, ST);               \
    } while (0)

// ---- quantize.hip ----
int quant_grid(int64_t n_b);
// fmt kDqNone writes the block constants to qscale [n_b] (qconst, qmean untouched).
hipError_t launch_quantize(const float* W, int64_t n, int64_t n_b, int64_t n_g, int fmt,
                           uint8_t* codes, int8_t* qconst, float* qscale, float* qmean,
                           float* ws_absmax, unsigned long long* ws_limbs, int grid,
                           hipStream_t st);
hipError_t launch_dequant_rows(const uint8_t* codes, const BlockConsts& bc, int64_t n, uint16_t* out,
                               hipStream_t st);

// ---- gemm_nt.hip ----
// C[M,N] = bf16( P[M,K1] Q[N,K1]^T + P2[M,K2] Q2[N,K2]^T ), all row-major, K contiguous.
// K1, K2 multiples of 64 (K2 may be 0); N multiple of 4. When the last round of
// 256 x 256 tiles holds at most 128 tiles, their K-steps are split over gemm_split().splits
// workgroups each, with fp32 partials in part (gemm_split_part_floats(M, N, K1) floats);
// a null part runs unsplit.
struct GemmSplit { int splits, full, rem; };
GemmSplit gemm_split(int64_t M, int64_t N, int64_t K1);
int64_t gemm_split_part_floats(int64_t M, int64_t N, int64_t K1);
// With codes (and bc) given, Q is instead the weight dequantised inside the GEMM from its
// packed NF4 codes ([N, K1] row-major, K1 % 64 == 0; Q and ldq are not used).
hipError_t launch_gemm_nt(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, int64_t K1,
                          const uint16_t* P2, int64_t ldp2, const uint16_t* Q2, int64_t ldq2,
                          int64_t K2, uint16_t* C, int64_t ldc, int64_t M, int64_t N, float* part,
                          hipStream_t st, const uint8_t* codes = nullptr, const BlockConsts* bc = nullptr);

// ---- prologue.hip ----
// One launch before the GEMM of a linear call: LoRA pre-pass
//   OUT[M, r_pad] = bf16(s * P[M,K] R[r,K]^T) (zero in columns r..r_pad-1, K % 64 == 0),
// an adapter layout job (adapt_mode 1: B [arows, acols] -> [arows, r_pad] zero-padded;
// 2: A [arows, acols] -> A^T [acols, r_pad] zero-padded; 0: none), and the double
// dequantisation to W_hat [d_out, d_in] or W_hat^T [d_in, d_out] (transposed; none if
// what is null). The pre-pass splits K over up to prepass_split(M, K).splits workgroups
// per 128 tokens. With an adapter job, r % 4 == 0 and at least two slices of r columns
// fitting in r_pad, slice s writes bf16(s * its partial) to OUT columns s r .. s r + r - 1
// (the rest zero) and the adapter layout repeats its r columns once per slice, so the
// GEMM adds the partials; otherwise the fp32 partials go to ppart (splits * M *
// 32 ceil(r/32) floats) and are added by a second small launch; a null ppart runs it
// unsplit.
struct PrepassSplit { int splits, kper; };
PrepassSplit prepass_split(int64_t M, int64_t K);
hipError_t launch_prologue(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                           bool transposed,
                           uint16_t* what, const uint16_t* P, int64_t ldp, int64_t M, int64_t K,
                           const uint16_t* R, int64_t ldr, bool r_kmajor, int r, float s, uint16_t* OUT,
                           int r_pad, int adapt_mode, const uint16_t* asrc, uint16_t* adst, int64_t arows,
                           int64_t acols, float* ppart, hipStream_t st);
// Two LoRA pre-passes over the same M tokens in one launch (and one reduction):
// OUT0 = bf16(s P0 R0^T) with R0 [r, K0] row stride ldr0, and OUT1 = bf16(s P1 R1^T)
// with R1 [r, K1] (or k-major [K1, r] when r1_kmajor). ppart0 / ppart1 hold each job's
// K-slice partials (prepass_split), or are null for one slice.
hipError_t launch_prepass_pair(const uint16_t* P0, int64_t ldp0, int64_t K0, const uint16_t* R0, int64_t ldr0,
                               uint16_t* OUT0, float* ppart0, const uint16_t* P1, int64_t ldp1, int64_t K1,
                               const uint16_t* R1, int64_t ldr1, bool r1_kmajor, uint16_t* OUT1, float* ppart1,
                               int64_t M, int r, float s, int r_pad, hipStream_t st);
// The pre-pass can take R k-major, as B [K, r] itself (r % 8 == 0 and r <= 32: one
// 32-rank MFMA tile, whose transposing reads keep the kernel's occupancy), which spares
// the input gradient a transpose of B.
inline bool prepass_takes_kmajor(int r) { return r % 8 == 0 && r <= 32; }
// dst[j, i] = i < rows ? src[i, j] : 0, for j < cols, i < ld_dst. src is rows x cols,
// 16-byte aligned; 1 <= cols <= 256, ld_dst >= rows and ld_dst % 8 == 0 (else an error).
hipError_t launch_transpose_pad(const uint16_t* src, int64_t rows, int64_t cols,
                                uint16_t* dst, int64_t ld_dst, hipStream_t st);

// ---- gemv.hip ----
// y[t, o] = sum_i w_hat[o,i] x[t, i] + s * sum_k B[o,k] (A x_t)[k], streaming the packed
// codes, for d_seq = 1, or for 2 <= d_seq <= kGemvMaxTokens tokens when r <= 16 and
// d_in <= 4096, or for 2 tokens when d_out > 4096 and d_in <= 8192 (gemv_takes_tokens); x rows at stride
// ldx, y rows at stride ldy (elements, multiples of 8); ws_part holds gemv_part_floats
// floats of partial A x sums (two-launch forms).
constexpr int kGemvMaxTokens = 3;
bool gemv_takes_tokens(int64_t d_seq, int64_t d_out, int64_t d_in, int r);
int64_t gemv_part_floats(int64_t d_seq, int64_t d_in, int r);
hipError_t launch_gemv_nf4(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                           const uint16_t* A, const uint16_t* B, int r, float s,
                           const uint16_t* x, int64_t ldx, int64_t d_seq, uint16_t* y, int64_t ldy, float* ws_part,
                           hipStream_t st);

// ---- skinny.hip ----
// Small-batch forward, 2 <= d_seq <= 64: Y = dequant(W) X + bf16(s X A^T) B^T from the
// packed codes, A x formed in the same launch. X rows at stride ldx, Y rows at stride ldy
// (elements, multiples of 8). part must hold skinny_splits(d_in, d_seq) * d_seq * d_out
// floats, part_a skinny_splits(d_in, d_seq) * d_seq * r_pad. d_out % 64 == 0, d_in % 64 == 0.
constexpr int kSkinnyMaxTokens = 64;
int skinny_splits(int64_t d_in, int64_t d_seq);
hipError_t launch_skinny_nf4(const uint8_t* codes, const BlockConsts& bc, int64_t d_out, int64_t d_in,
                             const uint16_t* X, int64_t ldx, int64_t d_seq,
                             const uint16_t* A, const uint16_t* B, int r, int r_pad, float s, float* part,
                             float* part_a, uint16_t* Y, int64_t ldy, hipStream_t st);

// ---- factors.hip ----
// Symmetric absmax INT8 per block of 64 flat elements of W [n] (padded with +0.0):
// q [ceil(n/64)*64] int8, absmax [ceil(n/64)] f32; and its bf16 dequantisation.
hipError_t launch_int8_quantize(const float* W, int64_t n, int8_t* q, float* absmax, hipStream_t st);
hipError_t launch_int8_dequant(const int8_t* q, const float* absmax, int64_t n, uint16_t* out, hipStream_t st);

// ---- lora_grads.hip ----
// Column-sum partials of out[n, j] = sum_m P[m, n] T[m, j] for the two adapter
// gradients, then their fixed-order sum:
//   dB [d_out, r] = dY^T T'   (P = dY, T = T' = bf16(s X A^T))
//   dA [r, d_in]  = U'^T X     (P = X,  T = U' = bf16(s dY B))
// T' and U' are [d_seq, r_pad] bf16; X and dY rows at strides ldx, lddy (elements,
// multiples of 8). part must hold lora_grads_partials(...) floats.
int64_t lora_grads_partials(int64_t d_out, int64_t d_in, int64_t d_seq, int r);
hipError_t launch_lora_grads(const uint16_t* X, int64_t ldx, const uint16_t* dY, int64_t lddy, const uint16_t* Tp,
                             const uint16_t* Up,
                             int64_t d_out, int64_t d_in, int64_t d_seq, int r, int r_pad,
                             float* part, float* dA, float* dB, hipStream_t st);

}  // namespace qn
