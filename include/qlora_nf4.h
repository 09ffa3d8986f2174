/*
 * qlora_nf4.h - C ABI of the MI355X (gfx950) QLoRA NF4 linear-layer library.
 *
 * The library implements the QLoRA linear layer described on these pages:
 *   [P1] whoami-wesleyyou.top, "LoRA 与 QLoRA" (sections "LoRA", "1. NF4",
 *        "2. Double Quantization (DQ)");
 *   [P2] learn.ifs.name, Dettmers et al. 2023 deck "3 QLoRA Finetuning", cards 1-4;
 *   [P4] jjjymmm.cn 2024/03 blog, sections "4-bit NormalFloat(NF4)",
 *        "Double Quantization", "QLoRA" and "量化原理";
 *   [P5] gist.science, "Sintesi Tecnica: GPTQ-intrinsic LoRA" (W ~ Q + L R with the
 *        low-rank factors at 4 or 8 bits).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - W0 is d_out x d_in, row-major (d_in contiguous), float32 on input.
 *  - Activations follow the pages' x in R^{d_in x d_seq} [P1 LoRA], stored as
 *    a torch-style [d_seq, d_in] row-major array: each token's d_in features
 *    are contiguous. Y and dY are [d_seq, d_out], dX is [d_seq, d_in]. Token t of
 *    an activation starts ld elements after token t-1 (ldx, ldy, lddy, lddx): ld
 *    is at least the row length (d_in or d_out) and a multiple of 8 (16-byte
 *    rows); a larger ld reads or writes rows of a wider array in place. Elements
 *    between the end of a row and the next row are neither read nor written.
 *  - A is r x d_in and B is d_out x r, both row-major [P1 LoRA shapes].
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - Every pointer argument is a DEVICE pointer (memory of the current HIP
 *    device), 16-byte aligned, unless stated otherwise. The caller allocates
 *    and owns every buffer, including workspaces; the library allocates no
 *    device memory and keeps no per-call state, so calls on different streams
 *    with different buffers may run concurrently.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on that stream and returns; outputs are ready once the
 *    stream has reached the enqueued work. Outputs are overwritten, never
 *    accumulated into.
 *  - Every call enqueues kernel launches only (no memset, copy, allocation or
 *    host synchronisation), so a call may be captured in a HIP graph; a replay
 *    reads whatever the captured input buffers hold at that time.
 *  - Quantised format (one NF4 + DQ weight):
 *      n   = d_out * d_in,  n_b = ceil(n / 64) blocks,  n_g = ceil(n_b / 256) groups
 *      codes  uint8 [n_b * 32] : 4-bit code of flat element 2i in the low nibble of
 *                                byte i, element 2i+1 in the high nibble; the flat
 *                                index is row-major over W0; elements past n are
 *                                zero padding and hold the exact-zero code 7.
 *      qconst int8  [n_b]      : 8-bit code of each block's absmax constant.
 *      qscale float [n_g]      : per-group scale b_g of the centred constants.
 *      qmean  float [1]        : mean mu of all block constants.
 *    That is the default second level (QN_DQ_INT8). The _ex entry points take the
 *    format `dq` explicitly; see "Second-level formats" below.
 *
 * Return codes: 0 success; -1 invalid argument (null or misaligned pointer,
 * non-positive size, ...); -2 unsupported shape; -3 workspace too small;
 * -4 HIP launch error. On a non-zero return nothing has been enqueued (except
 * for -4, where earlier kernels of the same call may have been). A short text
 * for the last error of the calling thread is returned by qn_last_error().
 * Asynchronous device faults surface at the caller's next synchronisation.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Second-level formats (the `dq` argument of the _ex entry points). The pages call
 * for 8-bit constants in blocks of 256 [P2 card 4 "8-bit floats"; P4 Double
 * Quantization "INT8"] and count 4.5 bit/param without the second level [P1 2. DQ].
 * In all three, r_j = (a_j - mu) / b_g is one float32 division and
 * a_hat_j = mu + b_g * T[q_j] one float32 multiply then one add.
 *   QN_DQ_INT8  qconst_j = round-half-even(r_j * 127) in [-127, 127]; T[q] = q / 127.
 *   QN_DQ_FP8   qconst_j = the OCP FP8 E4M3 code byte nearest to r_j * 448 (ties to
 *               the even code; 448 is E4M3's largest finite magnitude);
 *               T[q] = e4m3_value(q) / 448. Same buffer sizes as QN_DQ_INT8.
 *   QN_DQ_NONE  no second level: qscale [n_b] holds a_j itself (float32) and
 *               a_hat_j = a_j; qconst and qmean are not used and may be NULL.
 * A b_g of 0 gives q = 0 (a_hat = mu) in both 8-bit formats.
 */
#define QN_DQ_INT8 0
#define QN_DQ_FP8 1
#define QN_DQ_NONE 2

/* Library version, as major*10000 + minor*100 + patch. */
int qn_version(void);

/* Text describing the last non-zero return on the calling thread ("" if none).
 * The pointer stays valid until the next library call on the same thread. */
const char* qn_last_error(void);

/* Copies the library's 16-entry float32 NF4 code book into host memory `out16`
 * (ascending; entry 7 is the exact zero). Built from normal quantiles with
 * separate negative and positive halves sharing one zero [P2 card 3; P1 1. NF4;
 * P4 quant book]. Host pointer. Returns 0 or -1 (null pointer). */
int qn_codebook(float* out16);

/* Sizes of the quantised buffers for a d_out x d_in weight, in elements:
 * codes bytes (n_b*32), qconst entries (n_b), qscale entries (n_g).
 * Host pointers; any of them may be NULL. Returns 0, or -1 if a size is < 1. */
int qn_nf4_sizes(int64_t d_out, int64_t d_in, int64_t* codes_bytes,
                 int64_t* n_blocks, int64_t* n_groups);

/* Sizes for second-level format dq: codes bytes (n_b*32), qconst entries (n_b, or 0
 * for QN_DQ_NONE) and qscale entries (n_g, or n_b for QN_DQ_NONE); qmean is one
 * float for the 8-bit formats. Host pointers, any may be NULL. Returns 0, or -1 on a
 * bad size or format. */
int qn_nf4_sizes_ex(int64_t d_out, int64_t d_in, int dq, int64_t* codes_bytes,
                    int64_t* qconst_entries, int64_t* qscale_entries);

/* Workspace bytes nf4_quantize(_ex) needs for a d_out x d_in weight, any format
 * (0 on bad sizes). */
int64_t nf4_quantize_workspace_bytes(int64_t d_out, int64_t d_in);

/*
 * nf4_quantize - block-wise NF4 quantisation with Double Quantisation.
 *   [P1 归一化与匹配 and 2. DQ; P2 cards 2-4; P4 NF4 and Double Quantization]
 * Level 1, per block j of 64 consecutive flat elements: a_j = max|w|; each w is
 * normalised x = w / a_j (IEEE float32 division) and coded as the nearest of the
 * 16 code-book values, the lower index on an exact tie; a block of zeros codes
 * to 7.  Level 2: mu = the mean of all a_j, rounded once to float32; per group
 * g of 256 consecutive blocks, d_j = a_j - mu, b_g = max|d_j|, and
 * qconst_j = round-half-even((d_j / b_g) * 127) in [-127, 127] (0 if b_g = 0),
 * each step one float32 operation.
 *   W          [d_out*d_in] float32, finite values (non-finite input: unspecified codes)
 *   codes, qconst, qscale, qmean : outputs, sizes as in qn_nf4_sizes
 *   workspace  >= nf4_quantize_workspace_bytes(d_out, d_in) bytes of device memory
 * Any d_out, d_in >= 1 (n need not be a multiple of 64). Result is
 * deterministic and bit-identical for every launch configuration.
 */
int nf4_quantize(const float* W, int64_t d_out, int64_t d_in,
                 uint8_t* codes, int8_t* qconst, float* qscale, float* qmean,
                 void* workspace, int64_t workspace_bytes, void* stream);

/* nf4_quantize with second-level format dq (QN_DQ_INT8 gives nf4_quantize). The
 * first level and mu are the same in every format; QN_DQ_NONE writes a_j to qscale
 * [n_b] and leaves qconst and qmean alone (they may be NULL). -1 on an unknown dq. */
int nf4_quantize_ex(const float* W, int64_t d_out, int64_t d_in, int dq,
                    uint8_t* codes, int8_t* qconst, float* qscale, float* qmean,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * nf4_double_dequant - constants first, then weights, to BF16.
 *   [P4 QLoRA: doubleDequant; P1 2. DQ a_hat = mu + b r_hat; P1 4-bit -> BF16]
 * a_hat_j = mu + b_g * (qconst_j / 127) (separate float32 multiply and add),
 * w_hat = bf16_round_nearest_even(code_book[code] * a_hat_j).
 *   W_bf16 [d_out*d_in] uint16 output, row-major like W0.
 * Any d_out, d_in >= 1.
 */
int nf4_double_dequant(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                       const float* qmean, int64_t d_out, int64_t d_in,
                       uint16_t* W_bf16, void* stream);

/* nf4_double_dequant for a weight quantised in format dq (a_hat as defined under
 * "Second-level formats"). */
int nf4_double_dequant_ex(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                          const float* qmean, int64_t d_out, int64_t d_in, int dq,
                          uint16_t* W_bf16, void* stream);

/* Workspace bytes of qlora_linear_fwd(_ex) and of qlora_linear_bwd_x(_ex) for the given
 * sizes (0 on bad sizes). The forward with d_seq <= 64 streams the packed codes and needs
 * only partial sums (at most 8 KB at d_seq = 1); every other call dequantises W
 * into the workspace (2 bytes per weight). qlora_linear_workspace_bytes is the larger
 * of the two, enough for either call. */
int64_t qlora_linear_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r);
int64_t qlora_linear_fwd_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r);
int64_t qlora_linear_bwd_x_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r);

/*
 * qlora_linear_fwd - Y = dequant(W) X + s B (A X) with BF16 operands.
 *   [P1 LoRA: y = W0 x + s B(A x), sequence input x in R^{d_in x d_seq};
 *    P1 1. NF4: 4-bit -> dequant -> BF16 -> GEMM; P2 card 1]
 *   A [r, d_in], B [d_out, r], X [d_seq, d_in] bf16 with row stride ldx; Y [d_seq, d_out]
 *   bf16 output with row stride ldy (float32 accumulation, one final round to nearest
 *   even). s is the LoRA scale (float32). The workspace must hold
 *   qlora_linear_fwd_workspace_bytes(d_out, d_in, d_seq, r) bytes.
 * Requires d_in % 64 == 0 and d_out % 64 == 0 (-2 otherwise), 1 <= r <= 256,
 * d_seq >= 1, ldx >= d_in and ldy >= d_out, both multiples of 8 (-1 otherwise).
 * d_seq == 1 (and d_seq = 2, 3 when r <= 16 and d_in <= 4096) runs a
 * streaming GEMV over the packed codes; other d_seq <= 64 stream the codes once into
 * small MFMA tiles; larger d_seq runs the MFMA GEMM with the LoRA branch as extra
 * K-steps, on W_hat either dequantised to bf16 in the workspace first or formed tile by
 * tile inside the GEMM (qlora_set_fwd_gemm; the results are the same bits either way).
 */
int qlora_linear_fwd(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                     const float* qmean, int64_t d_out, int64_t d_in,
                     const uint16_t* A, const uint16_t* B, int r, float s,
                     const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qlora_set_fwd_gemm - choose how the forward product for d_seq > 64 tokens meets W_hat
 *   [P2 card 1: the 4-bit weights are dequantised to BF16 whenever a weight is used in a
 *    matrix product]
 *   QN_FWD_GEMM_AUTO    the library's choice for the shape (the default): fused for a
 *                       weight of 2^27 or more elements at up to 1024 tokens, else staged
 *   QN_FWD_GEMM_STAGED  the dequantiser writes W_hat [d_out, d_in] bf16 to the workspace
 *                       and the GEMM reads it back
 *   QN_FWD_GEMM_FUSED   the GEMM forms each K-step's 256 x 64 tile of W_hat in LDS from the
 *                       codes and block constants; W_hat never reaches memory
 * Both forms compute the same bf16 weights and run the same MFMA sequence, so Y is the
 * same bits. The choice is process-wide and applies to calls made after it returns;
 * workspace sizes do not depend on it. Returns the previous choice, or -1 (nothing
 * changed) for an unknown value.
 */
#define QN_FWD_GEMM_AUTO 0
#define QN_FWD_GEMM_STAGED 1
#define QN_FWD_GEMM_FUSED 2
int qlora_set_fwd_gemm(int form);

/*
 * qlora_set_ax_wait - how long a one-token forward on the persistent GEMV waits for s (A x)
 *   [whoami-wesleyyou.top "LoRA": y = W0 x + s B (A x), the rank term of every row]
 * When the rank term needs the A x slice sums (r > 16 or d_in > 4096) and the layer takes
 * the persistent GEMV (more than 4096 rows, or rows of several 4096-weight segments), the
 * first workgroups of the same launch form the slices and publish them; every workgroup
 * polls for them at most `polls` times per word (default 64, about 20 us) and past that forms every
 * slice itself. The outputs are the same bits either way (0 makes every workgroup that does
 * not find the slices already published form them itself: slower, for tests). Process-wide,
 * for calls made after it returns. Returns the previous value, or -1 (nothing changed) for
 * polls < 0.
 */
int qlora_set_ax_wait(int polls);

/* qlora_linear_fwd for a weight quantised in format dq. */
int qlora_linear_fwd_ex(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                        const float* qmean, int64_t d_out, int64_t d_in, int dq,
                        const uint16_t* A, const uint16_t* B, int r, float s,
                        const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy,
                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qlora_linear_fwd_noalloc - qlora_linear_fwd_ex for 1 <= d_seq <= 64 tokens that allocates
 * nothing and takes no workspace, for callers that cannot allocate device memory or pass
 * a workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, results (bit for bit) and kernels as qlora_linear_fwd_ex;
 * the partial sums those kernels keep go to a static device array of
 * QN_NOALLOC_SCRATCH_BYTES bytes that each device holds from the library's load until
 * the process ends. Every call on one device uses that device's array: calls that
 * overlap on one device (other streams, other threads) race and must not be made.
 * Nothing in the array needs to start at any value: a call writes all of it that it
 * reads. Returns -2 when d_seq > 64 (the GEMM path would need W dequantised into
 * scratch, 2 bytes per weight) or when the sizes need more scratch than the array
 * holds (e.g. 64 tokens of a 28672-row layer); -4 if the array's address cannot be
 * obtained. Otherwise as qlora_linear_fwd_ex.
 */
#define QN_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
int qlora_linear_fwd_noalloc(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                             const float* qmean, int64_t d_out, int64_t d_in, int dq,
                             const uint16_t* A, const uint16_t* B, int r, float s,
                             const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy,
                             void* stream);

/*
 * qlora_linear_bwd_x - input gradient dX = dequant(W)^T dY + s A^T (B^T dY).
 *   [P2 card 1: gradients flow through the dequantised weights, only A and B
 *    are trained; the formula is the adjoint of the forward above]
 *   dY [d_seq, d_out] bf16 with row stride lddy >= d_out; dX [d_seq, d_in] bf16 output
 *   with row stride lddx >= d_in. Same shape rules as qlora_linear_fwd; the workspace
 *   must hold qlora_linear_bwd_x_workspace_bytes(d_out, d_in, d_seq, r) bytes.
 */
int qlora_linear_bwd_x(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                       const float* qmean, int64_t d_out, int64_t d_in,
                       const uint16_t* A, const uint16_t* B, int r, float s,
                       const uint16_t* dY, int64_t lddy, int64_t d_seq, uint16_t* dX, int64_t lddx,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* qlora_linear_bwd_x for a weight quantised in format dq. */
int qlora_linear_bwd_x_ex(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                          const float* qmean, int64_t d_out, int64_t d_in, int dq,
                          const uint16_t* A, const uint16_t* B, int r, float s,
                          const uint16_t* dY, int64_t lddy, int64_t d_seq, uint16_t* dX, int64_t lddx,
                          void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Quantised low-rank factors: the W ~ Q + L R inference form with L and R kept at 4
 * or 8 bits [P5 gist.science "Sintesi Tecnica: GPTQ-intrinsic LoRA": W ~ Q + L R;
 * "Risultati Chiave / Empirici": the factors at 4 and 8 bits]. In the column form of
 * this layer (W0 is d_out x d_in) the correction (L R)^T is B A with B = R^T
 * [d_out, r] and A = L^T [r, d_in]; Q is the NF4 weight and s scales the product
 * (s = 1 for the pages' form).
 *
 * int8_quantize - symmetric absmax INT8 per block of 64 flat elements of a row-major
 * float32 matrix [rows, cols] (padded with +0.0) [P4 量化原理]:
 *   a_j = max|w|, q = round-half-even((w / a_j) * 127) in [-127, 127] (0 if a_j = 0),
 *   each step one float32 operation.
 *   q      int8  [ceil(rows*cols/64) * 64]   (output)
 *   absmax float [ceil(rows*cols/64)]        (output)
 * int8_dequant - w_hat = bf16_round_nearest_even((q / 127) * a_j) -> W_bf16 [rows, cols].
 * A factor "at 4 bits" is nf4_quantize_ex(..., QN_DQ_NONE, ...) of it: NF4 codes and the
 * float32 a_j per block.
 */
int int8_quantize(const float* W, int64_t rows, int64_t cols, int8_t* q, float* absmax, void* stream);
int int8_dequant(const int8_t* q, const float* absmax, int64_t rows, int64_t cols,
                 uint16_t* W_bf16, void* stream);

/* Workspace bytes qlr_linear_fwd needs (0 on bad sizes). */
int64_t qlr_linear_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r);

/*
 * qlr_linear_fwd - Y = dequant(Q) X + s B_hat (A_hat X), with the factors quantised:
 * qlora_linear_fwd_ex on the bf16 factors dequantised into the workspace.
 *   codes, qconst, qscale, qmean, dq : the NF4 weight Q (d_out x d_in) in format dq.
 *   a_bits, a_codes, a_scale : A [r, d_in]; a_bits 4 -> NF4 codes uint8 [n_b*32] and
 *       a_j float [n_b] (nf4_quantize_ex with QN_DQ_NONE); 8 -> int8 [n_b*64] and
 *       absmax float [n_b] (int8_quantize); n_b = ceil(r*d_in/64).
 *   b_bits, b_codes, b_scale : B [d_out, r] likewise, n_b = ceil(d_out*r/64) (blocks of
 *       64 consecutive flat elements, across rows when r < 64).
 *   The other arguments and the shape rules are those of qlora_linear_fwd; the
 *   workspace must hold qlr_linear_workspace_bytes(d_out, d_in, d_seq, r) bytes.
 */
int qlr_linear_fwd(const uint8_t* codes, const int8_t* qconst, const float* qscale,
                   const float* qmean, int64_t d_out, int64_t d_in, int dq,
                   int a_bits, const void* a_codes, const float* a_scale,
                   int b_bits, const void* b_codes, const float* b_scale,
                   int r, float s, const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y,
                   int64_t ldy, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes qlora_lora_grads needs (0 on bad sizes). */
int64_t qlora_lora_grads_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r);

/*
 * qlora_lora_grads - gradients of the trainable adapter factors.
 *   [P2 card 1: the 4-bit weight is frozen, gradients go to the LoRA adapters only;
 *    P1 LoRA: y = W0 x + s B(A x); the formulas are the derivatives of that forward
 *    with respect to A and B]
 *   With T = X A^T and U = dY B ([d_seq, r]):
 *     dA [r, d_in]  = s U^T X,     dB [d_out, r] = s dY^T T,
 *   computed from the bf16 operands U' = bf16(s U) and T' = bf16(s T) (the linear
 *   calls' GEMMs consume the same products, rounded to bf16 once or once per K-slice
 *   of their pre-pass), float32 accumulation, float32 outputs (overwritten). The
 *   quantised weight is not needed.
 *   A [r, d_in], B [d_out, r], X [d_seq, d_in] (row stride ldx >= d_in), dY [d_seq, d_out]
 *   (row stride lddy >= d_out) bf16 (device), strides multiples of 8; dA, dB float32
 *   (device).
 *   Same shape rules as qlora_linear_fwd (d_in, d_out multiples of 64, 1 <= r <= 256,
 *   d_seq >= 1). The result is deterministic (fixed summation order).
 */
int qlora_lora_grads(const uint16_t* A, const uint16_t* B, int r, float s,
                     const uint16_t* X, int64_t ldx, const uint16_t* dY, int64_t lddy,
                     int64_t d_out, int64_t d_in, int64_t d_seq, float* dA, float* dB,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Kernel timing, off by default. While enabled, the library brackets every kernel
 * it launches with a pair of HIP events recorded on that kernel's stream, so the
 * elapsed time of each kernel is measured on the stream it runs on.
 *   qn_profile_enable(1) clears old records and starts recording; (0) stops and clears.
 *   The events are created once (1024 of them when recording first starts, more as
 *   needed) and reused, so recording adds no event creation to a launch. Returns 0, or
 *   -4 on a HIP error (creating events needs a device).
 *   qn_profile_read waits for the recorded events and fills, per distinct kernel
 *   (up to `cap` of them), its name (NUL-terminated, truncated to name_len bytes,
 *   row i at names + i*name_len), launch count and total milliseconds. Host
 *   pointers. Returns the number of distinct kernels, or -1 on a bad argument,
 *   -4 on a HIP error.
 */
int qn_profile_enable(int on);
int qn_profile_read(char* names, int name_len, int64_t* launches, double* total_ms, int cap);
/*
 * The duration of each recorded launch of the kernel called `name` (as qn_profile_read
 * names it), in launch order: waits for those launches' events and writes the first
 * min(count, cap) milliseconds to ms (host pointer). Returns the number of such launches
 * (0 for a name never launched), or -1 on a bad argument, -4 on a HIP error.
 */
int qn_profile_durations(const char* name, float* ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
