/*
 * qn_calibrate.h - C ABI of libqn_calibrate.so: measurement aids for the benchmark of
 * the QLoRA NF4 linear-layer library. Nothing here computes any part of the layer; each
 * call streams memory in a known pattern so that a kernel of the layer can be put
 * against the time the same reads take on their own (the floor of that access
 * pattern on the machine at hand, below the published HBM peak).
 *
 * Device pointers, 16-byte aligned; `stream` is a hipStream_t (NULL = default stream);
 * the call only enqueues one kernel. Returns 0, -1 on a bad argument (nothing
 * enqueued), -4 on a HIP launch error.
 */
#ifndef QN_CALIBRATE_H
#define QN_CALIBRATE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The decode GEMV's loads of an NF4 weight in the default (INT8 second-level) layout of
 * qlora_nf4.h without its arithmetic, x or LoRA term: one workgroup of 16 waves per 16
 * rows, one wave per row; per 4096-weight segment, lane l reads 16-byte code words l
 * and 64 + l, block l's qconst byte and its group's qscale. out [d_out] uint32 receives
 * one XOR of each row's loads. Requires d_in % 64 == 0. */
int qn_calibrate_code_stream(const uint8_t* codes, const int8_t* qconst, const float* qscale, int64_t d_out,
                             int64_t d_in, uint32_t* out, void* stream);

/* A plain streaming read of `bytes` (a multiple of 16) with `grid` workgroups of 256
 * threads, four 16-byte loads in flight per thread; out [grid] uint32 receives one XOR
 * per workgroup. */
int qn_calibrate_read(const void* src, int64_t bytes, int grid, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QN_CALIBRATE_H */
