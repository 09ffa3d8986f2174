// Shared pieces of the BF16 MFMA contractions (gemm_nt.hip: operands from memory;
// gemm_nf4.hip: the weight operand dequantised from NF4 codes inside the kernel):
// tile shape, kernel arguments, tile raster, buffer descriptors and scheduling hints.
#pragma once
#include <hip/hip_runtime.h>

#include "internal.h"

namespace qn {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kChunks = BM * BK / 8;           // 16-byte chunks per operand tile (2048)
constexpr int kGroupM = 4;                     // tile rows per raster group

struct GemmArgs {
    const uint16_t* P; int64_t ldp;
    const uint16_t* Q; int64_t ldq; int kt1;
    const uint16_t* P2; int64_t ldp2;
    const uint16_t* Q2; int64_t ldq2; int kt2;
    uint16_t* C; int64_t ldc; int M, N, tiles_m, tiles_n;
    uint32_t bytesP, bytesQ, bytesP2, bytesQ2;   // buffer extents for the load descriptors
    float* part; int splits, kper;               // split path: partials [splits][rem][256 x 256], K-steps per split
    int full, rem;                               // split path: whole tiles, then rem split tiles
    // in-GEMM dequantisation (forward): Q of the main K-steps is W_hat [N, K1] formed
    // from the weight's packed NF4 codes (row-major, K1 % 64 == 0, so a K-step covers one
    // block of every row) instead of read from a bf16 copy
    const uint8_t* codes; BlockConsts bc; float code[16];
    uint32_t bytesC, bytesBq, bytesBs;           // extents of the codes, 8-bit constants, scales
};

// Launches the in-GEMM dequantising forward kernel (gemm_nf4.hip) on arguments set up
// as for gemm_nt: whole tiles, or (split) full whole tiles then rem tiles split
// `splits` ways whose fp32 partials gemm_split_reduce adds.
hipError_t launch_gemm_nf4_body(const GemmArgs& g, bool split, hipStream_t st);

namespace {

// Scheduling hints: interleave `n` groups of (1 LDS read, 2 MFMA).
#define QN_INTERLEAVE_DS_MFMA(n)                                  \
    _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {          \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);        \
    }

// logical tile index -> (tile row, tile column): grouped raster of kGroupM tile rows
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int logical, int& tm, int& tn) {
    const int gsize = kGroupM * g.tiles_n;
    const int grp = logical / gsize;
    const int first_m = grp * kGroupM;
    const int gm = min(g.tiles_m - first_m, kGroupM);
    tm = first_m + (logical % gsize) % gm;
    tn = (logical % gsize) / gm;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// Workgroup barrier without the memory fence __syncthreads() adds (which would wait
// for every in-flight load, including the stages fetched ahead). The loads a barrier
// certifies are waited for explicitly with QN_WAIT_VM before it; LDS has no cache.
// The "memory" clobber keeps the compiler from moving memory accesses across it.
#define QN_BARRIER() asm volatile("s_barrier" ::: "memory")

}  // namespace
}  // namespace qn
