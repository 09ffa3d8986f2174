"""The allocation-free forward (qlora_linear_fwd_noalloc): called through the C ABI, it
must give the bits of qlora_linear_fwd_ex (same kernels, their partial sums in the
library's static per-device scratch instead of a caller's workspace) on two calls in a
row, the second with a smaller input, and reject sizes its scratch cannot hold."""
import ctypes

import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
from bit_nf4_quantized_05_amd import _lib
import workloads as WL
from parity import dev, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu

# (first call, second smaller call): GEMV one-launch, GEMV two-launch (A x partials in
# scratch), 2-3 token GEMV, small batch with K-split partials in scratch, and the
# persistent GEMV of layers with more than 4096 rows (two-launch, then one-launch; at 1
# token, and at 2 tokens then 3)
PAIRS = [
    (WL.custom("k", 8192, 8192, 1, 64), WL.custom("l", 4160, 4096, 1, 16, seed=1)),
    (WL.custom("m", 8192, 8192, 2, 64), WL.custom("n", 4160, 4096, 3, 16, seed=1)),
    (WL.custom("a", 4096, 4096, 1, 16), WL.custom("b", 1024, 512, 1, 8, seed=1)),
    (WL.custom("c", 2048, 8192, 1, 64), WL.custom("d", 512, 1024, 1, 24, seed=1)),
    (WL.custom("e", 4096, 4096, 64, 16), WL.custom("f", 1024, 2048, 16, 8, seed=1)),
    (WL.custom("g", 4096, 11008, 33, 64), WL.custom("h", 256, 4096, 3, 16, seed=1)),
    (WL.custom("i", 8192, 4096, 16, 16, outlier_frac=0.001), WL.custom("j", 192, 4160, 9, 5, seed=1)),
]


def _setup(cfg):
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    return q, to_gpu_bf16(a), to_gpu_bf16(b), to_gpu_bf16(WL.make_x(cfg))


def _noalloc_c(q, A, B, s, X, Y):
    """Direct C-ABI call (ctypes), no Python wrapper."""
    lib = _lib.lib()
    return lib.qlora_linear_fwd_noalloc(q.codes.data_ptr(), q.qconst.data_ptr(), q.qscale.data_ptr(),
                                        q.qmean.data_ptr(), q.d_out, q.d_in, 0, A.data_ptr(), B.data_ptr(),
                                        A.shape[0], ctypes.c_float(s), X.data_ptr(), X.stride(0), X.shape[0],
                                        Y.data_ptr(), Y.stride(0), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("pair", PAIRS, ids=[f"{p[0].name}{p[1].name}" for p in PAIRS])
def test_noalloc_forward_equals_the_workspace_forward(pair):
    for cfg in pair:
        print(f"[no-alloc] {cfg.d_out}x{cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}", flush=True)
        q, A, B, X = _setup(cfg)
        want = qn.linear_fwd(q, A, B, cfg.s, X)
        got = torch.full_like(want, 7.0)
        assert _noalloc_c(q, A, B, cfg.s, X, got) == 0, _lib.lib().qn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), cfg.name


def test_noalloc_forward_repeated_and_through_the_binding():
    cfg = WL.custom("rep", 2048, 4096, 24, 32)
    q, A, B, X = _setup(cfg)
    want = qn.linear_fwd(q, A, B, cfg.s, X)
    for _ in range(3):
        got = qn.linear_fwd_noalloc(q, A, B, cfg.s, X)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_noalloc_forward_rejects_what_its_scratch_cannot_hold():
    lib = _lib.lib()
    F = 1 << 20
    args = lambda d_out, d_in, d_seq, r: [F, F, F, F, d_out, d_in, 0, F, F, r, ctypes.c_float(1.0), F, d_in,
                                          d_seq, F, d_out, None]
    assert lib.qlora_linear_fwd_noalloc(*args(4096, 4096, 65, 16)) == -2        # the GEMM path
    assert b"64 tokens" in lib.qn_last_error()
    assert lib.qlora_linear_fwd_noalloc(*args(28672, 8192, 64, 64)) == -2      # 29 MB of partials
    assert b"scratch" in lib.qn_last_error()
    assert lib.qlora_linear_fwd_noalloc(*args(4096, 4096, 0, 16)) == -1
