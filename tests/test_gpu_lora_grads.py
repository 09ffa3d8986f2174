"""GPU parity of qlora_lora_grads (adapter gradients dA, dB) against the float64
oracle, through the C ABI. Tolerance as for the GEMMs: max|err|/max|ref| <= 1e-2
and relative Frobenius error <= 4e-3 (the GPU consumes bf16(s X A^T) and
bf16(s dY B), as the forward and input-gradient GEMMs do)."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import check_close, dev, to_gpu_bf16

pytestmark = pytest.mark.gpu

CASES = [
    WL.CONFIGS["tiny"],
    WL.custom("ragged", 320, 192, 300, 100, s=1.5),
    WL.custom("r1", 64, 64, 5, 1, s=0.5),
    WL.custom("r256", 128, 256, 2, 256, s=2.0),
    WL.custom("tall", 576, 128, 513, 64, s=1.0),       # odd token count: a last unpaired token
    WL.custom("one_token", 192, 320, 1, 8, s=2.0),
    WL.custom("r33", 256, 448, 77, 33, s=0.75),
    WL.custom("r24", 320, 256, 129, 24, s=1.25),       # U' pre-pass reads B itself (r % 8 == 0, r <= 32)
    WL.custom("r32", 128, 192, 64, 32, s=0.5),
    WL.CONFIGS["prefill"],
    WL.CONFIGS["mlp_up"],
]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_lora_grads_match_oracle(cfg):
    _say(f"[lora_grads] {cfg.name} d_out={cfg.d_out} d_in={cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}")
    a, b = WL.make_lora(cfg)
    x, dy = WL.make_x(cfg), WL.make_dy(cfg)
    dA, dB = qn.lora_grads(to_gpu_bf16(a), to_gpu_bf16(b), cfg.s, to_gpu_bf16(x), to_gpu_bf16(dy))
    torch.cuda.synchronize()
    rA, rB = O.lora_grads(a, b, cfg.s, x, dy)
    check_close(dA.cpu().numpy().astype(np.float64), rA, f"dA {cfg.name}")
    check_close(dB.cpu().numpy().astype(np.float64), rB, f"dB {cfg.name}")


def test_lora_grads_deterministic_and_zero_b():
    cfg = WL.custom("det", 256, 512, 333, 16, s=2.0)
    a, b = WL.make_lora(cfg)
    x, dy = WL.make_x(cfg), WL.make_dy(cfg)
    A, B, X, dY = to_gpu_bf16(a), to_gpu_bf16(b), to_gpu_bf16(x), to_gpu_bf16(dy)
    g1 = qn.lora_grads(A, B, cfg.s, X, dY)
    g2 = qn.lora_grads(A, B, cfg.s, X, dY)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])
    # B = 0 (the usual initialisation): dA is exactly zero
    dA, dB = qn.lora_grads(A, torch.zeros_like(B), cfg.s, X, dY)
    torch.cuda.synchronize()
    assert not torch.any(dA)
    rA, rB = O.lora_grads(a, np.zeros_like(b), cfg.s, x, dy)
    check_close(dB.cpu().numpy().astype(np.float64), rB, "dB with B = 0")
