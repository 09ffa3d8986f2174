"""Seeded random sweep of layer shapes through the C ABI against the oracle (forward,
input gradient and adapter gradients, full outputs): token counts on both sides of every dispatch boundary (1,
2..64, 65+; whole and K-split GEMMs; K-split pre-pass), ranks 1..256 and the three
second-level formats."""
import random

import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import bf16_f64, check_close, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=2024):
    rng = random.Random(seed)
    seqs = [1, 2, 3, 15, 16, 17, 33, 63, 64, 65, 100, 129, 257, 300, 511, 700,
            4, 8, 31, 32, 48, 96, 128, 192, 255, 256, 384, 1000, 1024, 5, 7, 9]
    out = []
    for k in range(n):
        d_out = 64 * rng.randint(1, 24)
        d_in = 64 * rng.randint(1, 40)
        d_seq = seqs[k % len(seqs)]
        r = rng.choice([1, 3, 8, 16, 31, 33, 64, 100, 256])
        dq = ("int8", "fp8", "none")[k % 3]
        out.append((d_out, d_in, d_seq, r, dq, round(rng.uniform(0.25, 2.0), 3)))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{a}x{b}_t{c}_r{d}_{e}" for a, b, c, d, e, _ in CASES])
def test_random_shapes(case):
    d_out, d_in, d_seq, r, dq, s = case
    print(f"[sweep] {d_out}x{d_in} d_seq={d_seq} r={r} dq={dq} s={s}", flush=True)
    cfg = WL.custom("sweep", d_out, d_in, d_seq, r, s=s)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w), dq=dq)
    ref = O.quantize(w, dq=dq)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], d_out, d_in, dq=dq)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    x, dy = WL.make_x(cfg), WL.make_dy(cfg)
    y = qn.linear_fwd(q, A, B, s, to_gpu_bf16(x))
    dx = qn.linear_bwd_x(q, A, B, s, to_gpu_bf16(dy))
    torch.cuda.synchronize()
    check_close(bf16_f64(y), O.linear_fwd(wh, a, b, s, x), f"fwd {case}")
    check_close(bf16_f64(dx), O.linear_bwd_x(wh, a, b, s, dy), f"bwd_x {case}")
    dA, dB = qn.lora_grads(A, B, s, to_gpu_bf16(x), to_gpu_bf16(dy))
    torch.cuda.synchronize()
    rA, rB = O.lora_grads(a, b, s, x, dy)
    check_close(dA.cpu().numpy().astype(np.float64), rA, f"dA {case}")
    check_close(dB.cpu().numpy().astype(np.float64), rB, f"dB {case}")
