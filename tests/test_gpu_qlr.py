"""GPU parity of the quantised low-rank factors (W ~ Q + L R with L, R at 4 or 8 bits:
gist.science "Sintesi Tecnica: GPTQ-intrinsic LoRA"), through the C ABI.

Bit-exact: the 8-bit block quantiser (codes and absmax) and both factor dequantisers.
Tolerance (parity.py): the forward with quantised factors on the GEMV, small-batch and
GEMM paths, against the oracle's float64 product on the same dequantised operands."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import bf16_bits, bf16_f64, check_close, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _ties():
    # block max 2: w = +-1 gives x * 127 = +-63.5 exactly, a tie that goes to the even +-64; -0.0 codes 0
    b = np.zeros((2, 64), np.float32)
    b[0, 0], b[0, 1], b[0, 2], b[0, 3] = 2.0, 1.0, -1.0, -0.0
    b[1, :] = np.linspace(-3, 3, 64).astype(np.float32)
    return b


INT8_CASES = [
    ("a_16x4096", lambda: (np.random.default_rng(1).standard_normal((16, 4096)) * 0.01).astype(np.float32)),
    ("b_4096x16", lambda: (np.random.default_rng(2).standard_normal((4096, 16)) * 0.01).astype(np.float32)),
    ("ragged_3x50", lambda: (np.random.default_rng(3).standard_normal((3, 50))).astype(np.float32)),
    ("one_1x1", lambda: np.array([[-0.3]], np.float32)),
    ("zeros_8x64", lambda: np.zeros((8, 64), np.float32)),
    ("ties", _ties),
    ("wide_range_40x256", lambda: ((np.random.default_rng(4).standard_normal((40, 256))) * np.exp(
        np.random.default_rng(5).uniform(-30, 30, (40, 1)))).astype(np.float32)),
]


@pytest.mark.parametrize("name,make", INT8_CASES, ids=[c[0] for c in INT8_CASES])
def test_int8_quantize_and_dequant_bit_exact(name, make):
    w = make()
    _say(f"[int8] {name} {w.shape}")
    q, a = qn.int8_quantize(to_gpu_f32(w))
    wh = qn.int8_dequant(q, a, *w.shape)
    torch.cuda.synchronize()
    rq, ra = O.int8_quantize(w)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(bf16_bits(wh), O.int8_dequant(rq, ra, *w.shape))


@pytest.mark.parametrize("bits", [4, 8])
def test_factor_dequant_bit_exact(bits):
    cfg = WL.custom("f", 512, 1024, 1, 16)
    a, b = WL.make_lora(cfg)
    for m in (O.bf16_bits_to_f32(a), O.bf16_bits_to_f32(b)):
        f = qn.quantize_factor(to_gpu_f32(m), bits)
        got = qn.dequant_factor(f)
        torch.cuda.synchronize()
        codes, sc = O.quantize_factor(m, bits)
        assert np.array_equal(f.codes.cpu().numpy().view(np.uint8), codes.view(np.uint8))
        assert np.array_equal(f.scale.cpu().numpy().view(np.uint32), sc.view(np.uint32))
        assert np.array_equal(bf16_bits(got), O.dequant_factor(codes, sc, bits, *m.shape))


QLR = [
    WL.custom("qlr_gemv", 256, 1024, 1, 16, s=1.0),
    WL.custom("qlr_sb", 320, 2048, 9, 64, s=1.0),
    WL.custom("qlr_gemm", 192, 512, 200, 8, s=2.0),
]


@pytest.mark.parametrize("bits", [(4, 4), (8, 8), (4, 8), (8, 4)], ids=lambda b: f"A{b[0]}B{b[1]}")
@pytest.mark.parametrize("cfg", QLR, ids=[c.name for c in QLR])
def test_qlr_forward(cfg, bits):
    _say(f"[qlr] {cfg.name} d_out={cfg.d_out} d_in={cfg.d_in} d_seq={cfg.d_seq} r={cfg.r} bits={bits}")
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    af, bfl = O.bf16_bits_to_f32(a), O.bf16_bits_to_f32(b)
    q = qn.quantize(to_gpu_f32(w))
    Af = qn.quantize_factor(to_gpu_f32(af), bits[0])
    Bf = qn.quantize_factor(to_gpu_f32(bfl), bits[1])
    x = WL.make_x(cfg)
    y = qn.qlr_linear_fwd(q, Af, Bf, cfg.s, to_gpu_bf16(x))
    torch.cuda.synchronize()
    ref = O.quantize(w)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in)
    ah = O.dequant_factor(*O.quantize_factor(af, bits[0]), bits[0], cfg.r, cfg.d_in)
    bh = O.dequant_factor(*O.quantize_factor(bfl, bits[1]), bits[1], cfg.d_out, cfg.r)
    check_close(bf16_f64(y), O.linear_fwd(wh, ah, bh, cfg.s, x), f"qlr fwd {cfg.name} {bits}")


def test_qlr_forward_fp8_weight_full_layer():
    cfg = WL.CONFIGS["decode"]
    _say("[qlr] 4096x4096, FP8 second level, 8-bit factors, d_seq 1 and 16")
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    af, bfl = O.bf16_bits_to_f32(a), O.bf16_bits_to_f32(b)
    q = qn.quantize(to_gpu_f32(w), dq="fp8")
    Af, Bf = qn.quantize_factor(to_gpu_f32(af), 8), qn.quantize_factor(to_gpu_f32(bfl), 8)
    ref = O.quantize(w, dq="fp8")
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in, dq="fp8")
    ah = O.dequant_factor(*O.quantize_factor(af, 8), 8, cfg.r, cfg.d_in)
    bh = O.dequant_factor(*O.quantize_factor(bfl, 8), 8, cfg.d_out, cfg.r)
    for d_seq in (1, 16):
        x = WL.make_x(WL.custom("t", cfg.d_out, cfg.d_in, d_seq, cfg.r))
        y = qn.qlr_linear_fwd(q, Af, Bf, cfg.s, to_gpu_bf16(x))
        torch.cuda.synchronize()
        check_close(bf16_f64(y), O.linear_fwd(wh, ah, bh, cfg.s, x), f"qlr fwd 4096 d_seq={d_seq}")
