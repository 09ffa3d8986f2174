"""GPU parity of the second-level formats other than INT8, through the C ABI:
FP8 E4M3 codes of the centred block constants and no second level (a_j per block).

Bit-exact: codes, second-level codes, scales, the mean, the dequantised bf16 weight
(every small case of the INT8 suite, plus a group whose scaled constants land on and
next to E4M3 values and midpoints). Tolerance (parity.py): the forward on each of its
three paths (GEMV, small batch, dequantise + GEMM) and the input gradient."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import bf16_bits, bf16_f64, check_close, dev, to_gpu_bf16, to_gpu_f32
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

FORMATS = ["fp8", "none"]


def _say(*a):
    print(*a, flush=True)


def _quant(w: np.ndarray, dq: str):
    q = qn.quantize(to_gpu_f32(w), dq=dq)
    torch.cuda.synchronize()
    return q


def _assert_equal(q, ref):
    assert q.dq == ref["dq"]
    assert np.array_equal(q.codes.cpu().numpy(), ref["codes"]), "codes"
    assert np.array_equal(q.qscale.cpu().numpy().view(np.uint32), ref["qscale"].view(np.uint32)), "qscale"
    if ref["dq"] == "none":
        assert q.qconst.numel() == 0 and q.qmean.numel() == 0
    else:
        assert np.array_equal(q.qconst.cpu().numpy().view(np.uint8), ref["qconst"].view(np.uint8)), "qconst"
        assert np.array_equal(q.qmean.cpu().numpy().view(np.uint32), ref["qmean"].view(np.uint32)), "qmean"


def _e4m3_stress_weight():
    """One group of 256 blocks (block j = row j) with absmax a = 1 +- m 2^-12, m running
    over E4M3 values and midpoints up to 448: the mean is exactly 1, b = 448 2^-12, so
    the scaled constants r * 448 fall on or within a rounding of E4M3 values and ties."""
    v = O.e4m3_values()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2
    m = np.concatenate([v[1::2], mids[::2], [v[2], 448.0]])       # 63 + 63 + 2 = 128 pairs
    a = np.concatenate([1 + m * 2.0 ** -12, 1 - m * 2.0 ** -12]).astype(np.float32)
    shape = np.linspace(-1, 1, 63).astype(np.float32)
    w = np.empty((256, 64), np.float32)
    w[:, 0] = a
    w[:, 1:] = a[:, None] * shape[None, :] * np.float32(0.999)
    return w


CASES = SMALL + [("e4m3_ties_256x64", _e4m3_stress_weight)]


@pytest.mark.parametrize("dq", FORMATS)
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_quantize_and_dequant_bit_exact(dq, name, make):
    w = make()
    _say(f"[quantize {dq}] {name} shape={w.shape}")
    q = _quant(w, dq)
    ref = O.quantize(w, dq=dq)
    _assert_equal(q, ref)
    wh = qn.double_dequant(q)
    torch.cuda.synchronize()
    want = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], *w.shape, dq=dq)
    assert np.array_equal(bf16_bits(wh), want)


def test_e4m3_stress_weight_hits_ties():
    # the stress group really exercises the FP8 rounding: several scaled constants sit
    # exactly on an E4M3 value and others within one float32 ulp of a midpoint
    w = _e4m3_stress_weight()
    a = O.block_absmax(O.to_blocks(w))
    mu = O.exact_mean_f32(a)
    assert mu == np.float32(1.0)
    d = (a - mu).astype(np.float32)
    r = (d / np.max(np.abs(d))).astype(np.float32)
    s = np.abs((r * np.float32(448)).astype(np.float32)).astype(np.float64)
    v = O.e4m3_values()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2
    on_value = np.isin(s, v)
    near_mid = np.min(np.abs(s[:, None] - mids[None, :]) / np.maximum(s[:, None], 1e-30), axis=1) < 2 ** -22
    assert on_value.sum() >= 16 and near_mid.sum() >= 16


LINEAR = [
    WL.custom("f_gemv", 256, 1024, 1, 16, s=2.0),             # one 4096-weight segment per row
    WL.custom("f_gemv_ragged", 192, 4160, 1, 3, s=1.0),       # two segments, the last 64 wide
    WL.custom("f_sb_9", 256, 4160, 9, 8, s=2.0),
    WL.custom("f_sb_40", 128, 2048, 40, 64, s=1.0, outlier_frac=0.01),
    WL.custom("f_gemm", 320, 512, 200, 16, s=1.5),
]


@pytest.mark.parametrize("dq", FORMATS)
@pytest.mark.parametrize("cfg", LINEAR, ids=[c.name for c in LINEAR])
def test_linear_fwd_bwd(dq, cfg):
    _say(f"[linear {dq}] {cfg.name} d_out={cfg.d_out} d_in={cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}")
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = _quant(w, dq)
    ref = O.quantize(w, dq=dq)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in, dq=dq)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    x = WL.make_x(cfg)
    y = qn.linear_fwd(q, A, B, cfg.s, to_gpu_bf16(x))
    dy = WL.make_dy(cfg)
    dx = qn.linear_bwd_x(q, A, B, cfg.s, to_gpu_bf16(dy))
    torch.cuda.synchronize()
    check_close(bf16_f64(y), O.linear_fwd(wh, a, b, cfg.s, x), f"fwd {dq} {cfg.name}")
    check_close(bf16_f64(dx), O.linear_bwd_x(wh, a, b, cfg.s, dy), f"bwd_x {dq} {cfg.name}")


@pytest.mark.parametrize("dq", FORMATS)
def test_identity_input_returns_dequantised_weight(dq):
    cfg = WL.custom("eye", 192, 256, 256, 8)
    w = WL.make_weight(cfg)
    a, _ = WL.make_lora(cfg)
    q = _quant(w, dq)
    ref = O.quantize(w, dq=dq)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in, dq=dq)
    zeroB = torch.zeros(cfg.d_out, cfg.r, dtype=torch.bfloat16, device=dev())
    y = qn.linear_fwd(q, to_gpu_bf16(a), zeroB, 2.0, torch.eye(cfg.d_in, dtype=torch.bfloat16, device=dev()))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_f64(y), O.bf16_bits_to_f32(wh).astype(np.float64).T)


@pytest.mark.parametrize("dq", FORMATS)
def test_decode_layer_full_size(dq):
    cfg = WL.CONFIGS["decode"]
    _say(f"[gemv {dq}] decode 4096x4096 d_seq=1 r=16, and 16 tokens")
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = _quant(w, dq)
    ref = O.quantize(w, dq=dq)
    _assert_equal(q, ref)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in, dq=dq)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    for d_seq in (1, 16):
        c = WL.custom("t", cfg.d_out, cfg.d_in, d_seq, cfg.r, s=cfg.s)
        x = WL.make_x(c)
        y = qn.linear_fwd(q, A, B, cfg.s, to_gpu_bf16(x))
        torch.cuda.synchronize()
        check_close(bf16_f64(y), O.linear_fwd(wh, a, b, cfg.s, x), f"fwd {dq} decode d_seq={d_seq}")
