"""GPU checks of the leading-dimension arguments (ldx, ldy, lddy, lddx) of the C ABI.

The pages' sequence input x in R^{d_in x d_seq} (whoami-wesleyyou.top "LoRA") may be
a slice of a wider activation array. Each call below reads its activation from a
column window of a wider buffer and writes its output into a column window of
another, and must give the same bits as the call on contiguous arrays, while the
elements of the wider buffers outside the windows stay as they were. Every
dispatch path is covered: the GEMV (1, 2 and 3 tokens), the small-batch kernel,
the whole and the K-split GEMM, the input gradient, the adapter gradients and the
quantised-factor forward.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from parity import bf16_f64, check_close, dev, to_gpu_bf16, to_gpu_f32
from oracle import nf4_oracle as O

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0   # exactly representable in bf16

CASES = [
    WL.custom("gemv_1", 256, 1024, 1, 16),
    WL.custom("gemv_two_launch", 192, 4160, 1, 24),
    WL.custom("gemv_2", 320, 960, 2, 5),
    WL.custom("gemv_3", 128, 4096, 3, 16),
    WL.custom("small_16", 256, 1024, 16, 16),
    WL.custom("small_40", 192, 2048, 40, 33),
    WL.custom("gemm_200", 512, 1024, 200, 16),
    WL.custom("gemm_split", 512, 4096, 130, 64),
]


def _window(rows, cols, pad_lo, pad_hi, values: torch.Tensor | None = None):
    """A [rows, pad_lo + cols + pad_hi] bf16 buffer filled with SENTINEL and the
    [rows, cols] view at column pad_lo (optionally holding `values`)."""
    buf = torch.full((rows, pad_lo + cols + pad_hi), SENTINEL, dtype=torch.bfloat16, device=dev())
    view = buf[:, pad_lo:pad_lo + cols]
    if values is not None:
        view.copy_(values)
    return buf, view


def _outside_untouched(buf: torch.Tensor, pad_lo: int, cols: int) -> bool:
    keep = torch.ones_like(buf, dtype=torch.bool)
    keep[:, pad_lo:pad_lo + cols] = False
    return bool((buf[keep] == SENTINEL).all())


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_forward_and_input_gradient_on_strided_views(cfg):
    print(f"[strides] {cfg.name} d_out={cfg.d_out} d_in={cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}", flush=True)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w))
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = to_gpu_bf16(WL.make_x(cfg))
    dY = to_gpu_bf16(WL.make_dy(cfg))

    y_ref = qn.linear_fwd(q, A, B, cfg.s, X)
    dx_ref = qn.linear_bwd_x(q, A, B, cfg.s, dY)

    _, Xv = _window(cfg.d_seq, cfg.d_in, 64, 40, X)               # ldx = d_in + 104
    ybuf, Yv = _window(cfg.d_seq, cfg.d_out, 8, 72)               # ldy = d_out + 80
    qn.linear_fwd(q, A, B, cfg.s, Xv, out=Yv)
    _, dYv = _window(cfg.d_seq, cfg.d_out, 24, 8, dY)
    dxbuf, dXv = _window(cfg.d_seq, cfg.d_in, 136, 0)
    qn.linear_bwd_x(q, A, B, cfg.s, dYv, out=dXv)
    torch.cuda.synchronize()

    assert Xv.stride(0) == cfg.d_in + 104 and Yv.stride(0) == cfg.d_out + 80
    assert torch.equal(Yv.view(torch.int16), y_ref.view(torch.int16)), "forward on strided views"
    assert torch.equal(dXv.view(torch.int16), dx_ref.view(torch.int16)), "input gradient on strided views"
    assert _outside_untouched(ybuf, 8, cfg.d_out), "the forward wrote outside its output window"
    assert _outside_untouched(dxbuf, 136, cfg.d_in), "the input gradient wrote outside its output window"


def test_strided_forward_against_the_oracle():
    """The strided small-batch forward against the float64 oracle as well (the strided
    call equals the contiguous one above; this ties it to the pages' formula)."""
    cfg = WL.custom("strided_oracle", 256, 512, 24, 8, s=1.5)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    x = WL.make_x(cfg)
    q = qn.quantize(to_gpu_f32(w))
    _, Xv = _window(cfg.d_seq, cfg.d_in, 16, 16, to_gpu_bf16(x))
    ybuf, Yv = _window(cfg.d_seq, cfg.d_out, 0, 64)
    qn.linear_fwd(q, to_gpu_bf16(a), to_gpu_bf16(b), cfg.s, Xv, out=Yv)
    torch.cuda.synchronize()
    ref = O.quantize(w)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in)
    check_close(bf16_f64(Yv.contiguous()), O.linear_fwd(wh, a, b, cfg.s, x), "strided forward")
    assert _outside_untouched(ybuf, 0, cfg.d_out)


@pytest.mark.parametrize("shape", [(256, 512, 100, 16), (192, 320, 33, 40)], ids=["r16", "r40"])
def test_adapter_gradients_on_strided_views(shape):
    d_out, d_in, d_seq, r = shape
    print(f"[strides] lora grads {shape}", flush=True)
    cfg = WL.custom("g", d_out, d_in, d_seq, r)
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = to_gpu_bf16(WL.make_x(cfg))
    dY = to_gpu_bf16(WL.make_dy(cfg))
    dA0, dB0 = qn.lora_grads(A, B, 1.5, X, dY)
    _, Xv = _window(d_seq, d_in, 64, 64, X)
    _, dYv = _window(d_seq, d_out, 8, 0, dY)
    dA1, dB1 = qn.lora_grads(A, B, 1.5, Xv, dYv)
    torch.cuda.synchronize()
    assert torch.equal(dA0, dA1) and torch.equal(dB0, dB1)


def test_quantised_factor_forward_on_strided_views():
    cfg = WL.custom("qlr", 256, 1024, 96, 16)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w))
    Af = qn.quantize_factor(to_gpu_f32(O.bf16_bits_to_f32(a)), 8)
    Bf = qn.quantize_factor(to_gpu_f32(O.bf16_bits_to_f32(b)), 4)
    X = to_gpu_bf16(WL.make_x(cfg))
    y0 = qn.qlr_linear_fwd(q, Af, Bf, 1.0, X)
    _, Xv = _window(cfg.d_seq, cfg.d_in, 8, 8, X)
    ybuf, Yv = _window(cfg.d_seq, cfg.d_out, 64, 64)
    qn.qlr_linear_fwd(q, Af, Bf, 1.0, Xv, out=Yv)
    torch.cuda.synchronize()
    assert torch.equal(Yv.view(torch.int16), y0.view(torch.int16))
    assert _outside_untouched(ybuf, 64, cfg.d_out)


def test_row_stride_not_a_multiple_of_8_is_rejected():
    cfg = WL.custom("bad_ld", 64, 64, 4, 8)
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    buf = torch.zeros(4, 68, dtype=torch.bfloat16, device=dev())
    with pytest.raises(qn.QLoRAError):
        qn.linear_fwd(q, to_gpu_bf16(a), to_gpu_bf16(b), 1.0, buf[:, :64])
