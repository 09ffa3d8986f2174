"""GPU parity of the forward GEMM that forms W_hat inside the kernel (qlora_set_fwd_gemm
QN_FWD_GEMM_FUSED) against the form that stages W_hat in the workspace.

Both forms multiply the same bf16 weights (learn.ifs.name deck, card 1: the 4-bit weights
become BF16 for the matrix product; page 4 "QLoRA", doubleDequant) in the same MFMA order,
so their outputs must be the same bits; the staged form is itself checked against the
oracle in test_gpu_parity.py and test_gpu_full_size.py, and a few fused cases are checked
against the oracle here as well. Shapes cover: a single K-step (d_in = 64), odd and even
numbers of dequantising steps, ragged token and output tiles, the K-split path (at most
128 output tiles), LoRA ranks from 1 to 256 (one to four LoRA steps), all three
second-level formats, row-strided X and Y, and the full-size layers the benchmark times.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import bf16_f64, check_close, dev, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _restore_form():
    prev = qn.set_fwd_gemm(qn.FWD_GEMM_AUTO)
    yield
    qn.set_fwd_gemm(prev)


def _both_forms(q, A, B, s, X, **kw):
    qn.set_fwd_gemm(qn.FWD_GEMM_STAGED)
    y_staged = qn.linear_fwd(q, A, B, s, X, **kw).clone()
    qn.set_fwd_gemm(qn.FWD_GEMM_FUSED)
    y_fused = qn.linear_fwd(q, A, B, s, X, **kw)
    torch.cuda.synchronize()
    return y_staged, y_fused


def _assert_same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    ai, bi = a.view(torch.int16), b.view(torch.int16)
    diff = int((ai != bi).sum())
    assert diff == 0, f"{what}: {diff} of {a.numel()} outputs differ between the fused and staged forms"


# (name, d_out, d_in, d_seq, r, s, dq)
CASES = [
    ("k64_one_step", 256, 64, 100, 8, 2.0, "int8"),
    ("k128_two_steps", 320, 128, 77, 16, 1.5, "int8"),
    ("k192_three_steps", 192, 192, 65, 4, 0.5, "int8"),
    ("ragged_tiles", 576, 448, 300, 33, 1.5, "int8"),
    ("r1", 256, 512, 129, 1, 2.0, "int8"),
    ("r64", 512, 1024, 257, 64, 1.0, "int8"),
    ("r256", 256, 768, 96, 256, 0.75, "int8"),
    ("split_2_tiles", 512, 4096, 200, 16, 2.0, "int8"),     # 2 tiles: K split over 4 workgroups
    ("split_12_tiles", 1536, 1536, 300, 33, 1.5, "int8"),   # 12 tiles: 3 splits
    ("split_odd_k", 384, 4160, 130, 24, 1.0, "int8"),       # 65 K-steps over the splits
    ("fp8", 448, 640, 150, 16, 2.0, "fp8"),
    ("no_second_level", 448, 640, 150, 16, 2.0, "none"),
    ("fp8_split", 512, 2048, 90, 64, 0.5, "fp8"),
    ("outliers", 1024, 1024, 512, 16, 2.0, "int8"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_staged(case):
    name, d_out, d_in, d_seq, r, s, dq = case
    _say(f"[fused fwd] {name} d_out={d_out} d_in={d_in} d_seq={d_seq} r={r} dq={dq}")
    cfg = WL.custom(name, d_out, d_in, d_seq, r, s=s, outlier_frac=0.001 if name == "outliers" else 0.0)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w), dq=dq)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    x = WL.make_x(cfg)
    y_staged, y_fused = _both_forms(q, A, B, s, to_gpu_bf16(x))
    _assert_same_bits(y_fused, y_staged, name)
    if name in ("k64_one_step", "ragged_tiles", "fp8", "no_second_level", "split_odd_k"):
        ref = O.quantize(w, dq=dq)
        wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], d_out, d_in, dq=dq)
        check_close(bf16_f64(y_fused), O.linear_fwd(wh, a, b, s, x), f"fused fwd {name}")


def test_fused_strided_views():
    d_out, d_in, d_seq, r = 640, 512, 200, 16
    _say(f"[fused fwd] strided X and Y {d_out}x{d_in} d_seq={d_seq}")
    cfg = WL.custom("strided", d_out, d_in, d_seq, r, s=1.25)
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    xw = torch.randn(d_seq, d_in + 72, device=dev()).to(torch.bfloat16)
    X = xw[:, 40:40 + d_in]
    outs = []
    for form in (qn.FWD_GEMM_STAGED, qn.FWD_GEMM_FUSED):
        qn.set_fwd_gemm(form)
        yw = torch.full((d_seq, d_out + 24), 7.0, device=dev(), dtype=torch.bfloat16)
        qn.linear_fwd(q, A, B, 1.25, X, out=yw[:, 16:16 + d_out])
        torch.cuda.synchronize()
        assert bool((yw[:, :16] == 7.0).all()) and bool((yw[:, 16 + d_out:] == 7.0).all()), "wrote outside Y"
        outs.append(yw[:, 16:16 + d_out].clone())
    _assert_same_bits(outs[1], outs[0], "strided")


def test_fused_result_is_independent_of_a_previous_call():
    """The kernel keeps no state between calls: a second call on another layer gives the
    same bits as a first call on it in a fresh order."""
    cfgs = [WL.custom("p", 512, 1024, 300, 16, s=2.0, seed=3), WL.custom("q", 768, 512, 260, 8, s=1.0, seed=4)]
    layers = []
    for c in cfgs:
        q = qn.quantize(to_gpu_f32(WL.make_weight(c)))
        a, b = WL.make_lora(c)
        layers.append((q, to_gpu_bf16(a), to_gpu_bf16(b), c.s, to_gpu_bf16(WL.make_x(c))))
    qn.set_fwd_gemm(qn.FWD_GEMM_FUSED)
    first = [qn.linear_fwd(*L).clone() for L in layers]
    again = [qn.linear_fwd(*L).clone() for L in reversed(layers)][::-1]
    torch.cuda.synchronize()
    for u, v, c in zip(first, again, cfgs):
        _assert_same_bits(u, v, c.name)


@pytest.mark.parametrize("cfg_name,d_seq", [("prefill", None), ("mlp_up", None), ("mlp_down", None), ("large", None),
                                            ("large", 512), ("large", 1000)])
def test_fused_equals_staged_full_size(cfg_name, d_seq):
    cfg = WL.CONFIGS[cfg_name]
    if d_seq is not None:
        cfg = WL.custom(f"{cfg.name}_{d_seq}tok", cfg.d_out, cfg.d_in, d_seq, cfg.r, s=cfg.s, w_sigma=cfg.w_sigma)
    _say(f"[fused fwd] full size {cfg.name} {cfg.d_out}x{cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}")
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = torch.randn(cfg.d_seq, cfg.d_in, device=dev(), generator=torch.Generator(device=dev()).manual_seed(5)
                    ).to(torch.bfloat16)
    y_staged, y_fused = _both_forms(q, A, B, cfg.s, X)
    _assert_same_bits(y_fused, y_staged, cfg.name)


def test_auto_form_follows_the_shape_rule():
    """AUTO takes the fused form for a weight of 2^27 or more elements at up to 1024 tokens
    and stages W_hat otherwise; either way the result is the same bits as staged."""
    cfg = WL.custom("auto_large", 16384, 8192, 300, 16, s=1.0)
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = to_gpu_bf16(WL.make_x(cfg))
    qn.set_fwd_gemm(qn.FWD_GEMM_AUTO)
    qn.profile_enable(True)
    y_auto = qn.linear_fwd(q, A, B, cfg.s, X).clone()
    torch.cuda.synchronize()
    kernels = qn.profile_read()
    qn.profile_enable(False)
    assert any(k.startswith("gemm_nf4") for k in kernels), f"AUTO did not take the fused form: {sorted(kernels)}"
    y_staged, _ = _both_forms(q, A, B, cfg.s, X)
    _assert_same_bits(y_auto, y_staged, cfg.name)
