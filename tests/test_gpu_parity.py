"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: NF4 codes, INT8 constant codes, group scales, the mean, dequantised
bf16 weights. Tolerance (see parity.py): forward and input-gradient products.
Small and ragged shapes are checked in full here, as is the 4096 x 4096 decode
GEMV; the other full-size layers are in test_gpu_full_size.py.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import bf16_bits, bf16_f64, check_close, dev, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _normal(shape, seed, sigma=0.02):
    return (np.random.default_rng(seed).standard_normal(shape) * sigma).astype(np.float32)


def _gpu_quantize(w: np.ndarray):
    q = qn.quantize(to_gpu_f32(w))
    torch.cuda.synchronize()
    return q


def _assert_quant_equal(q, ref):
    assert np.array_equal(q.qmean.cpu().numpy().view(np.uint32), ref["qmean"].view(np.uint32)), "qmean"
    assert np.array_equal(q.qscale.cpu().numpy().view(np.uint32), ref["qscale"].view(np.uint32)), "qscale"
    assert np.array_equal(q.qconst.cpu().numpy(), ref["qconst"]), "qconst"
    assert np.array_equal(q.codes.cpu().numpy(), ref["codes"]), "codes"


def _tie_matrix():
    """Blocks whose normalised values sit exactly on, just below and just above
    every code midpoint, plus -0.0, subnormals, tiny and huge absmax blocks."""
    cb = O.codebook().astype(np.float64)
    vals = []
    for k in range(15):
        m = np.float32((cb[k] + cb[k + 1]) / 2)
        vals += [m, np.nextafter(m, np.float32(-2)), np.nextafter(m, np.float32(2))]
    vals = np.array(vals, np.float32)                       # 45 values in [-1, 1]
    rows = []
    for scale in (1.0, 0.5, 3.0e-3, 1.0e30, 1.0e-36):
        b = np.zeros(64, np.float32)
        b[0] = 1.0
        b[1:46] = vals
        b[46] = -0.0
        b[47] = -1.0
        b[48] = 1e-45
        rows.append((b * np.float32(scale)).astype(np.float32))
    rows.append(np.full(64, -0.0, np.float32))                # all -0: absmax 0
    rows.append(np.full(64, 7.0e-45, np.float32))             # subnormal absmax
    rows.append(np.linspace(-1, 1, 64).astype(np.float32))
    return np.stack(rows)


SMALL = [
    ("tiny_256x256", lambda: WL.make_weight(WL.CONFIGS["tiny"])),
    ("ragged_3x50", lambda: _normal((3, 50), 1)),
    ("one_1x1", lambda: np.array([[0.7]], np.float32)),
    ("ragged_100x37", lambda: _normal((100, 37), 2)),
    ("partial_group_1000x67", lambda: _normal((1000, 67), 3)),
    ("rows_64x16448", lambda: _normal((64, 64 * 257), 4)),
    ("tail_5x32771", lambda: _normal((5, 32771), 5)),
    ("zeros_128x128", lambda: np.zeros((128, 128), np.float32)),
    ("constant_64x256", lambda: np.full((64, 256), 0.5, np.float32)),
    ("ties_and_specials", _tie_matrix),
    ("outliers_512x1024", lambda: WL.make_weight(WL.custom("o", 512, 1024, 1, 8, outlier_frac=0.001))),
    ("wide_range_300x512", lambda: (_normal((300, 512), 6) * np.exp(
        np.random.default_rng(7).uniform(-40, 40, (300, 1))).astype(np.float32)).astype(np.float32)),
]


@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_quantize_and_dequant_bit_exact_small(name, make):
    w = make()
    _say(f"[quantize] {name} shape={w.shape}")
    q = _gpu_quantize(w)
    ref = O.quantize(w)
    _assert_quant_equal(q, ref)
    wh = qn.double_dequant(q)
    torch.cuda.synchronize()
    want = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], *w.shape)
    assert np.array_equal(bf16_bits(wh), want)


_F = np.float32
MEAN_CASES = [   # block absmax values, the float32 nearest their mean (ties to even)
    ([2.0, 2.0 ** -23], 1.0),                                     # exactly halfway: 1 + 2^-24
    ([2.0 + 2.0 ** -22, 2.0 ** -23], 1.0 + 2.0 ** -22),           # halfway between 1 + 2^-23 and 1 + 2^-22
    ([2.0, 2.0 ** -23 + 2.0 ** -46], 1.0 + 2.0 ** -23),           # 2^-47 above halfway
    ([2.0, 2.0 ** -23 - 2.0 ** -47], 1.0),                        # 2^-48 below halfway
    ([1.0, 1.0, 1.0 + 2.0 ** -23], 1.0),                          # a third of an ulp above 1
    ([2.0 ** -149, 0.0], 0.0),                                    # subnormal: halfway between 0 and 2^-149
    ([3 * 2.0 ** -149, 0.0], 2.0 ** -148),                        # halfway between 2^-149 and 2^-148
    ([2.0 ** -149] * 3 + [0.0], 2.0 ** -149),
    ([float(np.finfo(np.float32).max)] * 2, float(np.finfo(np.float32).max)),
]


@pytest.mark.parametrize("k", range(len(MEAN_CASES)))
def test_mean_rounding_at_midpoints(k):
    """The mean of the block constants at, and within far less than an ulp of, float32
    rounding midpoints (normal and subnormal), where the kernel cannot decide from a
    float64 estimate and has to divide the exact integer sum."""
    absmax, want = MEAN_CASES[k]
    pattern = np.linspace(-0.9, 0.9, 64).astype(np.float32)
    pattern[5] = 1.0
    w = np.stack([(pattern * _F(a)).astype(np.float32) for a in absmax])
    assert [float(np.abs(r).max()) for r in w] == [float(_F(a)) for a in absmax]
    _say(f"[mean] case {k}: {len(absmax)} blocks")
    q = _gpu_quantize(w)
    ref = O.quantize(w)
    assert ref["qmean"].view(np.uint32)[0] == np.array([want], np.float32).view(np.uint32)[0]
    _assert_quant_equal(q, ref)


def test_quantize_is_deterministic_and_reusable():
    w = _normal((777, 320), 11)
    q1 = _gpu_quantize(w)
    q2 = qn.quantize(to_gpu_f32(w), out=qn.alloc_weight(777, 320, dev()))
    torch.cuda.synchronize()
    for a, b in ((q1.codes, q2.codes), (q1.qconst, q2.qconst), (q1.qscale, q2.qscale), (q1.qmean, q2.qmean)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


# ---------------------------------------------------------------- products

def _layer(cfg):
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    return w, a, b


def _fwd_bwd_full_check(cfg, check_bwd=True):
    w, a, b = _layer(cfg)
    q = _gpu_quantize(w)
    ref = O.quantize(w)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    x = WL.make_x(cfg)
    y = qn.linear_fwd(q, A, B, cfg.s, to_gpu_bf16(x))
    torch.cuda.synchronize()
    check_close(bf16_f64(y), O.linear_fwd(wh, a, b, cfg.s, x), f"fwd {cfg.name}")
    if check_bwd:
        dy = WL.make_dy(cfg)
        dx = qn.linear_bwd_x(q, A, B, cfg.s, to_gpu_bf16(dy))
        torch.cuda.synchronize()
        check_close(bf16_f64(dx), O.linear_bwd_x(wh, a, b, cfg.s, dy), f"bwd_x {cfg.name}")


LINEAR_SMALL = [
    WL.CONFIGS["tiny"],
    WL.custom("ragged", 320, 192, 300, 100, s=1.5),
    WL.custom("r1", 64, 64, 5, 1, s=0.5),
    WL.custom("r256", 128, 256, 2, 256, s=2.0),
    WL.custom("tall", 576, 128, 513, 64, s=1.0, outlier_frac=0.01),
    WL.custom("long_k", 256, 2048, 96, 16, s=2.0),
    WL.custom("gemv_small", 192, 320, 1, 8, s=2.0),
    WL.custom("gemv_r64", 512, 1024, 1, 64, s=1.0),
    WL.custom("gemv_ragged", 320, 4160, 1, 3, s=2.0),       # 3 column chunks, the last 64 wide
    WL.custom("gemv_wide", 128, 11008, 1, 256, s=0.5),      # 6 column chunks, r = 256
    WL.custom("gemv_k20480", 256, 20480, 1, 64, s=1.0),     # x beyond the persistent kernel's LDS: 5 segments per workgroup
    # one launch forms A x in every workgroup when r <= 16 and d_in <= 4096; else two launches
    WL.custom("gemv_one_r1_k64", 64, 64, 1, 1, s=2.0),
    WL.custom("gemv_one_r16_k4096", 192, 4096, 1, 16, s=1.5),
    WL.custom("gemv_one_r5_k960", 320, 960, 1, 5, s=0.5),
    WL.custom("gemv_two_r17_k4096", 192, 4096, 1, 17, s=1.5),
    # 2 and 3 tokens with r <= 16 and d_in <= 4096 take the GEMV (one code lookup for all tokens)
    WL.custom("gemv_tok2_r16_k4096", 1024, 4096, 2, 16, s=1.5),
    WL.custom("gemv_tok3_r5_k960", 320, 960, 3, 5, s=0.5),
    WL.custom("gemv_tok3_r16_k64", 64, 64, 3, 16, s=2.0),
    # at most 128 output tiles: the GEMM splits K over 2..4 workgroups per tile
    WL.custom("split_fwd", 512, 4096, 200, 16, s=2.0),       # fwd 2 tiles -> 4 splits
    WL.custom("split_bwd", 4096, 512, 130, 64, s=1.0),       # dX 2 tiles -> 4 splits, ragged tokens
    WL.custom("split_both", 1536, 1536, 300, 33, s=1.5),     # 12 tiles each way -> 3 splits
    # the dX pre-pass reads B itself when r % 8 == 0 and r <= 32, else a transpose of B
    WL.custom("bmajor_r24", 256, 320, 100, 24, s=1.5),
    WL.custom("bmajor_r32", 192, 448, 77, 32, s=0.75),
    WL.custom("btrans_r40", 192, 448, 77, 40, s=0.75),
    # pre-pass K-slices: side by side in the LoRA columns (r = 16, 4 slices; r = 12, 5
    # slices and 4 zero columns), or fp32 partials plus a reduction when 4 slices of a
    # long K would each be far longer than the split they replace (d_in = 16384 fwd)
    WL.custom("slices_cat_r16", 1024, 4096, 256, 16, s=1.25),
    WL.custom("slices_cat_r12", 512, 2048, 160, 12, s=0.5),
    WL.custom("slices_long_k", 512, 16384, 128, 16, s=2.0),
]


@pytest.mark.parametrize("cfg", LINEAR_SMALL, ids=[c.name for c in LINEAR_SMALL])
def test_linear_fwd_bwd_small(cfg):
    _say(f"[linear] {cfg.name} d_out={cfg.d_out} d_in={cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}")
    _fwd_bwd_full_check(cfg)


# 2 <= d_seq <= 64 runs the small-batch kernel (codes streamed once, dequantised in
# registers into 16x16x32 MFMAs): 1..4 token tiles, ragged token counts, K-slices
# that end inside a block pair (d_in 4160: 65 blocks), several K-splits per
# workgroup (d_in 11008: 22 slices over 8 splits), r up to 256; also a single block per
# row (d_in 64), block counts below one slice, ranks 1, 3, 7 and 17 (ragged rank tiles)
# and outlier weights at 16 tokens or fewer.
SMALL_BATCH = [
    WL.custom("sb_4_r1_k64", 64, 64, 4, 1, s=2.0),
    WL.custom("sb_9_r7_k192", 320, 192, 9, 7, s=0.5),
    WL.custom("sb_13_r3_k1280", 128, 1280, 13, 3, s=1.0),
    WL.custom("sb_16_r16_k4096", 1024, 4096, 16, 16, s=1.5),
    WL.custom("sb_5_r16_outliers", 448, 1024, 5, 16, s=2.0, outlier_frac=0.01),
    WL.custom("sb_16_r17", 256, 1024, 16, 17, s=1.0),
    WL.custom("sb_2", 128, 256, 2, 8, s=2.0),
    WL.custom("sb_15", 192, 4160, 15, 3, s=1.0),
    WL.custom("sb_16", 256, 1024, 16, 16, s=2.0),
    WL.custom("sb_17", 320, 512, 17, 64, s=0.5),
    WL.custom("sb_33", 128, 11008, 33, 16, s=2.0, outlier_frac=0.01),
    WL.custom("sb_48", 64, 2048, 48, 100, s=1.5),
    WL.custom("sb_64", 512, 768, 64, 256, s=1.0),
]


@pytest.mark.parametrize("cfg", SMALL_BATCH, ids=[c.name for c in SMALL_BATCH])
def test_small_batch_forward(cfg):
    _say(f"[small batch] {cfg.name} d_out={cfg.d_out} d_in={cfg.d_in} d_seq={cfg.d_seq} r={cfg.r}")
    _fwd_bwd_full_check(cfg, check_bwd=False)


def test_small_batch_forward_full_layer():
    base = WL.CONFIGS["decode"]
    cfg = WL.custom("decode_64tok", base.d_out, base.d_in, 64, base.r, s=base.s)
    _say("[small batch] 4096x4096 d_seq=64 r=16")
    _fwd_bwd_full_check(cfg, check_bwd=False)


# Every path must stay inside the workspace size the library reports for that call: the
# workspace is allocated with a guard region behind it, filled with a pattern that must
# survive the call (covers the GEMV, small-batch, whole and split GEMMs and the K-split
# pre-pass); the forward gets exactly qlora_linear_fwd_workspace_bytes (no W_hat region
# when it streams the codes), the input gradient qlora_linear_bwd_x_workspace_bytes.
GUARD_CASES = [(4096, 4096, 1, 16), (4096, 4096, 16, 16), (256, 2048, 65, 8), (512, 4096, 200, 16),
               (4096, 512, 130, 64), (1536, 1536, 300, 33), (320, 192, 300, 100), (11008, 4096, 2048, 64),
               (192, 4160, 1, 24), (4096, 4096, 3, 16), (1024, 2048, 64, 64)]


@pytest.mark.parametrize("shape", GUARD_CASES, ids=[f"{a}x{b}_t{c}_r{d}" for a, b, c, d in GUARD_CASES])
def test_calls_stay_inside_reported_workspace(shape):
    d_out, d_in, d_seq, r = shape
    _say(f"[workspace guard] {d_out}x{d_in} d_seq={d_seq} r={r}")
    cfg = WL.custom("g", d_out, d_in, d_seq, r)
    q = _gpu_quantize(_normal((d_out, d_in), 21))
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    guard = 1 << 20
    X = torch.randn(d_seq, d_in, device=dev()).to(torch.bfloat16)
    dY = torch.randn(d_seq, d_out, device=dev()).to(torch.bfloat16)
    for name, need, call in (
            ("forward", qn.linear_fwd_workspace_bytes(d_out, d_in, d_seq, r),
             lambda ws: qn.linear_fwd(q, A, B, cfg.s, X, workspace=ws)),
            ("input gradient", qn.linear_bwd_x_workspace_bytes(d_out, d_in, d_seq, r),
             lambda ws: qn.linear_bwd_x(q, A, B, cfg.s, dY, workspace=ws))):
        buf = torch.full((need + guard,), 0xAB, dtype=torch.uint8, device=dev())
        call(buf[:need])
        torch.cuda.synchronize()
        assert bool((buf[need:] == 0xAB).all()), f"the {name} wrote past its reported workspace"
    if d_seq <= 64:
        assert qn.linear_fwd_workspace_bytes(d_out, d_in, d_seq, r) < d_out * d_in, "no W_hat region when streaming"


def test_identity_input_returns_dequantised_weight_exactly():
    cfg = WL.custom("eye", 192, 256, 256, 8)
    w, a, b = _layer(cfg)
    q = _gpu_quantize(w)
    ref = O.quantize(w)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], cfg.d_out, cfg.d_in)
    A = to_gpu_bf16(a)
    zeroB = torch.zeros(cfg.d_out, cfg.r, dtype=torch.bfloat16, device=dev())
    eye_in = torch.eye(cfg.d_in, dtype=torch.bfloat16, device=dev())
    y = qn.linear_fwd(q, A, zeroB, 2.0, eye_in)           # Y[t, o] = W_hat[o, t]
    eye_out = torch.eye(cfg.d_out, dtype=torch.bfloat16, device=dev())
    dx = qn.linear_bwd_x(q, A, zeroB, 2.0, eye_out)        # dX[t, i] = W_hat[t, i]
    torch.cuda.synchronize()
    # compare values (+0 == -0): one nonzero product per dot product is exact
    assert np.array_equal(bf16_f64(y), O.bf16_bits_to_f32(wh).astype(np.float64).T)
    assert np.array_equal(bf16_f64(dx), O.bf16_bits_to_f32(wh).astype(np.float64))


def test_decode_gemv_full_size():
    cfg = WL.CONFIGS["decode"]
    _say("[gemv] decode 4096x4096 d_seq=1 r=16")
    _fwd_bwd_full_check(cfg, check_bwd=True)


# layers of more than 4096 rows take the persistent decode kernel (one workgroup per CU
# walking many 16-row groups); the first 4096 rows of such a layer, quantised as part of
# it, form a layer of exactly 256 groups, which takes the one-group-per-workgroup kernel
# when a row is one segment (d_in <= 4096) and the persistent kernel with one group per
# workgroup when it has several. Both must give the same bits on those rows. Shapes: the one-launch A x form (r <= 16,
# d_in <= 4096), the two-launch form with 1, 2 (the second 64 wide) and 3 segments per
# row, d_in = 64; 260 row groups (4 workgroups take two, the rest one), 272 (16 take two)
# and 516 (4 take three, the rest two).
PERSIST = [
    (4160, 4096, 16, "int8"),
    (4160, 4096, 64, "int8"),
    (4160, 2048, 33, "fp8"),
    (4160, 64, 1, "int8"),
    (4352, 4160, 3, "fp8"),
    (4160, 11008, 64, "int8"),
    (8256, 8192, 64, "none"),
]


@pytest.mark.parametrize("shape", PERSIST, ids=[f"{s[0]}x{s[1]}_r{s[2]}_{s[3]}" for s in PERSIST])
def test_persistent_decode_equals_per_group_kernel(shape):
    d_out, d_in, r, dq = shape
    _say(f"[gemv persist] {d_out}x{d_in} r={r} dq={dq}")
    cfg = WL.custom("persist", d_out, d_in, 1, r, s=1.5)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w), dq=dq)
    A, B, X = to_gpu_bf16(a), to_gpu_bf16(b), to_gpu_bf16(WL.make_x(cfg))
    y = qn.linear_fwd(q, A, B, cfg.s, X)
    rows = 4096
    nb = rows * d_in // 64
    assert nb % 256 == 0
    sub = qn.NF4Weight(codes=q.codes[:nb * 32], qconst=q.qconst[:nb] if dq != "none" else q.qconst,
                       qscale=q.qscale[:nb // 256] if dq != "none" else q.qscale[:nb], qmean=q.qmean,
                       d_out=rows, d_in=d_in, dq=dq)
    y_sub = qn.linear_fwd(sub, A, B[:rows].contiguous(), cfg.s, X)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :rows].contiguous().view(torch.int16), y_sub.view(torch.int16))
    if d_in <= 4160:
        ref = O.quantize(w, dq=dq)
        wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], d_out, d_in, dq=dq)
        check_close(bf16_f64(y), O.linear_fwd(wh, a, b, cfg.s, WL.make_x(cfg)), f"decode {d_out}x{d_in}")


# Few tokens on layers of more than 4096 rows take the persistent GEMV too: 2 or 3 with the
# rows of A in the same launch (r <= 16, d_in <= 4096; the first 4096 rows must equal the
# 256-group kernel's bits), 2 after the two-token A x slice kernel (r > 16 or d_in > 4096,
# d_in <= 8192). Every output is also checked against float64, one case on row windows of
# wider X and Y buffers.
PERSIST_TOKENS = [
    (4160, 4096, 16, 2, "int8"),
    (4160, 64, 1, 3, "int8"),
    (4160, 8192, 64, 2, "int8"),
    (4352, 4160, 3, 2, "fp8"),
    (4352, 1024, 33, 2, "none"),
]


@pytest.mark.parametrize("shape", PERSIST_TOKENS,
                         ids=[f"{s[0]}x{s[1]}_r{s[2]}_t{s[3]}_{s[4]}" for s in PERSIST_TOKENS])
def test_persistent_gemv_few_tokens(shape):
    d_out, d_in, r, t, dq = shape
    _say(f"[gemv persist tokens] {d_out}x{d_in} r={r} tokens={t} dq={dq}")
    cfg = WL.custom("persist_t", d_out, d_in, t, r, s=0.75)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w), dq=dq)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    x = WL.make_x(cfg)
    if d_in == 1024:
        xw = torch.zeros(t, d_in + 64, dtype=torch.bfloat16, device=dev())
        xw[:, 32:32 + d_in] = to_gpu_bf16(x)
        X = xw[:, 32:32 + d_in]
        yw = torch.full((t, d_out + 128), 3.0, dtype=torch.bfloat16, device=dev())
        qn.linear_fwd(q, A, B, cfg.s, X, out=yw[:, 64:64 + d_out])
        torch.cuda.synchronize()
        assert bool((yw[:, :64] == 3.0).all()) and bool((yw[:, 64 + d_out:] == 3.0).all()), "wrote outside Y"
        y = yw[:, 64:64 + d_out].contiguous()
    else:
        X = to_gpu_bf16(x)
        y = qn.linear_fwd(q, A, B, cfg.s, X)
    if r <= 16 and d_in <= 4096:
        rows = 4096
        nb = rows * d_in // 64
        sub = qn.NF4Weight(codes=q.codes[:nb * 32], qconst=q.qconst[:nb], qscale=q.qscale[:nb // 256],
                           qmean=q.qmean, d_out=rows, d_in=d_in, dq=dq)
        y_sub = qn.linear_fwd(sub, A, B[:rows].contiguous(), cfg.s, X.contiguous())
        torch.cuda.synchronize()
        assert torch.equal(y[:, :rows].contiguous().view(torch.int16), y_sub.view(torch.int16))
    torch.cuda.synchronize()
    ref = O.quantize(w, dq=dq)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], d_out, d_in, dq=dq)
    check_close(bf16_f64(y), O.linear_fwd(wh, a, b, cfg.s, x), f"gemv {t} tokens {d_out}x{d_in}")


def test_decode_result_does_not_depend_on_workspace_contents():
    """The decode GEMV keeps nothing from call to call in its workspace: whatever the
    workspace held before (zeros, all ones, random bytes, the previous call's partials),
    the result is the same bits."""
    cfg = WL.CONFIGS["decode"]
    w, a, b = _layer(cfg)
    q = _gpu_quantize(w)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = to_gpu_bf16(WL.make_x(cfg))
    need = qn.linear_fwd_workspace_bytes(cfg.d_out, cfg.d_in, 1, cfg.r)
    want = qn.linear_fwd(q, A, B, cfg.s, X)
    torch.cuda.synchronize()
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    gen = torch.Generator(device="cpu").manual_seed(3)
    fills = [lambda t: t.zero_(), lambda t: t.fill_(0xFF),
             lambda t: t.copy_(torch.randint(0, 256, (need,), generator=gen, dtype=torch.uint8))]
    for fill in fills:
        fill(ws)
        for _ in range(3):
            got = qn.linear_fwd(q, A, B, cfg.s, X, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_decode_under_graph_replay_with_new_inputs():
    """Replays of a captured decode call with new x and new A in place must each equal
    the eager call on the same inputs."""
    cfg = WL.CONFIGS["decode"]
    w, a, b = _layer(cfg)
    q = _gpu_quantize(w)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = torch.empty(1, cfg.d_in, dtype=torch.bfloat16, device=dev())
    Y = torch.empty(1, cfg.d_out, dtype=torch.bfloat16, device=dev())
    ws = torch.empty(qn.linear_fwd_workspace_bytes(cfg.d_out, cfg.d_in, 1, cfg.r), dtype=torch.uint8, device=dev())
    X.copy_(torch.randn(1, cfg.d_in, device=dev()).to(torch.bfloat16))
    qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=ws)      # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=ws)
    for i in range(4):
        X.copy_(torch.randn(1, cfg.d_in, device=dev()).to(torch.bfloat16))
        A.copy_((torch.randn(cfg.r, cfg.d_in, device=dev()) * 0.01).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = Y.clone()
        ref = qn.linear_fwd(q, A, B, cfg.s, X)                    # eager, its own workspace
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"


def test_kernel_timing_records_each_launch_and_changes_no_result():
    """qn_profile_enable / qn_profile_read / qn_profile_durations: one duration per launch,
    in launch order, summing to the aggregate; outputs are the same bits with timing on."""
    cfg = WL.custom("timed", 512, 768, 300, 16, s=2.0)
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    A, B, X = to_gpu_bf16(a), to_gpu_bf16(b), to_gpu_bf16(WL.make_x(cfg))
    y_plain = qn.linear_fwd(q, A, B, cfg.s, X).clone()
    qn.profile_enable(True)
    try:
        ys = [qn.linear_fwd(q, A, B, cfg.s, X).clone() for _ in range(3)]
        torch.cuda.synchronize()
        agg = qn.profile_read()
        gemm = [k for k in agg if k.startswith("gemm_")]
        assert gemm, f"no GEMM launch recorded: {sorted(agg)}"
        for k, (n, total_ms) in agg.items():
            each = qn.profile_durations(k)
            assert len(each) == n, k
            assert all(t > 0.0 for t in each), k
            assert abs(sum(each) - total_ms) <= 1e-6 * n + 1e-6 * total_ms, k
        assert agg[gemm[0]][0] % 3 == 0
    finally:
        qn.profile_enable(False)
    assert qn.profile_durations(gemm[0]) == []
    for y in ys:
        assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))


# One token on the persistent GEMV with the A x slices formed in the same launch (r > 16
# or d_in > 4096): the first workgroups publish each slice as (value, tag) words that the
# others wait for. Shapes: 512 x 8192 (32 row groups, 16 slices), 64 x 8192 (4 row groups:
# 12 workgroups only form a slice), 4352 x 4160 at r = 200 (5 slices of 200 ranks), and the
# MLP down-projection shape. For each: any prior workspace content, HIP graph replays with
# new x and A in place, and the fallback where every workgroup forms the slices itself (no
# polling) must give the eager call's bits; the output is checked against float64.
PUBLISHED_AX = [(512, 8192, 64, "int8"), (64, 8192, 64, "int8"), (4352, 4160, 200, "none"), (4096, 11008, 64, "int8")]


@pytest.mark.parametrize("shape", PUBLISHED_AX, ids=[f"{s[0]}x{s[1]}_r{s[2]}_{s[3]}" for s in PUBLISHED_AX])
def test_decode_with_published_ax_slices(shape):
    d_out, d_in, r, dq = shape
    _say(f"[gemv published A x] {d_out}x{d_in} r={r} dq={dq}")
    cfg = WL.custom("pub_ax", d_out, d_in, 1, r, s=1.25)
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    q = qn.quantize(to_gpu_f32(w), dq=dq)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    X = torch.empty(1, d_in, dtype=torch.bfloat16, device=dev())
    X.copy_(to_gpu_bf16(WL.make_x(cfg)))
    want = qn.linear_fwd(q, A, B, cfg.s, X).clone()
    torch.cuda.synchronize()
    ref = O.quantize(w, dq=dq)
    wh = O.double_dequant(ref["codes"], ref["qconst"], ref["qscale"], ref["qmean"], d_out, d_in, dq=dq)
    check_close(bf16_f64(want), O.linear_fwd(wh, a, b, cfg.s, WL.make_x(cfg)), f"decode {d_out}x{d_in} r={r}")

    need = qn.linear_fwd_workspace_bytes(d_out, d_in, 1, r)
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    gen = torch.Generator(device="cpu").manual_seed(5)
    fills = [lambda t: t.zero_(), lambda t: t.fill_(0xFF),
             lambda t: t.copy_(torch.randint(0, 256, (need,), generator=gen, dtype=torch.uint8))]
    for k, fill in enumerate(fills):
        fill(ws)
        for i in range(3):
            got = qn.linear_fwd(q, A, B, cfg.s, X, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"fill {k} call {i}"

    prev = qn.set_ax_wait(0)
    try:
        for i in range(2):
            got = qn.linear_fwd(q, A, B, cfg.s, X, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"no polling, call {i}"
    finally:
        qn.set_ax_wait(prev)

    Y = torch.empty(1, d_out, dtype=torch.bfloat16, device=dev())
    qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=ws)      # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=ws)
    tg = torch.Generator(device="cpu").manual_seed(11)
    for i in range(4):
        X.copy_(torch.randn(1, d_in, generator=tg).to(torch.bfloat16))
        A.copy_((torch.randn(r, d_in, generator=tg) * 0.01).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = Y.clone()
        eager = qn.linear_fwd(q, A, B, cfg.s, X)                  # eager, its own workspace
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
    del g
