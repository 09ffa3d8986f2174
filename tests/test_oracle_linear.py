"""Pins of the oracle's dequantiser and linear layer.

- bf16 rounding against torch's own conversion (a different implementation).
- y = W0 x + s B(A x) and its input gradient against pure-Python loops on tiny
  shapes (whoami-wesleyyou.top "LoRA").
- rank(s B A) <= r, counted by the singular-value gap (same page, "rank 的证明").
- B = 0 / s = 0 reduce to W_hat X; X = I returns W_hat exactly.
- Adjoint identity <dY, fwd(X)> = <bwd_x(dY), X>: dX is the transpose of the
  forward through the same dequantised weights (learn.ifs.name card 1).
"""
import numpy as np
import torch

import workloads as WL
from oracle import nf4_oracle as O


def _rand_bits(rng, shape, scale=1.0):
    return WL.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    base = rng.integers(0, 2 ** 16, 4000, dtype=np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)                 # exact halfway cases
    near = (base | 0x7FFF).view(np.float32)
    allx = np.concatenate([x, ties, near, np.array([0.0, -0.0, 1.0, -1.0], np.float32)])
    allx = allx[np.isfinite(allx)]
    want = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(allx), want)


def test_double_dequant_hand_block():
    # block of 64 codes 0..15 repeated, one constant a_hat = mu exactly (b = 0)
    codes = O.pack_codes(np.tile(np.arange(16, dtype=np.uint8), 4))
    qconst = np.zeros(1, np.int8)
    qscale = np.zeros(1, np.float32)
    mu = np.float32(0.5)
    w = O.double_dequant(codes, qconst, qscale, np.array([mu]), 1, 64)
    vals = O.bf16_bits_to_f32(w).reshape(-1)
    cb = O.codebook()
    # c * 0.5 is exact in float32; then bf16 rounding of those values
    want = torch.from_numpy(np.tile(cb * np.float32(0.5), 4)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(vals, want)
    assert vals[7] == 0 and vals[0] == -0.5 and vals[15] == 0.5


def _loops_fwd(W, A, B, s, X):
    d_seq, d_in = X.shape
    d_out, r = B.shape
    Y = np.zeros((d_seq, d_out))
    for t in range(d_seq):
        ax = [sum(A[k, i] * X[t, i] for i in range(d_in)) for k in range(r)]
        for o in range(d_out):
            Y[t, o] = sum(W[o, i] * X[t, i] for i in range(d_in)) + s * sum(B[o, k] * ax[k] for k in range(r))
    return Y


def _loops_bwd(W, A, B, s, dY):
    d_seq, d_out = dY.shape
    r, d_in = A.shape
    dX = np.zeros((d_seq, d_in))
    for t in range(d_seq):
        bd = [sum(B[o, k] * dY[t, o] for o in range(d_out)) for k in range(r)]
        for i in range(d_in):
            dX[t, i] = sum(W[o, i] * dY[t, o] for o in range(d_out)) + s * sum(A[k, i] * bd[k] for k in range(r))
    return dX


def test_linear_against_python_loops():
    rng = np.random.default_rng(1)
    d_out, d_in, d_seq, r, s = 5, 7, 3, 2, 1.5
    W = _rand_bits(rng, (d_out, d_in), 0.02)
    A = _rand_bits(rng, (r, d_in), 0.1)
    B = _rand_bits(rng, (d_out, r), 0.1)
    X = _rand_bits(rng, (d_seq, d_in))
    dY = _rand_bits(rng, (d_seq, d_out))
    f = lambda b: O.bf16_bits_to_f32(b).astype(np.float64)
    y = O.linear_fwd(W, A, B, s, X)
    assert np.allclose(y, _loops_fwd(f(W), f(A), f(B), s, f(X)), rtol=1e-13, atol=1e-15)
    dx = O.linear_bwd_x(W, A, B, s, dY)
    assert np.allclose(dx, _loops_bwd(f(W), f(A), f(B), s, f(dY)), rtol=1e-13, atol=1e-15)


def test_lora_update_rank_is_r():
    rng = np.random.default_rng(2)
    d_out, d_in, r, s = 96, 80, 8, 2.0
    A = O.bf16_bits_to_f32(_rand_bits(rng, (r, d_in), 0.01)).astype(np.float64)
    B = O.bf16_bits_to_f32(_rand_bits(rng, (d_out, r), 0.01)).astype(np.float64)
    sv = np.linalg.svd(s * B @ A, compute_uv=False)
    # count singular values before the largest log-gap (P4's counting method)
    gaps = np.diff(np.log(np.maximum(sv, 1e-300)))
    rank = int(np.argmin(gaps)) + 1
    assert rank == r


def test_zero_adapter_and_identity_input():
    rng = np.random.default_rng(3)
    cfg = WL.custom("t", 48, 64, 64, 4)
    q = O.quantize(WL.make_weight(cfg))
    wh = O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"], 48, 64)
    A, B = WL.make_lora(cfg)
    X = WL.make_x(cfg)
    zeroB = np.zeros_like(B)
    plain = O.bf16_bits_to_f32(X).astype(np.float64) @ O.bf16_bits_to_f32(wh).astype(np.float64).T
    assert np.array_equal(O.linear_fwd(wh, A, zeroB, 2.0, X), plain)
    assert np.array_equal(O.linear_fwd(wh, A, B, 0.0, X), plain)
    eye = WL.to_bf16_bits(np.eye(64, dtype=np.float32))
    y = O.linear_fwd(wh, A, zeroB, 2.0, eye)           # X = I (64 tokens = d_in)
    assert np.array_equal(y, O.bf16_bits_to_f32(wh).astype(np.float64).T)
    eye_o = WL.to_bf16_bits(np.eye(48, dtype=np.float32))
    dx = O.linear_bwd_x(wh, A, zeroB, 2.0, eye_o)      # dY = I returns W_hat
    assert np.array_equal(dx, O.bf16_bits_to_f32(wh).astype(np.float64))
    del rng


def test_adjoint_identity():
    cfg = WL.custom("t", 72, 128, 9, 8, s=1.75)
    q = O.quantize(WL.make_weight(cfg))
    wh = O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"], cfg.d_out, cfg.d_in)
    A, B = WL.make_lora(cfg)
    X, dY = WL.make_x(cfg), WL.make_dy(cfg)
    y = O.linear_fwd(wh, A, B, cfg.s, X)
    dx = O.linear_bwd_x(wh, A, B, cfg.s, dY)
    lhs = float(np.sum(O.bf16_bits_to_f32(dY).astype(np.float64) * y))
    rhs = float(np.sum(dx * O.bf16_bits_to_f32(X).astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_dequant_rows_matches_full_dequant():
    cfg = WL.custom("t", 40, 192, 1, 4)
    q = O.quantize(WL.make_weight(cfg))
    full = O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"], 40, 192)
    rows = np.array([0, 7, 39])
    assert np.array_equal(O.dequant_rows(q, 192, rows), full[rows])
