"""Pins of the oracle's quantised low-rank factors (W ~ Q + L R with L and R kept at 4
or 8 bits: gist.science "Sintesi Tecnica: GPTQ-intrinsic LoRA", "Risultati Chiave");
the 8-bit factor is absmax INT8 per block of 64 (jjjymmm.cn "量化原理")."""
import numpy as np
import pytest

import oracle.nf4_oracle as O
import workloads as WL


def test_int8_hand_worked_block():
    # [1, 2, 3, 4] / 4 * 127 = [31.75, 63.5, 95.25, 127]: 63.5 is a tie and goes to the even 64
    q, a = O.int8_quantize(np.array([[1, 2, 3, 4]], np.float32))
    assert a.tolist() == [4.0]
    assert q[:4].tolist() == [32, 64, 95, 127]
    assert np.all(q[4:] == 0)                                  # the +0.0 padding of the block
    wh = O.bf16_bits_to_f32(O.int8_dequant(q, a, 1, 4))
    for k, v in zip((32, 64, 95, 127), wh[0]):
        assert abs(v - k * 4 / 127) <= 2 ** -8 * abs(v)        # one bf16 rounding
    assert wh[0, 3] == 4.0


def test_int8_zero_block_and_extremes():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((7, 192)) * 0.01).astype(np.float32)
    w[2, 64:128] = 0.0
    q, a = O.int8_quantize(w)
    qb = q.reshape(-1, 64)
    assert a[2 * 3 + 1] == 0 and np.all(qb[2 * 3 + 1] == 0)
    assert np.all(np.abs(qb) <= 127)
    nz = a > 0
    assert np.all(np.max(np.abs(qb[nz]), axis=1) == 127)      # the block max maps to +-127
    wh = O.bf16_bits_to_f32(O.int8_dequant(q, a, 7, 192))
    assert np.all(wh[2, 64:128] == 0)


def test_int8_error_bound():
    cfg = WL.CONFIGS["tiny"]
    w = WL.make_weight(cfg)
    q, a = O.int8_quantize(w)
    wh = O.bf16_bits_to_f32(O.int8_dequant(q, a, *w.shape)).astype(np.float64)
    aj = np.repeat(a, 64)[: w.size].reshape(w.shape).astype(np.float64)
    bound = aj / 254 * (1 + 1e-6) + np.abs(w) * 2.0 ** -8
    assert np.all(np.abs(wh - w) <= bound)


def test_int8_integer_grid_round_trips():
    # values k in [-127, 127] with block max 127 come back exactly
    rng = np.random.default_rng(1)
    k = rng.integers(-127, 128, (4, 64)).astype(np.float32)
    k[:, 0] = 127
    q, a = O.int8_quantize(k)
    assert np.array_equal(q.reshape(4, 64), k.astype(np.int8))
    assert np.array_equal(O.bf16_bits_to_f32(O.int8_dequant(q, a, 4, 64)), k)


def test_factor_formats():
    cfg = WL.CONFIGS["tiny"]
    a_bits, b_bits = WL.make_lora(cfg)
    A = O.bf16_bits_to_f32(a_bits)                              # [r, d_in]
    B = O.bf16_bits_to_f32(b_bits)                              # [d_out, r]: 64-blocks span 64/r rows
    for bits in (4, 8):
        for M in (A, B):
            codes, sc = O.quantize_factor(M, bits)
            got = O.bf16_bits_to_f32(O.dequant_factor(codes, sc, bits, *M.shape))
            rel = np.linalg.norm(got - M) / np.linalg.norm(M)
            assert rel < (0.12 if bits == 4 else 0.008), (bits, rel)   # step/sqrt(12) of a Gaussian block
    q4 = O.quantize(A, dq="none")
    c4, s4 = O.quantize_factor(A, 4)
    assert np.array_equal(c4, q4["codes"]) and np.array_equal(s4, q4["absmax"])
    with pytest.raises(ValueError):
        O.quantize_factor(A, 3)


def test_quantised_factor_forward_is_close_to_bf16_factors():
    # W ~ Q + L R in the layer's column form: Y = X Q_hat^T + s (X A_hat^T) B_hat^T.
    # With 8-bit factors the change of Y stays below the bf16 output rounding
    # (the factors' error of ~0.4 % hits a term that is a few % of Y).
    cfg = WL.CONFIGS["tiny"]
    w = WL.make_weight(cfg)
    a_bits, b_bits = WL.make_lora(cfg)
    x = WL.make_x(cfg)
    q = O.quantize(w)
    wh = O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"], cfg.d_out, cfg.d_in)
    y_ref = O.linear_fwd(wh, a_bits, b_bits, cfg.s, x)
    rels = {}
    for bits in (4, 8):
        ca, sa = O.quantize_factor(O.bf16_bits_to_f32(a_bits), bits)
        cb, sb = O.quantize_factor(O.bf16_bits_to_f32(b_bits), bits)
        ah = O.dequant_factor(ca, sa, bits, cfg.r, cfg.d_in)
        bh = O.dequant_factor(cb, sb, bits, cfg.d_out, cfg.r)
        y = O.linear_fwd(wh, ah, bh, cfg.s, x)
        rels[bits] = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rels[8] < 2.0 ** -9
    assert rels[4] < 0.02
