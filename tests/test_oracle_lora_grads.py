"""Pins of the oracle's adapter gradients (dA, dB) against facts that do not use
its formulas: finite differences of the loss L = <dY, Y> (exact for a function
that is linear in each factor), an Euler identity of the bilinear LoRA term, and
the zero cases. CPU only."""
import numpy as np
import pytest

import workloads as WL
from oracle import nf4_oracle as O


def _bits(x):
    return O.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _case(d_out=24, d_in=40, d_seq=7, r=3, seed=5):
    rng = np.random.default_rng(seed)
    w = _bits(rng.normal(0, 0.05, (d_out, d_in)))
    a = _bits(rng.normal(0, 0.1, (r, d_in)))
    b = _bits(rng.normal(0, 0.1, (d_out, r)))
    x = _bits(rng.normal(0, 1, (d_seq, d_in)))
    dy = _bits(rng.normal(0, 1, (d_seq, d_out)))
    return w, a, b, x, dy


def _loss(w, A, B, s, x, dy):
    """L = <dY, Y> for float64 factors A [r, d_in], B [d_out, r] (not bf16-rounded)."""
    W, X, dY = O._f64(w), O._f64(x), O._f64(dy)
    Y = X @ W.T + s * ((X @ A.T) @ B.T)
    return float(np.sum(dY * Y))


def test_finite_differences_match_both_gradients():
    w, a, b, x, dy = _case()
    s = 1.75
    dA, dB = O.lora_grads(a, b, s, x, dy)
    A, B = O._f64(a), O._f64(b)
    eps = 0.5          # L is linear in A for fixed B (and in B for fixed A): any step is exact
    for (j, i) in [(0, 0), (2, 39), (1, 17)]:
        E = np.zeros_like(A)
        E[j, i] = eps
        fd = (_loss(w, A + E, B, s, x, dy) - _loss(w, A - E, B, s, x, dy)) / (2 * eps)
        assert fd == pytest.approx(dA[j, i], rel=1e-9, abs=1e-9)
    for (o, j) in [(0, 0), (23, 2), (11, 1)]:
        E = np.zeros_like(B)
        E[o, j] = eps
        fd = (_loss(w, A, B + E, s, x, dy) - _loss(w, A, B - E, s, x, dy)) / (2 * eps)
        assert fd == pytest.approx(dB[o, j], rel=1e-9, abs=1e-9)


def test_euler_identity_of_the_bilinear_term():
    # the LoRA part s <dY, X A^T B^T> is linear in A and in B, so
    # <dA, A> = <dB, B> = that part of the loss
    w, a, b, x, dy = _case(seed=9)
    s = 0.5
    dA, dB = O.lora_grads(a, b, s, x, dy)
    A, B = O._f64(a), O._f64(b)
    lora_part = _loss(w, A, B, s, x, dy) - _loss(w, A, np.zeros_like(B), s, x, dy)
    assert np.sum(dA * A) == pytest.approx(lora_part, rel=1e-10)
    assert np.sum(dB * B) == pytest.approx(lora_part, rel=1e-10)


def test_zero_cases():
    w, a, b, x, dy = _case(seed=3)
    zb = np.zeros_like(b)                    # B = 0 (the usual LoRA init): dA = 0, dB generally not
    dA, dB = O.lora_grads(a, zb, 2.0, x, dy)
    assert not np.any(dA)
    assert np.any(dB)
    dA, dB = O.lora_grads(a, b, 0.0, x, dy)  # s = 0 switches the branch off
    assert not np.any(dA) and not np.any(dB)


def test_tiny_config_shapes():
    cfg = WL.CONFIGS["tiny"]
    a, b = WL.make_lora(cfg)
    dA, dB = O.lora_grads(a, b, cfg.s, WL.make_x(cfg), WL.make_dy(cfg))
    assert dA.shape == (cfg.r, cfg.d_in) and dB.shape == (cfg.d_out, cfg.r)
    assert np.all(np.isfinite(dA)) and np.all(np.isfinite(dB))
