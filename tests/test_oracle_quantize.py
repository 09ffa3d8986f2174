"""Pins of the oracle's quantiser: nearest code, blocks, Double Quantisation.

Independent checks: exact rational nearest-code search (Fractions), values at
the printed code points, hand-worked DQ examples, exact-mean tie cases, and
the pages' storage figures (4.127 / 4.5 / 0.127 / 0.373 bit, ~3 GB at 65B).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4_oracle as O


def _f32(v):
    return np.float32(v)


def _exact_nearest(x, book):
    """Nearest index by exact rational distance, lower index on ties."""
    fx = Fraction(float(x))
    best, bi = None, None
    for i, c in enumerate(book):
        dist = abs(fx - Fraction(float(c)))
        if best is None or dist < best:
            best, bi = dist, i
    return bi


def _probe_points():
    c = O.codebook()
    pts = []
    for k in range(15):
        lo, hi = float(c[k]), float(c[k + 1])
        m = np.float32((lo + hi) / 2)
        for step in range(-40, 41):
            pts.append(np.nextafter(m, np.float32(np.inf if step > 0 else -np.inf), dtype=np.float32)
                       if step else m)
            v = m
            for _ in range(abs(step)):
                v = np.nextafter(v, np.float32(np.inf if step > 0 else -np.inf), dtype=np.float32)
            pts.append(v)
    rng = np.random.default_rng(123)
    pts += list(rng.uniform(-1, 1, 3000).astype(np.float32))
    pts += [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0),
            np.float32(1e-45), np.float32(-1e-45), np.float32(1.1754944e-38), np.float32(-3e-39)]
    pts += list(c)
    return np.array(pts, dtype=np.float32)


def test_nearest_code_equals_exact_rational_search():
    book = O.codebook()
    x = _probe_points()
    got = O.nearest_code(x)
    want = np.array([_exact_nearest(v, book) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_exact_ties_take_the_lower_index():
    book = O.codebook().astype(np.float64)
    ties = 0
    for k in range(15):
        m = (book[k] + book[k + 1]) / 2          # exact in float64
        if float(np.float32(m)) == m:            # midpoint representable in float32
            ties += 1
            assert O.nearest_code(np.array([m], np.float32))[0] == k
            up = np.nextafter(np.float32(m), np.float32(2))
            assert O.nearest_code(np.array([up], np.float32))[0] == k + 1
    assert ties >= 1


def test_printed_code_points_map_to_their_index(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        printed = np.array(json.load(f)["nf4_quant_book_4dp"]["value"], dtype=np.float32)
    assert np.array_equal(O.nearest_code(printed), np.arange(16))
    mids = (printed[:-1] + printed[1:]) / 2
    assert np.array_equal(O.nearest_code((mids - 1e-3).astype(np.float32)), np.arange(15))
    assert np.array_equal(O.nearest_code((mids + 1e-3).astype(np.float32)), np.arange(1, 16))


def test_block_scaled_by_absmax_hand_case(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        printed = np.array(json.load(f)["nf4_quant_book_4dp"]["value"], dtype=np.float32)
    # one block: the 16 printed points scaled by 0.5, four times -> absmax 0.5
    w = np.tile(printed * np.float32(0.5), 4).astype(np.float32).reshape(1, 64)
    q = O.quantize(w)
    assert q["absmax"][0] == np.float32(0.5)
    codes = O.unpack_codes(q["codes"])
    assert np.array_equal(codes, np.tile(np.arange(16), 4))


def test_zero_block_and_ragged_tail_use_exact_zero_code():
    w = np.zeros((3, 50), np.float32)   # n = 150: 2 full blocks + a 22-element tail
    w[2, 49] = 0.25
    q = O.quantize(w)
    a = q["absmax"]
    assert a.shape == (3,) and a[0] == 0 and a[1] == 0 and a[2] == np.float32(0.25)
    codes = O.unpack_codes(q["codes"])
    assert codes.size == 3 * 64
    nz = np.nonzero(codes != 7)[0]
    assert nz.tolist() == [149]       # flat index of w[2, 49]
    assert codes[149] == 15


def test_pack_unpack_round_trip_and_nibble_order():
    c = np.arange(64, dtype=np.uint8) % 16
    p = O.pack_codes(c)
    assert p.size == 32 and p[0] == (0 | (1 << 4))
    assert np.array_equal(O.unpack_codes(p), c)


def test_dq_hand_worked_group():
    # a = [1, 2, 3, 4]: mean 2.5; centred [-1.5, -0.5, 0.5, 1.5]; b = 1.5;
    # r = [-1, -1/3, 1/3, 1] (1/3 rounded to float32); r*127 = [-127, -42.33.., 42.33.., 127]
    a = np.array([1, 2, 3, 4], np.float32)
    mu = O.exact_mean_f32(a)
    assert mu == np.float32(2.5)
    q, b = O.dq_encode(a, mu)
    assert b.tolist() == [1.5]
    assert q.tolist() == [-127, -42, 42, 127]
    ahat = O.dq_decode(q, b, mu)
    assert ahat[0] == np.float32(1.0) and ahat[3] == np.float32(4.0)
    # a_hat_1 = 2.5 + 1.5 * fl32(-42/127)
    assert ahat[1] == np.float32(np.float32(2.5) + np.float32(np.float32(1.5) * np.float32(np.float32(-42) / np.float32(127))))
    assert abs(float(ahat[1]) - (2.5 - 1.5 * 42 / 127)) < 1e-6


def test_dq_constant_group_is_exact():
    a = np.full(300, 0.0625, np.float32)      # two groups (256 + 44), all equal
    mu = O.exact_mean_f32(a)
    q, b = O.dq_encode(a, mu)
    assert mu == np.float32(0.0625) and np.all(b == 0) and np.all(q == 0)
    assert np.all(O.dq_decode(q, b, mu) == np.float32(0.0625))


def test_dq_reconstruction_error_bound():
    rng = np.random.default_rng(5)
    a = np.abs(rng.standard_normal(4096 * 3 + 17).astype(np.float32)) * np.float32(0.05)
    mu = O.exact_mean_f32(a)
    q, b = O.dq_encode(a, mu)
    assert q.dtype == np.int8 and int(np.max(np.abs(q.astype(int)))) == 127
    ahat = O.dq_decode(q, b, mu)
    bj = np.repeat(b, 256)[: a.size].astype(np.float64)
    err = np.abs(ahat.astype(np.float64) - a.astype(np.float64))
    assert np.all(err <= bj / 254 + 4 * np.spacing(np.float32(1.0)) * (np.abs(a) + bj + abs(float(mu))))


def test_exact_mean_ties_and_subnormals():
    one = np.float32(1.0)
    u = np.float32(2.0 ** -23)
    # mean 1 + 2^-24: halfway between 1 and 1+2^-23 -> even -> 1
    assert O.exact_mean_f32(np.array([one, one + u], np.float32)) == one
    # mean 1 + 1.5*2^-23: halfway between 1+2^-23 (odd) and 1+2^-22 (even)
    m = O.exact_mean_f32(np.array([one + u, one + 2 * u], np.float32))
    assert m == np.float32(1.0 + 2.0 ** -22)
    tiny = np.float32(2.0 ** -149)
    assert O.exact_mean_f32(np.array([tiny, 0], np.float32)) == 0           # tie -> even (0)
    assert O.exact_mean_f32(np.array([tiny, tiny, tiny, 0], np.float32)) == tiny
    assert O.exact_mean_f32(np.array([0.0, 0.0], np.float32)) == 0
    assert O.exact_mean_f32(np.array([3.0, 0.0, 0.0], np.float32)) == 1
    big = np.float32(3.0e38)
    assert O.exact_mean_f32(np.array([big, big], np.float32)) == big


def test_exact_mean_matches_float64_mean_within_half_ulp():
    rng = np.random.default_rng(7)
    for n in (1, 5, 256, 10007):
        a = (np.abs(rng.standard_normal(n)) * rng.choice([1e-3, 1.0, 1e3], n)).astype(np.float32)
        m = O.exact_mean_f32(a)
        ref = np.mean(a.astype(np.float64))      # float64 error << float32 half ulp
        assert abs(float(m) - ref) <= 0.5 * float(np.spacing(np.float32(ref))) * (1 + 1e-6)


def test_f32_from_rational_against_float_conversion():
    rng = np.random.default_rng(11)
    for _ in range(2000):
        num = int(rng.integers(1, 2 ** 62)) * int(rng.integers(1, 2 ** 20))
        den = int(rng.integers(1, 2 ** 40))
        got = O.f32_from_rational(num, den)
        d = float(Fraction(num, den))             # correctly rounded to float64
        want = np.float32(d)
        # float64 -> float32 double rounding can only err when d is (nearly) a tie
        if got != want:
            lo, hi = sorted([float(got), float(want)])
            assert hi == float(np.nextafter(np.float32(lo), np.float32(np.inf)))
            assert abs(d - (lo + hi) / 2) <= abs(d) * 2 ** -52


def test_storage_bits_match_the_pages(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        g = {k: v["value"] for k, v in json.load(f).items()}
    for n in (4096 * 4096, 11008 * 4096, 28672 * 8192):
        assert abs(O.storage_bits_per_param(n) - g["bits_per_param_with_dq"]) < 5e-4
        assert O.storage_bits_per_param(n, double_quant=False) == g["bits_per_param_without_dq"]
        const_bits = O.storage_bits_per_param(n) - 4
        assert abs(const_bits - g["dq_constant_bits"]) < 5e-4
        saving = O.storage_bits_per_param(n, False) - O.storage_bits_per_param(n)
        assert abs(saving - g["dq_saving_bits"]) < 5e-4
    saving_65b = (O.storage_bits_per_param(65 * 2 ** 30 // 64 * 64, False)
                  - O.storage_bits_per_param(65 * 2 ** 30 // 64 * 64)) * 65e9 / 8 / 1e9
    assert abs(saving_65b - g["dq_saving_65b_gigabytes"]) < 0.1


def test_quantize_buffer_sizes():
    w = np.ones((256, 256), np.float32)
    q = O.quantize(w)
    assert q["codes"].size == 65536 // 2 and q["qconst"].size == 1024
    assert q["qscale"].size == 4 and q["qmean"].size == 1


def test_round_trip_error_is_plausible_for_gaussian_weights():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((128, 512)) * 0.02).astype(np.float32)
    q = O.quantize(w)
    wh = O.bf16_bits_to_f32(O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"], 128, 512))
    rel = np.linalg.norm(wh - w) / np.linalg.norm(w)
    assert 0.05 < rel < 0.12
