"""Pins of the oracle's NF4 code book against what the pages fix.

- The printed 16-value quant book (jjjymmm.cn 2024/03, "4-bit NormalFloat(NF4)").
- Exact zero, ends at -1/+1, 7 negative + zero + 8 positive values
  (learn.ifs.name QLoRA deck, card 3; whoami-wesleyyou.top "归一化与匹配").
- Equal probability mass per bin on each half (deck card 2), checked with the
  forward CDF, a different routine from the inverse used to build the book.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import ndtr, ndtri

from oracle import nf4_oracle as O


@pytest.fixture(scope="module")
def printed(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        return np.array(json.load(f)["nf4_quant_book_4dp"]["value"], dtype=np.float64)


def test_matches_printed_table_to_4dp(printed):
    c = O.codebook_f64()
    # A 4-decimal print is within half a unit of the 4th place of the true value.
    # Entry 6 (-0.091049976) sits 2.4e-8 past that half unit from the printed
    # -0.0911, hence the 3e-8 slack.
    assert np.all(np.abs(c - printed) <= 5e-5 + 3e-8), np.abs(c - printed)
    # all but that one entry round to exactly the printed digits
    rounded = np.round(c, 4)
    mism = np.nonzero(rounded != printed)[0]
    assert set(mism.tolist()) <= {6}


def test_structure_exact_zero_and_ends():
    c = O.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[7] == 0.0 and not np.signbit(c[7])
    assert c[0] == -1.0 and c[15] == 1.0
    assert np.all(np.diff(c) > 0)
    assert int(np.sum(c < 0)) == 7 and int(np.sum(c > 0)) == 8


def test_independent_inverse_cdf_gives_same_float32_bits():
    a = O.codebook_f64()
    b = O.codebook_f64(inv_cdf=lambda p: float(ndtri(p)))
    assert np.max(np.abs(a - b)) < 1e-14
    assert np.array_equal(a.astype(np.float32).view(np.uint32), b.astype(np.float32).view(np.uint32))


def test_equal_probability_steps_on_each_half():
    c = O.codebook_f64()
    d = O.nf4_offset()
    scale = ndtri(d)
    p = ndtr(c * scale)              # probabilities of the un-normalised quantiles
    pos = p[7:]                      # 0.5 then 8 increasing values up to d
    neg = p[:8]                      # 1-d ... 0.5
    assert abs(pos[0] - 0.5) < 1e-15 and abs(pos[-1] - d) < 1e-12
    assert np.allclose(np.diff(pos), (d - 0.5) / 8, atol=1e-12, rtol=0)
    assert abs(neg[0] - (1 - d)) < 1e-12
    assert np.allclose(np.diff(neg), (d - 0.5) / 7, atol=1e-12, rtol=0)


def test_outer_offset_is_between_the_15_and_16_level_half_bins():
    d = O.nf4_offset()
    assert 1 - 1 / 30 < d < 1 - 1 / 32
    # the interval of offsets whose book rounds to the printed digits
    # (except the borderline entry 6) contains this value
    assert abs(d - 0.96770833) < 1e-8


def test_page1_literal_sample_formula_is_not_the_printed_book(printed):
    # whoami-wesleyyou.top "分位数采样与端点问题" quotes q_i = (Q(i/17) + Q((i+1)/17))/2.
    # Taken literally (i = 1..15, normalised) it is symmetric with 15 values and
    # misses the printed book by ~0.07; the asymmetric construction is used instead.
    q = [0.5 * (ndtri(i / 17) + ndtri((i + 1) / 17)) for i in range(1, 16)]
    q = np.array(q) / np.max(np.abs(q))
    assert q.size == 15 and abs(q[1] - printed[1]) > 0.05
