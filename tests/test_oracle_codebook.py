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
    # a 4-decimal print is within half a unit of the 4th place of the true value,
    # on every one of the 16 entries
    assert np.all(np.abs(c - printed) <= 5e-5), np.abs(c - printed)
    assert np.array_equal(np.round(c, 4), printed)
    # the float32 book the layer uses rounds to the same digits
    assert np.array_equal(np.round(O.codebook().astype(np.float64), 4), printed)


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


def _book_for(d):
    """The asymmetric book for outer probabilities d (scalar or 1-D array), written
    with scipy's ndtri (a different inverse-CDF routine from the oracle's)."""
    d = np.atleast_1d(np.asarray(d, np.float64))[:, None]
    pos = ndtri(d - np.arange(8)[None, :] * (d - 0.5) / 8)
    neg = -ndtri(d - np.arange(7)[None, :] * (d - 0.5) / 7)
    v = np.concatenate([neg, np.zeros((d.shape[0], 1)), pos], axis=1)
    return np.squeeze(np.sort(v, axis=1) / ndtri(d))


def test_offset_lies_inside_the_interval_the_printed_book_allows(printed):
    # Scan the outer probability over (0.55, 1) in steps of 2.2e-7: the offsets whose
    # book rounds to all 16 printed digits form one short interval, and the oracle's
    # offset is inside it with room on both sides.
    grid = np.linspace(0.55, 0.99999, 2_000_001)
    ok = np.nonzero(np.all(np.round(_book_for(grid), 4) == printed[None, :], axis=1))[0]
    assert ok.size > 0, "no offset reproduces the printed book"
    assert ok[-1] - ok[0] + 1 == ok.size, "the matching offsets are not one interval"
    lo, hi = grid[ok[0]], grid[ok[-1]]
    assert hi - lo < 1e-5
    d = O.nf4_offset()
    assert lo < d < hi

    def fits(x):
        return np.array_equal(np.round(_book_for(x), 4), printed)

    # the interval's edges, to 1e-9 by bisection from the scanned points
    def edge(good, bad):
        for _ in range(40):
            mid = 0.5 * (good + bad)
            good, bad = (mid, bad) if fits(mid) else (good, mid)
        return good

    lo_e, hi_e = edge(d, d - 1e-4), edge(d, d + 1e-4)
    assert fits(d) and hi_e - lo_e > 5e-6
    assert lo_e + 1e-6 < d < hi_e - 1e-6
    # every entry at least 2e-6 inside its printed rounding interval
    assert np.min(5e-5 - np.abs(_book_for(d) - printed)) >= 2e-6
    # and between the half-bin offsets of 15 and 16 equal-probability levels
    assert 1 - 1 / 30 < d < 1 - 1 / 32


def test_page1_literal_sample_formula_is_not_the_printed_book(printed):
    # whoami-wesleyyou.top "分位数采样与端点问题" quotes q_i = (Q(i/17) + Q((i+1)/17))/2.
    # Taken literally (i = 1..15, normalised) it is symmetric with 15 values and
    # misses the printed book by ~0.07; the asymmetric construction is used instead.
    q = [0.5 * (ndtri(i / 17) + ndtri((i + 1) / 17)) for i in range(1, 16)]
    q = np.array(q) / np.max(np.abs(q))
    assert q.size == 15 and abs(q[1] - printed[1]) > 0.05
