"""Pins of the oracle's second-level formats other than INT8: FP8 E4M3 codes of the
centred block constants ("8-bit floats", learn.ifs.name deck card 4) and no second
level at all (the float32 a_j per block of 64, 4.5 bit/param: whoami-wesleyyou.top
"2. Double Quantization (DQ)").

The E4M3 table and encoder are pinned to the OCP FP8 definition's fixed points and
to torch's own float8_e4m3fn conversion (an independent implementation); the DQ
steps to a hand-worked group, an error bound and the degenerate cases."""
import math

import numpy as np
import pytest
import torch

import oracle.nf4_oracle as O
import workloads as WL


def test_e4m3_table_fixed_points():
    v = O.e4m3_values()
    assert v[0x7E] == 448.0                  # largest finite magnitude, 1.75 * 2^8
    assert v[0x08] == 2.0 ** -6              # smallest normal
    assert v[0x01] == 2.0 ** -9              # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9          # largest subnormal
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0xB8] == -1.0
    assert v[0x00] == 0.0 and not np.signbit(v[0x00]) and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)          # codes 0x00..0x7E ascend with the value
    assert np.array_equal(v[0x80:0xFF], -pos)


def test_e4m3_table_matches_torch():
    ours = O.e4m3_values()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], theirs[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(theirs[fin]))


def _probe_values():
    v = O.e4m3_values()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2                       # exact ties (all representable in float32)
    rng = np.random.default_rng(7)
    parts = [v, -v, mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
             np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
             rng.uniform(-448, 448, 50000),
             rng.uniform(-1, 1, 50000) * 2.0 ** rng.integers(-24, 0, 50000),
             [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -149, 3 * 2.0 ** -11]]
    return np.concatenate([np.asarray(p, np.float64) for p in parts]).astype(np.float32)


def test_e4m3_encode_matches_torch():
    x = _probe_values()
    ours = O.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_encode_ties_go_to_even_code():
    v = O.e4m3_values()[:0x7F]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    code = O.e4m3_encode(mids)
    assert np.all(code % 2 == 0)
    assert np.all((code == np.arange(0x7E)) | (code == np.arange(1, 0x7F)))


def test_e4m3_encode_roundtrip_and_nearest():
    v = O.e4m3_values()
    fin = np.array([u for u in range(256) if not np.isnan(v[u])])
    assert np.array_equal(O.e4m3_encode(v[fin].astype(np.float32)), fin.astype(np.uint8))
    # brute force: no finite code is strictly nearer than the chosen one
    x = _probe_values()[::37]
    got = v[O.e4m3_encode(x)]
    dist = np.abs(x.astype(np.float64)[:, None] - v[None, fin])
    assert np.all(np.abs(x.astype(np.float64) - got) <= dist.min(axis=1))
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([449.0], np.float32))


def test_fp8_dq_hand_worked_group():
    # a = [1, 2, 3, 4]: mu = 2.5, d = [-1.5, -0.5, 0.5, 1.5], b = 1.5, r = [-1, -1/3, 1/3, 1];
    # r * 448 = [-448, -149.33, 149.33, 448]; in [128, 256) E4M3 steps by 16, so 149.33
    # goes to 144 = 1.125 * 2^7: exponent field 14, mantissa 1 -> 0x71 (0xF1 negative).
    a = np.array([1, 2, 3, 4], np.float32)
    mu = O.exact_mean_f32(a)
    assert mu == np.float32(2.5)
    q, b = O.dq_encode(a, mu, group=4, fmt="fp8")
    assert b.tolist() == [1.5]
    assert q.view(np.uint8).tolist() == [0xFE, 0xF1, 0x71, 0x7E]
    ahat = O.dq_decode(q, b, mu, group=4, fmt="fp8")
    assert ahat[0] == np.float32(1.0) and ahat[3] == np.float32(4.0)
    assert abs(float(ahat[1]) - (2.5 - 1.5 * 144 / 448)) < 1e-6
    assert abs(float(ahat[2]) - (2.5 + 1.5 * 144 / 448)) < 1e-6


def test_fp8_dq_zero_group_and_full_range():
    a = np.full(256, 0.125, np.float32)              # one constant group: b = 0
    q, b = O.dq_encode(a, O.exact_mean_f32(a), fmt="fp8")
    assert b[0] == 0 and np.all(q == 0)
    assert np.all(O.dq_decode(q, b, np.float32(0.125), fmt="fp8") == np.float32(0.125))
    rng = np.random.default_rng(3)
    a = np.abs(rng.normal(0, 0.02, 4096)).astype(np.float32)
    q, b = O.dq_encode(a, O.exact_mean_f32(a), fmt="fp8")
    u = q.view(np.uint8).reshape(-1, 256)
    assert np.all(np.any((u == 0x7E) | (u == 0xFE), axis=1))   # each group's extreme maps to +-448


def test_fp8_dq_error_bound():
    # |a_hat - a| <= b * (half an E4M3 step at |r| * 448) / 448 plus float32 rounding
    cfg = WL.CONFIGS["tiny"]
    a = O.block_absmax(O.to_blocks(WL.make_weight(cfg)))
    mu = O.exact_mean_f32(a)
    q, b = O.dq_encode(a, mu, fmt="fp8")
    ahat = O.dq_decode(q, b, mu, fmt="fp8").astype(np.float64)
    bj = np.repeat(b, O.DQ_GROUP)[: a.size].astype(np.float64)
    m = np.abs((a.astype(np.float64) - float(mu)) / np.where(bj > 0, bj, 1.0)) * 448.0
    step = np.where(m >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(m, 2.0 ** -6))) - 3), 2.0 ** -9)
    bound = bj * step / 2 / 448.0 + 4 * np.finfo(np.float32).eps * (abs(float(mu)) + bj)
    assert np.all(np.abs(ahat - a) <= bound)
    # finer than INT8 near the mean, coarser at the group's extremes: both cases occur
    qi, bi = O.dq_encode(a, mu)
    ei = np.abs(O.dq_decode(qi, bi, mu).astype(np.float64) - a)
    ef = np.abs(ahat - a)
    assert np.any(ef < ei) and np.any(ef > ei)


def test_no_second_level_keeps_absmax():
    cfg = WL.CONFIGS["tiny"]
    w = WL.make_weight(cfg)
    qn = O.quantize(w, dq="none")
    qi = O.quantize(w)
    assert np.array_equal(qn["codes"], qi["codes"])             # first level unchanged
    assert np.array_equal(qn["qscale"].view(np.uint32), qi["absmax"].view(np.uint32))
    assert np.array_equal(O.block_constants(qn), qi["absmax"])
    wh = O.double_dequant(qn["codes"], qn["qconst"], qn["qscale"], qn["qmean"], cfg.d_out, cfg.d_in, dq="none")
    # element check: bf16(c[code] * a_j) for a few entries, written out directly
    cb = O.codebook()
    codes = O.unpack_codes(qn["codes"])
    for k in (0, 1, 63, 64, 4095, cfg.d_out * cfg.d_in - 1):
        prod = np.float32(cb[codes[k]] * qi["absmax"][k // 64])
        u = int(np.array([prod], np.float32).view(np.uint32)[0])
        assert int(wh.reshape(-1)[k]) == (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    assert O.storage_bits_per_param(cfg.d_out * cfg.d_in, double_quant=False) == 4.5


def test_fp8_quantize_round_trip_error():
    # the weight error of NF4 + FP8 DQ stays at the NF4 level (the constants are a
    # small part of it): within 2 % of the INT8 layout's error on the same weight
    cfg = WL.CONFIGS["tiny"]
    w = WL.make_weight(cfg)
    errs = {}
    for fmt in ("int8", "fp8", "none"):
        q = O.quantize(w, dq=fmt)
        wh = O.bf16_bits_to_f32(O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"],
                                                cfg.d_out, cfg.d_in, dq=fmt))
        errs[fmt] = math.sqrt(float(np.sum((wh.astype(np.float64) - w) ** 2) / np.sum(w.astype(np.float64) ** 2)))
    assert abs(errs["fp8"] - errs["none"]) < 0.02 * errs["none"]
    assert abs(errs["int8"] - errs["none"]) < 0.02 * errs["none"]
