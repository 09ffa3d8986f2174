"""Plain, slow CPU oracle for the QLoRA NF4 + Double-Quantisation linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the package's smoke check and the CPU-baseline leg
of the benchmark do. It shares no code, table or constant generator with the
HIP library; the only thing both sides share is the seeded input module.

Every float32 step below is a single numpy ufunc on float32 operands, so each
is one IEEE-754 operation rounded to nearest-even with no fused multiply-add.
Matrix products are float64. Sources (web pages on QLoRA; section names as
they appear on each page):

  [P1] whoami-wesleyyou.top, "LoRA 与 QLoRA": sections "LoRA" (y = W0 x + s B(A x),
       shapes), "rank 的证明", "1. NF4" (4-bit -> dequant -> BF16 -> GEMM,
       "Gaussian 假设与分位数", "分位数采样与端点问题", "归一化与匹配") and
       "2. Double Quantization (DQ)".
  [P2] learn.ifs.name, Dettmers et al. 2023 "3 QLoRA Finetuning" deck, cards 1-4.
  [P4] jjjymmm.cn 2024/03 blog, sections "4-bit NormalFloat(NF4)" (printed quant
       book), "Double Quantization" (blocks of 64, 8-bit constants in blocks of
       256, the 0.127 bit/param count), "QLoRA" (doubleDequant order) and
       "量化原理" (absmax integer quantisation).
  [P5] gist.science, "Sintesi Tecnica: GPTQ-intrinsic LoRA": W ~ Q + L R, and the
       low-rank factors kept at 4 or 8 bits ("Risultati Chiave", "Empirici").

Readings taken where the pages are silent (each is listed with its reason in
the design notes): code-book probability offset, nearest-code tie rule, nibble
order, the mean of the block constants rounded exactly, symmetric INT8 with step
127 for the second level, and the separate multiply-then-add reconstruction.

Second-level formats: "int8" (the default above); "fp8", the "8-bit floats" of
[P2 card 4] taken as OCP FP8 E4M3 codes of r * 448 (448 is the largest finite
E4M3 magnitude, as 127 is for INT8); "none", no second level: the float32 a_j is
stored per block (the 4.5 bit/param layout of [P1 2. DQ]).
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

BLOCK = 64        # weights per first-level block [P1 DQ section; P4 DQ example]
DQ_GROUP = 256    # first-level constants per second-level block [P2 card 4; P4 DQ example]
INT8_STEP = 127   # largest INT8 code magnitude (symmetric absmax INT8, [P4 量化原理])
E4M3_MAX = 448    # largest finite OCP FP8 E4M3 magnitude (1.75 * 2^8)
DQ_FORMATS = ("int8", "fp8", "none")


# --------------------------------------------------------------------------
# NF4 code book [P1 1. NF4; P2 cards 2-3; P4 printed quant book]
# --------------------------------------------------------------------------

def nf4_offset() -> float:
    """Probability of the outermost code.

    Equal-probability bins place the outermost sample inside the open end of the
    CDF, avoiding the infinite quantile at p = 1 [P1 分位数采样与端点问题]; the pages
    do not say how far inside. It is the one free parameter of the construction,
    and the printed quant book [P4 4-bit NormalFloat(NF4)] fixes it: the 16 values
    round to the printed 4 decimals exactly for offsets in [0.9677024, 0.9677083]
    and for no other. The offset used is 0.967704, the six-decimal value that keeps
    every entry farthest inside the rounding interval of its printed digits (at
    least 2.0e-6 from either edge). It lies between the half-bin offsets of a
    15-level and a 16-level scheme, 1 - 1/30 and 1 - 1/32."""
    return 0.967704


def codebook_f64(inv_cdf=None) -> np.ndarray:
    """The 16 NF4 values in float64, ascending, normalised to [-1, 1].

    Asymmetric construction with one shared exact zero [P2 card 3; P1 exact-zero
    remark]: 8 positive values from quantiles at probabilities evenly spaced from
    the offset down to (not including) 1/2, 7 negative values likewise, then
    normalised by the largest quantile so the ends are exactly -1 and +1 [P1
    归一化与匹配; P2 card 2]."""
    q = NormalDist().inv_cdf if inv_cdf is None else inv_cdf
    d = nf4_offset()
    pos = [q(d - i * (d - 0.5) / 8.0) for i in range(8)]
    neg = [-q(d - i * (d - 0.5) / 7.0) for i in range(7)]
    vals = np.sort(np.array(pos + neg + [0.0], dtype=np.float64))
    return vals / q(d)


def codebook() -> np.ndarray:
    """The code book as float32 (each value rounded to nearest), ascending."""
    return codebook_f64().astype(np.float32)


# --------------------------------------------------------------------------
# First level: absmax per block of 64 and nearest code [P1 归一化与匹配; P4 NF4]
# --------------------------------------------------------------------------

def nearest_code(x: np.ndarray) -> np.ndarray:
    """Index of the code-book value nearest to each float32 x in [-1, 1].

    Written as the plain definition: argmin over the 16 values of |x - c_i|,
    the first (lower) index on an exact tie. Distances are taken in float64;
    for float32 operands in [-1, 1] they are exact wherever two distances can
    be close enough to compete, so the argmin is the exact one."""
    c = codebook().astype(np.float64)
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1).astype(np.float64)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 20
    for lo in range(0, flat.size, step):
        d = np.abs(flat[lo:lo + step, None] - c[None, :])
        out[lo:lo + step] = np.argmin(d, axis=1)
    return out.reshape(x.shape)


def to_blocks(w: np.ndarray) -> np.ndarray:
    """Row-major flatten of W, padded with +0.0 to a multiple of 64, as [n_b, 64]."""
    flat = np.asarray(w, dtype=np.float32).reshape(-1)
    n_b = -(-flat.size // BLOCK)
    if n_b * BLOCK != flat.size:
        flat = np.concatenate([flat, np.zeros(n_b * BLOCK - flat.size, np.float32)])
    return flat.reshape(n_b, BLOCK)


def block_absmax(blocks: np.ndarray) -> np.ndarray:
    """a_j = max |W_j| per block, float32 (exact) [P1 DQ section, W_j ~ a_j q]."""
    return np.max(np.abs(blocks), axis=1)


def block_codes(blocks: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Codes [n_b, 64]: x = fl32(w / a_j), then the nearest code.

    A block whose absmax is 0 holds only zeros and takes the exact-zero code
    (index 7) [P2 card 3]."""
    a = np.asarray(a, dtype=np.float32)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)
    x[a == 0] = np.float32(0.0)
    return nearest_code(x)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2i in the low nibble, 2i+1 in the high."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Second level: Double Quantisation of the block constants
# [P1 2. DQ: r_j = (a_j - mu) / b, 8-bit r_hat, a_hat = mu + b r_hat;
#  P2 card 4; P4 Double Quantization]
# --------------------------------------------------------------------------

def f32_from_rational(num: int, den: int) -> np.float32:
    """num/den (num >= 0, den > 0) rounded to the nearest float32, ties to even."""
    if num < 0 or den <= 0:
        raise ValueError("f32_from_rational wants num >= 0, den > 0")
    if num == 0:
        return np.float32(0.0)
    # e such that 2^e <= num/den < 2^(e+1)
    e = num.bit_length() - den.bit_length()
    if (num << max(-e, 0)) < (den << max(e, 0)):
        e -= 1
    # keep 24 significant bits for normal results, a fixed 2^-149 grid below 2^-126
    scale = 23 - e if e >= -126 else 149
    n2, d2 = (num << scale, den) if scale >= 0 else (num, den << -scale)
    q, rem = divmod(n2, d2)
    if 2 * rem > d2 or (2 * rem == d2 and (q & 1)):
        q += 1
    val = math.ldexp(q, -scale)  # q <= 2^24: exact in float64
    if val > float(np.finfo(np.float32).max):
        raise OverflowError("mean outside float32 range")
    return np.float32(val)


def exact_mean_f32(a: np.ndarray) -> np.float32:
    """mu = mean of the block constants, rounded once to float32 (nearest, even).

    The pages subtract "the mean" [P1 DQ]; the order of a float32 running sum
    is not given, so the exact mean (computed with integers) is rounded once.
    Every float32 a >= 0 is an integer multiple of 2^-149."""
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    if a.size == 0:
        raise ValueError("empty")
    bits = a.view(np.uint32).astype(np.int64)
    if np.any(bits >> 31):
        raise ValueError("block constants are absolute maxima, never negative")
    expo = (bits >> 23) & 0xFF
    mant = bits & 0x7FFFFF
    mant = np.where(expo > 0, mant | 0x800000, mant)
    shift = np.maximum(expo, 1) - 1            # a = mant * 2^(shift - 149)
    total = 0
    for sv in np.unique(shift):
        total += int(mant[shift == sv].sum()) << int(sv)
    return f32_from_rational(total, a.size << 149)


def e4m3_values() -> np.ndarray:
    """The 256 OCP FP8 E4M3 codes as float64 values, indexed by the code byte.

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the mantissa.
    Exponent field 0 is subnormal: (m / 8) * 2^-6. Otherwise (1 + m / 8) * 2^(e - 7),
    except that S.1111.111 is NaN (the format has no infinities)."""
    out = np.empty(256, np.float64)
    for u in range(256):
        sign = -1.0 if u & 0x80 else 1.0
        e, m = (u >> 3) & 0xF, u & 0x7
        if e == 0xF and m == 0x7:
            out[u] = np.nan
        elif e == 0:
            out[u] = sign * math.ldexp(m, -9)
        else:
            out[u] = sign * math.ldexp(8 + m, e - 10)
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (uint8) of each float32 v with |v| <= 448.

    The magnitude goes to the nearest of the 127 finite non-negative values (codes
    0x00..0x7E, ascending with the code); an exact tie goes to the even code. The
    sign bit is v's sign bit (-0.0 -> 0x80). The midpoint test 2|v| vs lo + hi is
    exact in float64 (both sides are sums of at most two short dyadic numbers)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_encode expects |v| <= 448")
    pos = e4m3_values()[:0x7F]
    lo = np.clip(np.searchsorted(pos, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    two_a, mid2 = 2.0 * a, pos[lo] + pos[hi]
    up = (two_a > mid2) | ((two_a == mid2) & (hi % 2 == 0))
    code = np.where(up, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def dq_step(qconst: np.ndarray, fmt: str) -> np.ndarray:
    """r_hat = T[q] in float32: fl32(q / 127) for int8, fl32(e4m3(q) / 448) for fp8."""
    if fmt == "int8":
        q = np.asarray(qconst, dtype=np.int8).reshape(-1)
        return (q.astype(np.float32) / np.float32(INT8_STEP)).astype(np.float32)
    if fmt == "fp8":
        u = np.asarray(qconst).reshape(-1).view(np.uint8)
        val = e4m3_values()[u].astype(np.float32)          # exact: 4 significant bits
        return (val / np.float32(E4M3_MAX)).astype(np.float32)
    raise ValueError(fmt)


def dq_encode(a: np.ndarray, mu: np.float32, group: int = DQ_GROUP, fmt: str = "int8"):
    """8-bit codes of the centred constants, one fp32 scale per group of 256.

    d_j = fl32(a_j - mu); b_g = max |d_j| over the group (absmax, as for the
    first level); r_j = fl32(d_j / b_g) in [-1, 1]; then for int8 q_j = round-
    half-even of fl32(r_j * 127), for fp8 q_j = the nearest E4M3 code of
    fl32(r_j * 448). A group with b_g = 0 gets q = 0 (+0 in both formats).
    Returns (q int8 [n_b] (fp8: the code bytes), b float32 [n_g])."""
    a = np.asarray(a, dtype=np.float32).reshape(-1)
    mu = np.float32(mu)
    d = (a - mu).astype(np.float32)
    n_g = -(-a.size // group)
    pad = n_g * group - a.size
    dp = np.concatenate([d, np.zeros(pad, np.float32)]) if pad else d
    b = np.max(np.abs(dp.reshape(n_g, group)), axis=1).astype(np.float32)
    bj = np.repeat(b, group)[: a.size]
    safe = np.where(bj > 0, bj, np.float32(1.0)).astype(np.float32)
    r = (d / safe).astype(np.float32)
    if fmt == "int8":
        q = np.rint((r * np.float32(INT8_STEP)).astype(np.float32))
        q[bj == 0] = 0
        return q.astype(np.int8), b
    if fmt == "fp8":
        code = e4m3_encode((r * np.float32(E4M3_MAX)).astype(np.float32))
        code[bj == 0] = 0
        return code.view(np.int8), b
    raise ValueError(fmt)


def dq_decode(qconst: np.ndarray, qscale: np.ndarray, mu: np.float32, group: int = DQ_GROUP,
              fmt: str = "int8") -> np.ndarray:
    """a_hat_j = fl32(mu + fl32(b_g * T[q_j])), a separate multiply then add; with
    no second level ("none") a_hat_j is the stored a_j itself."""
    if fmt == "none":
        return np.asarray(qscale, dtype=np.float32).reshape(-1).copy()
    rhat = dq_step(qconst, fmt)
    b = np.repeat(np.asarray(qscale, dtype=np.float32), group)[: rhat.size]
    return (np.float32(mu) + (b * rhat).astype(np.float32)).astype(np.float32)


def quantize(w: np.ndarray, dq: str = "int8") -> dict:
    """Full NF4 quantisation of a float32 weight matrix, second level `dq`.

    Returns codes (uint8, 32 bytes per block), qconst (int8 [n_b]; empty for
    "none"), qscale (float32 [n_g]; the a_j themselves [n_b] for "none"), qmean
    (float32 [1]; 0 for "none", where it is not part of the format), the format
    name and the first-level absmax (float32 [n_b], kept for checks)."""
    if dq not in DQ_FORMATS:
        raise ValueError(dq)
    blocks = to_blocks(w)
    a = block_absmax(blocks)
    codes = pack_codes(block_codes(blocks, a))
    if dq == "none":
        return {"codes": codes, "qconst": np.zeros(0, np.int8), "qscale": a.copy(),
                "qmean": np.zeros(1, np.float32), "absmax": a, "dq": dq}
    mu = exact_mean_f32(a)
    qconst, qscale = dq_encode(a, mu, fmt=dq)
    return {"codes": codes, "qconst": qconst, "qscale": qscale,
            "qmean": np.array([mu], np.float32), "absmax": a, "dq": dq}


def block_constants(q: dict) -> np.ndarray:
    """a_hat of every block of a quantize() result."""
    return dq_decode(q["qconst"], q["qscale"], np.float32(q["qmean"][0]), fmt=q.get("dq", "int8"))


def storage_bits_per_param(n: int, double_quant: bool = True) -> float:
    """Bits per weight of the stored buffers for n weights.

    With DQ: 4-bit codes + an 8-bit constant per 64 weights + an fp32 scale per
    256 constants + one fp32 mean. Without DQ: codes + an fp32 constant per 64."""
    n_b = -(-n // BLOCK)
    n_g = -(-n_b // DQ_GROUP)
    if double_quant:
        nbytes = n_b * (BLOCK // 2) + n_b + 4 * n_g + 4
    else:
        nbytes = n_b * (BLOCK // 2) + 4 * n_b
    return 8.0 * nbytes / n


# --------------------------------------------------------------------------
# Double dequantisation to BF16 [P4 QLoRA: constants first, then weights;
# P1 4-bit -> dequant -> BF16; P2 card 1]
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) on the bit pattern; finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def double_dequant(codes: np.ndarray, qconst: np.ndarray, qscale: np.ndarray,
                   qmean, d_out: int, d_in: int, dq: str = "int8") -> np.ndarray:
    """W_hat as bf16 bits [d_out, d_in]: w_hat = bf16(fl32(c[code] * a_hat_j))."""
    n = d_out * d_in
    ahat = dq_decode(qconst, qscale, np.float32(np.asarray(qmean).reshape(-1)[0]), fmt=dq)
    cb = codebook()
    vals = cb[unpack_codes(codes)[: ahat.size * BLOCK]].reshape(-1, BLOCK)
    prod = (vals * ahat[:, None]).astype(np.float32).reshape(-1)[:n]
    return f32_to_bf16_bits(prod).reshape(d_out, d_in)


def dequant_rows(q: dict, d_in: int, rows: np.ndarray) -> np.ndarray:
    """Selected rows of W_hat (bf16 bits) from a quantize() result; d_in % 64 == 0."""
    if d_in % BLOCK:
        raise ValueError("row extraction needs whole blocks per row")
    per_row = d_in // BLOCK
    ahat = block_constants(q)
    cb = codebook()
    out = np.empty((len(rows), d_in), np.uint16)
    codes = q["codes"].reshape(-1, BLOCK // 2)
    for k, row in enumerate(rows):
        bj = np.arange(row * per_row, (row + 1) * per_row)
        vals = cb[unpack_codes(codes[bj])].reshape(per_row, BLOCK)
        out[k] = f32_to_bf16_bits((vals * ahat[bj][:, None]).astype(np.float32)).reshape(-1)
    return out


# --------------------------------------------------------------------------
# 8-bit block quantisation of a weight (adapter factors of the W ~ Q + L R form)
# [P4 量化原理: absmax integer quantisation; P5 (gist.science GPTQ-intrinsic LoRA),
#  "Risultati Chiave / Empirici": the factors L and R kept at 4 or 8 bits]
# --------------------------------------------------------------------------

def int8_quantize(w: np.ndarray):
    """Symmetric absmax INT8 per block of 64 flat elements (row-major, padded with
    +0.0): a_j = max |w|; x = fl32(w / a_j); q = round-half-even(fl32(x * 127)) in
    [-127, 127]; a zero block gets q = 0. Returns (q int8 [n_b * 64], a float32 [n_b])."""
    blocks = to_blocks(w)
    a = block_absmax(blocks)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)
    q = np.rint((x * np.float32(INT8_STEP)).astype(np.float32))
    q[a == 0] = 0
    return q.astype(np.int8).reshape(-1), a


def int8_dequant(q: np.ndarray, a: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """w_hat = bf16(fl32(fl32(q / 127) * a_j)) as bf16 bits [rows, cols]."""
    n = rows * cols
    qf = (np.asarray(q, dtype=np.int8).reshape(-1, BLOCK).astype(np.float32) / np.float32(INT8_STEP)).astype(np.float32)
    prod = (qf * np.asarray(a, dtype=np.float32)[:, None]).astype(np.float32).reshape(-1)[:n]
    return f32_to_bf16_bits(prod).reshape(rows, cols)


def quantize_factor(w: np.ndarray, bits: int):
    """A low-rank factor at 4 bits (NF4 codes, float32 a_j per block: the layout
    without a second level) or 8 bits (int8_quantize). Returns (codes, a)."""
    if bits == 4:
        q = quantize(w, dq="none")
        return q["codes"], q["qscale"]
    if bits == 8:
        return int8_quantize(w)
    raise ValueError("bits must be 4 or 8")


def dequant_factor(codes: np.ndarray, a: np.ndarray, bits: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bits [rows, cols] of a factor from quantize_factor."""
    if bits == 4:
        return double_dequant(codes, np.zeros(0, np.int8), a, np.zeros(1, np.float32), rows, cols, dq="none")
    if bits == 8:
        return int8_dequant(codes, a, rows, cols)
    raise ValueError("bits must be 4 or 8")


# --------------------------------------------------------------------------
# The linear layer [P1 LoRA: y = W0 x + s B (A x), x in R^{d_in x d_seq};
# P2 card 1: gradients flow through the dequantised weights]
# --------------------------------------------------------------------------

def _f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def linear_fwd(w_hat: np.ndarray, a: np.ndarray, b: np.ndarray, s: float, x: np.ndarray) -> np.ndarray:
    """Y = W_hat X + s B (A X) in float64.

    Arrays are bf16 bits in torch layout: w_hat [d_out, d_in], a [r, d_in],
    b [d_out, r], x [d_seq, d_in] (one token per row). Returns Y as
    [d_seq, d_out] float64, i.e. (W_hat X)^T in the pages' column convention."""
    W, A, B, X = _f64(w_hat), _f64(a), _f64(b), _f64(x)
    s = float(np.float32(s))
    return X @ W.T + s * ((X @ A.T) @ B.T)


def linear_bwd_x(w_hat: np.ndarray, a: np.ndarray, b: np.ndarray, s: float, dy: np.ndarray) -> np.ndarray:
    """dX = W_hat^T dY + s A^T (B^T dY) in float64, the adjoint of linear_fwd.

    dy is bf16 bits [d_seq, d_out]; returns dX as [d_seq, d_in] float64."""
    W, A, B, dY = _f64(w_hat), _f64(a), _f64(b), _f64(dy)
    s = float(np.float32(s))
    return dY @ W + s * ((dY @ B) @ A)


def lora_grads(a: np.ndarray, b: np.ndarray, s: float, x: np.ndarray, dy: np.ndarray):
    """Gradients of the adapter factors, (dA [r, d_in], dB [d_out, r]) in float64.

    Only A and B are trained; the frozen quantised weight gets no update
    [P2 card 1; P1 LoRA]. For the loss gradient dY = dL/dY of the forward
    Y = X W_hat^T + s (X A^T) B^T (torch layout, one token per row):
        dB = s dY^T (X A^T),   dA = s (dY B)^T X.
    Neither depends on W_hat. Inputs are bf16 bits: a [r, d_in], b [d_out, r],
    x [d_seq, d_in], dy [d_seq, d_out]."""
    A, B, X, dY = _f64(a), _f64(b), _f64(x), _f64(dy)
    s = float(np.float32(s))
    dB = s * (dY.T @ (X @ A.T))
    dA = s * ((dY @ B).T @ X)
    return dA, dB
