"""The largest linear layer the library accepts, through the C ABI, against the oracle.

Every operand of the GEMM is addressed with 32-bit byte offsets, so the API takes a
weight of fewer than 2^31 entries (W_hat under 4 GiB in bf16). This layer is
32768 x 65472 = 2 145 386 496 weights (4 GiB - 4 MiB of W_hat), W ~ N(0, 0.02^2),
LoRA r = 16: quantisation (constants in full, codes of sampled blocks including the
last ones) and dequantisation bit-exact, then the forward on each of its three paths
(1, 16 and 65 tokens) and the input gradient within the GEMM tolerance, on sampled
rows / column blocks that include the last ones. Host memory: about 30 GB."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from oracle import nf4_oracle as O
from parity import OracleLayer, bf16_bits, bf16_f64, check_close, dev, to_gpu_bf16

pytestmark = pytest.mark.gpu

D_OUT, D_IN, R, S = 32768, 65472, 16, 2.0


def _say(*a):
    print(*a, flush=True)


def test_largest_accepted_layer():
    n = D_OUT * D_IN
    assert 2 * n < 2 ** 32 <= 2 * (D_OUT + 64) * D_IN      # 64 more rows would reach 4 GiB
    _say(f"[max size] generating W {D_OUT}x{D_IN}")
    w = np.random.default_rng(2026).standard_normal(n, dtype=np.float32).reshape(D_OUT, D_IN)
    w *= np.float32(0.02)
    Wd = torch.from_numpy(w).to(dev())
    q = qn.quantize(Wd)
    torch.cuda.synchronize()
    del Wd
    torch.cuda.empty_cache()
    _say("[max size] oracle constants")
    ol = OracleLayer(w)
    del w
    assert np.array_equal(q.qmean.cpu().numpy().view(np.uint32), np.array([ol.mu], np.float32).view(np.uint32))
    assert np.array_equal(q.qscale.cpu().numpy().view(np.uint32), ol.qscale.view(np.uint32))
    assert np.array_equal(q.qconst.cpu().numpy(), ol.qconst)
    n_b = ol.absmax.size
    rng = np.random.default_rng(3)
    sel = np.unique(np.concatenate([np.arange(64), n_b - 256 + np.arange(256), rng.choice(n_b, 4096, replace=False)]))
    got = q.codes.cpu().numpy().reshape(-1, 32)[sel]
    assert np.array_equal(got, O.pack_codes(ol.codes_of(sel)).reshape(-1, 32)), "codes (sampled blocks)"

    _say("[max size] dequantise")
    rows = np.unique(np.concatenate([[0, 1, D_OUT - 2, D_OUT - 1], rng.choice(D_OUT, 12, replace=False)]))
    rt = torch.from_numpy(rows).to(dev())
    wh = qn.double_dequant(q)
    torch.cuda.synchronize()
    w_rows = ol.rows(rows)
    assert np.array_equal(bf16_bits(wh[rt]), w_rows)
    del wh
    torch.cuda.empty_cache()

    cfg = WL.custom("max", D_OUT, D_IN, 65, R, s=S)
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    for d_seq in (1, 16, 65):
        _say(f"[max size] forward, {d_seq} tokens")
        x = WL.make_x(cfg, d_seq)
        y = qn.linear_fwd(q, A, B, S, to_gpu_bf16(x))
        torch.cuda.synchronize()
        check_close(bf16_f64(y[:, rt]), O.linear_fwd(w_rows, a, b[rows], S, x), f"fwd max size, {d_seq} tokens")
        del y

    _say("[max size] input gradient, 65 tokens")
    dy = WL.make_dy(cfg, 65)
    dx = qn.linear_bwd_x(q, A, B, S, to_gpu_bf16(dy))
    torch.cuda.synchronize()
    cblk = np.array([0, 1, D_IN // 64 - 1])
    cols = (cblk[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    got = bf16_f64(dx[:, torch.from_numpy(cols).to(dev())])
    check_close(got, O.linear_bwd_x(ol.col_blocks(cblk), a[:, cols], b, S, dy), "bwd_x max size")


def test_long_sequence():
    """131072 tokens on a 1024 x 1024 layer (r = 16): the pre-pass runs 1024 token
    tiles unsplit, the GEMMs 512 x 4 tiles, the adapter gradients many token slices;
    forward, input gradient and adapter gradients on sampled tokens (incl. the last)."""
    cfg = WL.custom("long", 1024, 1024, 131072, 16, s=1.5)
    _say(f"[long sequence] {cfg.d_out}x{cfg.d_in}, {cfg.d_seq} tokens")
    w = WL.make_weight(cfg)
    q = qn.quantize(torch.from_numpy(w).to(dev()))
    ol = OracleLayer(w)
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    x, dy = WL.make_x(cfg), WL.make_dy(cfg)
    X, dY = to_gpu_bf16(x), to_gpu_bf16(dy)
    y = qn.linear_fwd(q, A, B, cfg.s, X)
    dx = qn.linear_bwd_x(q, A, B, cfg.s, dY)
    dA, dB = qn.lora_grads(A, B, cfg.s, X, dY)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    toks = np.unique(np.concatenate([[0, 127, 128, cfg.d_seq - 129, cfg.d_seq - 1], rng.choice(cfg.d_seq, 59, replace=False)]))
    tt = torch.from_numpy(toks).to(dev())
    wh = ol.rows(np.arange(cfg.d_out))
    check_close(bf16_f64(y[tt]), O.linear_fwd(wh, a, b, cfg.s, x[toks]), "fwd long sequence (sampled tokens)")
    check_close(bf16_f64(dx[tt]), O.linear_bwd_x(wh, a, b, cfg.s, dy[toks]), "bwd_x long sequence (sampled tokens)")
    # adapter gradients sum over every token: checked in full against the oracle
    rA, rB = O.lora_grads(a, b, cfg.s, x, dy)
    check_close(dA.cpu().numpy().astype(np.float64), rA, "dA long sequence")
    check_close(dB.cpu().numpy().astype(np.float64), rB, "dB long sequence")
