"""Every entry point captured in a HIP graph and replayed with new inputs.

The library enqueues only kernel launches (no memsets, copies, allocations or host
synchronisation), and each launch reads its inputs from the pointers it was given, so
a captured call replays correctly when the caller rewrites the input buffers in place.
Each replay here follows fresh inputs and some unrelated eager work, and must equal
the eager call on the same inputs bit for bit (every kernel is deterministic)."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_05_amd as qn
import workloads as WL
from parity import dev, to_gpu_bf16, to_gpu_f32

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _say(*a):
    print(*a, flush=True)


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _other_eager_work():
    a = torch.randn(512, 512, device=dev())
    (a @ a).sum().item()


def _bf16(shape, gen):
    return torch.randn(shape, generator=gen, device=dev()).to(torch.bfloat16)


CASES = [
    ("decode_4096x4096", WL.CONFIGS["decode"], 1),                 # one-launch GEMV (r = 16)
    ("decode_two_launch", WL.custom("g2", 512, 4160, 1, 24), 1),   # A x slice kernel + GEMV
    ("gemv_three_tokens", WL.custom("g3", 1024, 4096, 3, 16), 3),  # the GEMV on 3 tokens
    ("small_batch", WL.custom("gs", 1024, 2048, 16, 16), 16),      # small-batch kernel + reduce
    ("small_batch_40", WL.custom("gs2", 1024, 2048, 40, 16), 40),  # the same on three token tiles
    ("gemm_path", WL.custom("gg", 1024, 1536, 300, 16), 300),      # prologue (+ reduce) + GEMM, dX with B itself
    ("gemm_split_r40", WL.custom("gk", 512, 4096, 200, 40), 200),  # split GEMM; dX through a transpose of B
]


@pytest.mark.parametrize("name,cfg,d_seq", CASES, ids=[c[0] for c in CASES])
def test_linear_calls_replay(name, cfg, d_seq):
    _say(f"[graph] {name} {cfg.d_out}x{cfg.d_in} d_seq={d_seq} r={cfg.r}")
    q = qn.quantize(to_gpu_f32(WL.make_weight(cfg)))
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    gen = torch.Generator(device=dev()).manual_seed(11)
    X = _bf16((d_seq, cfg.d_in), gen)
    dY = _bf16((d_seq, cfg.d_out), gen)
    Y = torch.empty(d_seq, cfg.d_out, dtype=torch.bfloat16, device=dev())
    dX = torch.empty(d_seq, cfg.d_in, dtype=torch.bfloat16, device=dev())
    ws = torch.empty(qn.linear_workspace_bytes(cfg.d_out, cfg.d_in, d_seq, cfg.r), dtype=torch.uint8, device=dev())

    def calls():
        qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=ws)
        qn.linear_bwd_x(q, A, B, cfg.s, dY, out=dX, workspace=ws)

    g = _capture(calls)
    Ye, dXe = torch.empty_like(Y), torch.empty_like(dX)
    ws_e = torch.empty_like(ws)
    for k in range(REPLAYS):
        X.copy_(_bf16(X.shape, gen))
        dY.copy_(_bf16(dY.shape, gen))
        A.copy_(_bf16(A.shape, gen) * 0.01)         # the adapters change between steps too
        _other_eager_work()
        g.replay()
        torch.cuda.synchronize()
        qn.linear_fwd(q, A, B, cfg.s, X, out=Ye, workspace=ws_e)
        qn.linear_bwd_x(q, A, B, cfg.s, dY, out=dXe, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Ye.view(torch.int16)), f"forward, replay {k}"
        assert torch.equal(dX.view(torch.int16), dXe.view(torch.int16)), f"input gradient, replay {k}"


def test_quantize_and_lora_grads_replay():
    cfg = WL.custom("gq", 768, 1024, 96, 16)
    _say("[graph] quantize + adapter gradients 768x1024, 96 tokens, r=16")
    W = to_gpu_f32(WL.make_weight(cfg))
    q = qn.quantize(W)
    qws = torch.empty(qn.quantize_workspace_bytes(cfg.d_out, cfg.d_in), dtype=torch.uint8, device=dev())
    a, b = WL.make_lora(cfg)
    A, B = to_gpu_bf16(a), to_gpu_bf16(b)
    gen = torch.Generator(device=dev()).manual_seed(12)
    X = _bf16((cfg.d_seq, cfg.d_in), gen)
    dY = _bf16((cfg.d_seq, cfg.d_out), gen)
    dA = torch.empty(cfg.r, cfg.d_in, dtype=torch.float32, device=dev())
    dB = torch.empty(cfg.d_out, cfg.r, dtype=torch.float32, device=dev())
    gws = torch.empty(qn.lora_grads_workspace_bytes(cfg.d_out, cfg.d_in, cfg.d_seq, cfg.r), dtype=torch.uint8,
                      device=dev())

    def calls():
        qn.quantize(W, out=q, workspace=qws)
        qn.lora_grads(A, B, cfg.s, X, dY, dA=dA, dB=dB, workspace=gws)

    g = _capture(calls)
    qe = qn.quantize(W)
    dAe, dBe = torch.empty_like(dA), torch.empty_like(dB)
    for k in range(REPLAYS):
        W.copy_(torch.randn(W.shape, generator=gen, device=dev()) * 0.02)
        X.copy_(_bf16(X.shape, gen))
        dY.copy_(_bf16(dY.shape, gen))
        _other_eager_work()
        g.replay()
        torch.cuda.synchronize()
        qn.quantize(W, out=qe, workspace=torch.empty_like(qws))
        qn.lora_grads(A, B, cfg.s, X, dY, dA=dAe, dB=dBe, workspace=torch.empty_like(gws))
        torch.cuda.synchronize()
        for x, y, what in ((q.codes, qe.codes, "codes"), (q.qconst, qe.qconst, "qconst"),
                           (q.qscale, qe.qscale, "qscale"), (q.qmean, qe.qmean, "qmean")):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{what}, replay {k}"
        assert torch.equal(dA, dAe) and torch.equal(dB, dBe), f"adapter gradients, replay {k}"
