#!/usr/bin/env python3
"""Throughput of the QLoRA NF4 linear-layer hot path on one MI355X.

One step = every stage of the path on the 4096 x 4096 layer (NF4 blocks of 64,
DQ groups of 256, LoRA r = 16, s = 2), inputs already resident in HBM:
    nf4_quantize(W)                  block absmax, NF4 codes, DQ constants
    qlora_linear_fwd(X), d_seq=4096  dequant + A X pre-pass + fused MFMA GEMM
    qlora_linear_bwd_x(dY)           transposed dequant + B^T dY + fused MFMA GEMM
    qlora_linear_fwd(x), d_seq=1     streaming GEMV on one of 32 rotated layer copies
`value` = algorithmic flops of the step (both GEMMs with their LoRA terms and the
GEMV; quantisation counts 0 flops) / step time, in TFLOP/s.

Also reported: per-kernel average durations (HIP events recorded by the library
on each kernel's own stream, in a second pass of the same K steps right after the
timed one, so the event records do not perturb `value`), the MFMA roofline fraction of
the dominant kernel (the GEMM), the decode path's effective GB/s over 32 layer
copies (> 256 MB, beyond the Infinity Cache), the small-batch forward (2, 16 and 64
tokens) over the same rotated copies, quantise and decode with the FP8 and no-DQ
second levels next to INT8, quantise / forward / dX of the MLP pair (11008x4096 and
4096x11008, r = 64, 2048 tokens) and the large layer (28672x8192, r = 64, 8192
tokens), and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "QLoRA linear TFLOP/s (prefill/bwd) + effective GB/s (d_seq=1) at 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-copies", type=int, default=32)
    ap.add_argument("--decode-iters", type=int, default=256)
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the MLP-pair and large-layer legs (quantise, fwd, dX on 11008x4096, 4096x11008 "
                         "and 28672x8192)")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the prefill workload the CPU oracle runs (0 = skip the CPU baseline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three plain 512 MiB device copies (the reference for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


_ROOT = os.path.dirname(os.path.abspath(__file__))
# counter summaries under profiles/ and the kernel source each was measured with
GEMM_TRAFFIC = ("gemm_nt_kernel_4096x4096x4160_traffic.md", "gemm_nt.hip")
DECODE_TRAFFIC = ("gemv_nf4_kernel_4096x4096_decode_traffic.md", "gemv.hip")


def measured_traffic(which):
    """HBM bytes per launch (per call for the decode pair) from a committed counter
    summary, or None when the kernel source has changed since the counters were taken
    (the summary records the SHA-256 of the source file it was measured with)."""
    import hashlib
    import re
    profile, source = which
    try:
        text = open(os.path.join(_ROOT, "profiles", profile)).read()
        src = os.path.join(_ROOT, "bit_nf4_quantized_05_amd", "csrc", source)
        src_hash = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not h or not t or h.group(1) != src_hash:
        return None
    return int(t.group(1))


def copy_calibration():
    """Three plain copies of 512 MiB: each reads and writes exactly 2^29 bytes."""
    import torch
    n = 512 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def weight_bytes(cfg, dq: str = "int8") -> int:
    """Stored bytes of the quantised weight: packed codes plus the block constants
    (8-bit codes, group scales and the mean; or one float32 per block without DQ)."""
    n = cfg.d_out * cfg.d_in
    n_b = n // 64
    n_g = -(-n_b // 256)
    return n // 2 + (4 * n_b if dq == "none" else n_b + 4 * n_g + 4)


def decode_bytes(cfg, dq: str = "int8", d_seq: int = 1) -> int:
    """Algorithmic HBM bytes of one forward call with few tokens: the quantised
    weight, A, B, X and Y."""
    return weight_bytes(cfg, dq) + 2 * cfg.r * (cfg.d_in + cfg.d_out) + 2 * d_seq * (cfg.d_in + cfg.d_out)


def timed_calls(qn, torch, fn, iters: int):
    """Back-to-back microseconds per call of fn(i), then the library's per-kernel
    averages (HIP events on each kernel's stream) over a second pass."""
    for i in range(4):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        fn(i)
    torch.cuda.synchronize()
    call_us = 1e6 * (time.perf_counter() - t0) / iters
    qn.profile_enable(True)
    for i in range(iters):
        fn(i)
    torch.cuda.synchronize()
    prof = qn.profile_read()
    qn.profile_enable(False)
    return call_us, {k: round(1e3 * ms / n, 3) for k, (n, ms) in sorted(prof.items())}


def layer_leg(qn, torch, WL, name: str, dev) -> dict:
    """Quantise, forward and input gradient of one full-size layer (inputs resident in
    HBM): call times back to back, and the GEMM's TFLOP/s from its kernel events."""
    import numpy as np
    cfg = WL.CONFIGS[name]

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    W = torch.from_numpy(WL.make_weight(cfg)).to(dev)
    a, b = WL.make_lora(cfg)
    A, B = bf16(a), bf16(b)
    X, dY = bf16(WL.make_x(cfg)), bf16(WL.make_dy(cfg))
    q = qn.quantize(W)
    qws = torch.empty(qn.quantize_workspace_bytes(cfg.d_out, cfg.d_in), dtype=torch.uint8, device=dev)
    lws = torch.empty(qn.linear_workspace_bytes(cfg.d_out, cfg.d_in, cfg.d_seq, cfg.r), dtype=torch.uint8, device=dev)
    Y = torch.empty(cfg.d_seq, cfg.d_out, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(cfg.d_seq, cfg.d_in, dtype=torch.bfloat16, device=dev)
    n = cfg.d_out * cfg.d_in
    q_us, q_k = timed_calls(qn, torch, lambda i: qn.quantize(W, out=q, workspace=qws), 5)
    f_us, f_k = timed_calls(qn, torch, lambda i: qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=lws), 3)
    b_us, b_k = timed_calls(qn, torch, lambda i: qn.linear_bwd_x(q, A, B, cfg.s, dY, out=dX, workspace=lws), 3)
    gemm_flops = cfg.fwd_flops()                     # fwd and dX have the same algorithmic flops

    def tf(us):
        return round(gemm_flops / (us * 1e-6) / 1e12, 1)

    def gemm_us(k):
        # the GEMM of a call: one gemm_nt_kernel, or (few tiles) gemm_nt_split + its reduce
        return sum(v for name, v in k.items() if name.startswith("gemm_"))
    gf, gb = gemm_us(f_k), gemm_us(b_k)
    out = {"d_out": cfg.d_out, "d_in": cfg.d_in, "d_seq": cfg.d_seq, "r": cfg.r,
           "quantize_us": round(q_us, 2), "quantize_kernel_us": q_k,
           "quantize_GBps": round(4.516 * n / (q_us * 1e-6) / 1e9, 1),
           "fwd_call_us": round(f_us, 2), "fwd_kernel_us": f_k, "fwd_TFLOPs": tf(f_us),
           "bwd_x_call_us": round(b_us, 2), "bwd_x_kernel_us": b_k, "bwd_x_TFLOPs": tf(b_us),
           "fwd_gemm_TFLOPs": tf(gf), "fwd_gemm_frac_of_peak": round(gemm_flops / (gf * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "bwd_x_gemm_TFLOPs": tf(gb),
           "bwd_x_gemm_frac_of_peak": round(gemm_flops / (gb * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del W, X, dY, Y, dX, lws, qws, q
    torch.cuda.empty_cache()
    return out


def rotated_copies(qn, q, n: int, dev) -> list:
    """n device copies of the quantised weight q (rotating through them keeps each
    call's weight out of the 256 MB Infinity Cache)."""
    out = []
    for _ in range(n):
        c = qn.alloc_weight(q.d_out, q.d_in, dev, q.dq)
        for dst, src in ((c.codes, q.codes), (c.qconst, q.qconst), (c.qscale, q.qscale), (c.qmean, q.qmean)):
            dst.copy_(src)
        out.append(c)
    return out


def cpu_baseline(cfg, dcfg, tokens: int) -> dict:
    """The oracle, as it stands, on the step's workload (or a token sample of it):
    full quantise + dequantise of W, forward and input gradient for `tokens`
    tokens, and the d_seq = 1 forward, in float64 with numpy."""
    import numpy as np
    import workloads as WL
    from oracle import nf4_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    w = WL.make_weight(cfg)
    a, b = WL.make_lora(cfg)
    x = WL.make_x(cfg)[:tokens]
    dy = WL.make_dy(cfg)[:tokens]
    x1 = WL.make_x(dcfg)
    t0 = time.perf_counter()
    q = O.quantize(w)
    wh = O.double_dequant(q["codes"], q["qconst"], q["qscale"], q["qmean"], cfg.d_out, cfg.d_in)
    O.linear_fwd(wh, a, b, cfg.s, x)
    O.linear_bwd_x(wh, a, b, cfg.s, dy)
    O.linear_fwd(wh, a, b, dcfg.s, x1)
    dt = time.perf_counter() - t0
    flops = 2 * (2 * cfg.d_out * cfg.d_in * tokens + 2 * cfg.r * tokens * (cfg.d_in + cfg.d_out)) + dcfg.fwd_flops()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": (f"{cfg.d_out}x{cfg.d_in} layer: full NF4+DQ quantise and bf16 dequantise, fwd + dX for "
                       f"{tokens} of the {cfg.d_seq} tokens and the d_seq=1 forward, float64 numpy "
                       f"(BLAS threads = cores)")}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU path is design-only in this library.", flush=True)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_05_amd as qn
    import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", flush=True)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    cfg = WL.CONFIGS["prefill"]
    dcfg = WL.CONFIGS["decode"]
    assert (cfg.d_out, cfg.d_in, cfg.r, cfg.s) == (dcfg.d_out, dcfg.d_in, dcfg.r, dcfg.s)

    def bf16(bits):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    log("[bench] generating inputs")
    W = torch.from_numpy(WL.make_weight(cfg)).to(dev)
    a_bits, b_bits = WL.make_lora(cfg)
    A, B = bf16(a_bits), bf16(b_bits)
    X = bf16(WL.make_x(cfg))
    dY = bf16(WL.make_dy(cfg))
    x1 = bf16(WL.make_x(dcfg))

    q = qn.quantize(W)
    qws = torch.empty(qn.quantize_workspace_bytes(cfg.d_out, cfg.d_in), dtype=torch.uint8, device=dev)
    lws = torch.empty(qn.linear_workspace_bytes(cfg.d_out, cfg.d_in, cfg.d_seq, cfg.r), dtype=torch.uint8,
                      device=dev)
    dws = torch.empty(qn.linear_workspace_bytes(dcfg.d_out, dcfg.d_in, 1, dcfg.r), dtype=torch.uint8, device=dev)
    Y = torch.empty(cfg.d_seq, cfg.d_out, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(cfg.d_seq, cfg.d_in, dtype=torch.bfloat16, device=dev)
    y1 = torch.empty(1, dcfg.d_out, dtype=torch.bfloat16, device=dev)
    copies = rotated_copies(qn, q, args.decode_copies, dev)
    torch.cuda.synchronize()

    def step(i):
        qn.quantize(W, out=q, workspace=qws)
        qn.linear_fwd(q, A, B, cfg.s, X, out=Y, workspace=lws)
        qn.linear_bwd_x(q, A, B, cfg.s, dY, out=dX, workspace=lws)
        qn.linear_fwd(copies[i % len(copies)], A, B, dcfg.s, x1, out=y1, workspace=dws)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    step_flops = 2 * cfg.fwd_flops() + dcfg.fwd_flops()
    value = step_flops / (elapsed / args.steps) / 1e12

    # ---- the same K steps again with the library's per-kernel HIP events on
    log(f"[bench] profiled pass of {args.steps} steps")
    qn.profile_enable(True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof_elapsed = time.perf_counter() - t0
    prof = qn.profile_read()
    qn.profile_enable(False)
    kernels = {k: {"launches": n, "avg_us": round(1e3 * ms / n, 3)} for k, (n, ms) in sorted(prof.items())}
    log("[bench] kernels:", json.dumps(kernels))

    # dominant kernel: the fused GEMM (fwd and dX launches have equal algorithmic flops)
    g_n, g_ms = prof["gemm_nt_kernel"]
    gemm_flops = 2 * cfg.d_seq * cfg.d_out * cfg.d_in + 2 * cfg.d_seq * cfg.d_out * cfg.r
    achieved = gemm_flops / (g_ms / g_n * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "gemm_nt_kernel", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(GEMM_TRAFFIC)}

    # ---- decode (d_seq = 1) over rotated layer copies
    log(f"[bench] decode: {args.decode_iters} calls over {len(copies)} copies")
    for i in range(len(copies)):
        qn.linear_fwd(copies[i], A, B, dcfg.s, x1, out=y1, workspace=dws)
    torch.cuda.synchronize()
    qn.profile_enable(True)
    t0 = time.perf_counter()
    for i in range(args.decode_iters):
        qn.linear_fwd(copies[i % len(copies)], A, B, dcfg.s, x1, out=y1, workspace=dws)
    torch.cuda.synchronize()
    d_elapsed = time.perf_counter() - t0
    dprof = qn.profile_read()
    qn.profile_enable(False)
    nbytes = decode_bytes(dcfg)
    # the same calls captured once in a HIP graph and replayed (a serving loop without host
    # launch cost): GPU time per call including the gaps between launches
    log("[bench] decode: the calls over all copies in one HIP graph")

    def decode_all():
        for i in range(len(copies)):
            qn.linear_fwd(copies[i], A, B, dcfg.s, x1, out=y1, workspace=dws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_all()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g_reps = max(1, args.decode_iters // len(copies))
    e0.record()
    for _ in range(g_reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_call_us = 1e3 * e0.elapsed_time(e1) / (g_reps * len(copies))
    del graph

    # one launch when A fits one segment (this layer); else the A x slice kernel runs first
    dk = {k: 1e3 * ms / n for k, (n, ms) in dprof.items() if k in ("gemv_nf4_kernel", "lora_ax_partial_kernel")}
    gv_n, gv_ms = dprof["gemv_nf4_kernel"]
    kern_us = sum(dk.values())
    # value: GPU time per call from the graph replay (HIP events around many calls on the
    # launch stream, gaps between launches included); per-kernel events add about 2.5 us
    # of their own to a launch this short and are reported beside it
    d_gbps = nbytes / (graph_call_us * 1e-6) / 1e9
    decode = {"metric": "effective GB/s (d_seq=1)", "value": round(d_gbps, 1),
              "unit": "GB/s", "bytes_per_call": nbytes, "call_us_graph_replay": round(graph_call_us, 3),
              "kernel_us_events": round(kern_us, 3), "gemv_kernel_us_events": round(1e3 * gv_ms / gv_n, 3),
              "call_us_back_to_back": round(1e6 * d_elapsed / args.decode_iters, 3),
              "copies": len(copies),
              "roofline": {"bound": "hbm", "kernel": " + ".join(sorted(dk)),
                           "achieved": round(d_gbps, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(d_gbps / PEAK_HBM_GBPS, 4),
                           "traffic": measured_traffic(DECODE_TRAFFIC)}}

    # ---- adapter gradients (dA, dB) of the same layer, outside the timed step
    log(f"[bench] adapter gradients: {args.steps} calls")
    gws = torch.empty(qn.lora_grads_workspace_bytes(cfg.d_out, cfg.d_in, cfg.d_seq, cfg.r), dtype=torch.uint8,
                      device=dev)
    gA = torch.empty(cfg.r, cfg.d_in, dtype=torch.float32, device=dev)
    gB = torch.empty(cfg.d_out, cfg.r, dtype=torch.float32, device=dev)
    for _ in range(2):
        qn.lora_grads(A, B, cfg.s, X, dY, dA=gA, dB=gB, workspace=gws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        qn.lora_grads(A, B, cfg.s, X, dY, dA=gA, dB=gB, workspace=gws)
    torch.cuda.synchronize()
    g_elapsed = (time.perf_counter() - t0) / args.steps
    qn.profile_enable(True)
    for _ in range(args.steps):
        qn.lora_grads(A, B, cfg.s, X, dY, dA=gA, dB=gB, workspace=gws)
    torch.cuda.synchronize()
    gprof = qn.profile_read()
    qn.profile_enable(False)
    # algorithmic bytes: one read of X and dY, A and B, the fp32 gradients written
    g_bytes = 2 * cfg.d_seq * (cfg.d_in + cfg.d_out) + 2 * 2 * cfg.r * (cfg.d_in + cfg.d_out) + \
        4 * cfg.r * (cfg.d_in + cfg.d_out)
    lora_grads = {"metric": "adapter gradients dA, dB (effective GB/s)",
                  "value": round(g_bytes / g_elapsed / 1e9, 1), "unit": "GB/s", "bytes_per_call": g_bytes,
                  "call_us": round(1e6 * g_elapsed, 2),
                  "kernel_us": {k: round(1e3 * ms / n, 2) for k, (n, ms) in sorted(gprof.items())}}

    # ---- small batch (2 <= d_seq <= 64): codes streamed once, over the rotated copies
    small_batch = {}
    for d_seq in (2, 16, 64):
        xs = bf16(WL.make_x(WL.custom("sb", dcfg.d_out, dcfg.d_in, d_seq, dcfg.r, s=dcfg.s)))
        ys = torch.empty(d_seq, dcfg.d_out, dtype=torch.bfloat16, device=dev)
        sws = torch.empty(qn.linear_workspace_bytes(dcfg.d_out, dcfg.d_in, d_seq, dcfg.r), dtype=torch.uint8,
                          device=dev)
        log(f"[bench] small batch d_seq={d_seq}")
        call_us, kus = timed_calls(qn, torch, lambda i: qn.linear_fwd(copies[i % len(copies)], A, B, dcfg.s, xs,
                                                                      out=ys, workspace=sws), args.decode_iters)
        kern = sum(kus.values())
        nb = decode_bytes(dcfg, "int8", d_seq)
        small_batch[str(d_seq)] = {"call_us_back_to_back": round(call_us, 3), "kernel_us": kus,
                                   "bytes_per_call": nb, "effective_GBps": round(nb / (kern * 1e-6) / 1e9, 1)}

    # ---- second-level formats: quantise and decode with FP8 constants and with none
    dq_formats = {}
    for dq in ("int8", "fp8", "none"):
        log(f"[bench] format {dq}")
        qf = qn.quantize(W, dq=dq)
        q_us, q_k = timed_calls(qn, torch, lambda i: qn.quantize(W, out=qf, workspace=qws, dq=dq), args.steps)
        fcopies = rotated_copies(qn, qf, args.decode_copies, dev)
        d_us, d_k = timed_calls(qn, torch, lambda i: qn.linear_fwd(fcopies[i % len(fcopies)], A, B, dcfg.s, x1,
                                                                    out=y1, workspace=dws), args.decode_iters)
        nb = decode_bytes(dcfg, dq)
        dq_formats[dq] = {"bits_per_param": round(8 * weight_bytes(dcfg, dq) / (dcfg.d_out * dcfg.d_in), 4),
                          "quantize_call_us": round(q_us, 3), "quantize_kernel_us": q_k,
                          "decode_call_us_back_to_back": round(d_us, 3), "decode_kernel_us": d_k,
                          "decode_bytes_per_call": nb,
                          "decode_effective_GBps": round(nb / (sum(d_k.values()) * 1e-6) / 1e9, 1)}
        del fcopies

    # ---- the MLP pair and the large layer (outside the timed step)
    layers = {}
    if not args.no_layers:
        for name in ("mlp_up", "mlp_down", "large"):
            log(f"[bench] layer {name}")
            layers[name] = layer_leg(qn, torch, WL, name, dev)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian weights and activations, workloads.py)",
        "config": {"workload": "4096x4096 NF4/64+DQ/256 layer, r=16 s=2: quantize + fwd and dX at d_seq=4096 "
                               "+ decode GEMV at d_seq=1",
                   "d_out": cfg.d_out, "d_in": cfg.d_in, "d_seq": cfg.d_seq, "r": cfg.r, "s": cfg.s,
                   "decode_copies": len(copies)},
        "roofline": roofline,
        "decode": decode,
        "lora_grads": lora_grads,
        "small_batch": small_batch,
        "dq_formats": dq_formats,
        "layers": layers,
        "kernels": kernels,
        "ms_per_step_profiled": round(prof_elapsed * 1e3 / args.steps, 4),
    }
    if args.cpu_tokens > 0:
        log(f"[bench] cpu baseline: oracle on {args.cpu_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(cfg, dcfg, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
