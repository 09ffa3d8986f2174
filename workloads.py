"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module only draws random numbers and shapes them; it holds none of the
layer's arithmetic (no quantisation, no dequantisation, no products). Both the
CPU oracle tests and the GPU path take their inputs from here, so the two sides
always see identical bytes.

Value distributions follow the pages' premise that pretrained weights are
roughly zero-centred normal (whoami-wesleyyou.top "LoRA 与 QLoRA", section
"Gaussian 假设与分位数"; learn.ifs.name QLoRA deck, card 2), with the layer
shapes of a 4096-wide decoder block, an MLP pair and a large projection.

bf16 tensors are returned as uint16 bit patterns; the float32 -> bf16 rounding
of the random draws is done by torch's own conversion (round to nearest even).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    d_out: int
    d_in: int
    d_seq: int
    r: int
    s: float
    w_sigma: float
    ab_sigma: float = 0.01
    outlier_frac: float = 0.0      # fraction of W entries scaled by outlier_scale
    outlier_scale: float = 10.0
    seed: int = 0

    @property
    def n(self) -> int:
        return self.d_out * self.d_in

    def fwd_flops(self) -> int:
        """Algorithmic flops of Y = W X + s B (A X) (dequantisation not counted)."""
        return 2 * self.d_out * self.d_in * self.d_seq + 2 * self.r * self.d_seq * (self.d_in + self.d_out)

    bwd_x_flops = fwd_flops  # dX = W^T dY + s A^T (B^T dY) has the same count


# The five layer workloads. Sizes, distributions, ranks and scales follow the
# QLoRA linear-layer study: tiny 256x256 check layer, a 4096x4096 layer in
# decode (one token) and prefill (4096 tokens), an 11008/4096 MLP pair with
# 0.1% outlier weights, and a 28672x8192 projection.
CONFIGS = {
    "tiny": LayerConfig("tiny", 256, 256, 16, 8, 2.0, 0.02),
    "decode": LayerConfig("decode", 4096, 4096, 1, 16, 2.0, 0.02),
    "prefill": LayerConfig("prefill", 4096, 4096, 4096, 16, 2.0, 0.02),
    "mlp_up": LayerConfig("mlp_up", 11008, 4096, 2048, 64, 2.0, 0.02, outlier_frac=0.001),
    "mlp_down": LayerConfig("mlp_down", 4096, 11008, 2048, 64, 2.0, 0.02, outlier_frac=0.001, seed=1),
    "large": LayerConfig("large", 28672, 8192, 8192, 64, 1.0, 0.015),
}


def _streams(seed: int):
    # Independent child streams in a fixed order: W, A, B, X, dY.
    children = np.random.SeedSequence(seed).spawn(5)
    return [np.random.default_rng(c) for c in children]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), via torch's RNE conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_weight(cfg: LayerConfig) -> np.ndarray:
    """W0 as float32 [d_out, d_in], N(0, w_sigma^2), optional outliers x outlier_scale."""
    rng = _streams(cfg.seed)[0]
    w = rng.standard_normal((cfg.d_out, cfg.d_in), dtype=np.float32)
    w *= np.float32(cfg.w_sigma)
    if cfg.outlier_frac > 0:
        k = int(round(cfg.outlier_frac * cfg.n))
        idx = rng.choice(cfg.n, size=k, replace=False)
        flat = w.reshape(-1)
        flat[idx] *= np.float32(cfg.outlier_scale)
    return w


def make_lora(cfg: LayerConfig):
    """A [r, d_in] and B [d_out, r] as bf16 bits, both N(0, ab_sigma^2) (B nonzero)."""
    s = _streams(cfg.seed)
    a = s[1].standard_normal((cfg.r, cfg.d_in), dtype=np.float32) * np.float32(cfg.ab_sigma)
    b = s[2].standard_normal((cfg.d_out, cfg.r), dtype=np.float32) * np.float32(cfg.ab_sigma)
    return to_bf16_bits(a), to_bf16_bits(b)


def make_x(cfg: LayerConfig, d_seq: int | None = None) -> np.ndarray:
    """Activations X as bf16 bits, torch layout [d_seq, d_in] (each token's features contiguous)."""
    d_seq = cfg.d_seq if d_seq is None else d_seq
    x = _streams(cfg.seed)[3].standard_normal((d_seq, cfg.d_in), dtype=np.float32)
    return to_bf16_bits(x)


def make_dy(cfg: LayerConfig, d_seq: int | None = None) -> np.ndarray:
    """Output gradient dY as bf16 bits, torch layout [d_seq, d_out]."""
    d_seq = cfg.d_seq if d_seq is None else d_seq
    dy = _streams(cfg.seed)[4].standard_normal((d_seq, cfg.d_out), dtype=np.float32)
    return to_bf16_bits(dy)


def custom(name: str, d_out: int, d_in: int, d_seq: int, r: int, s: float = 2.0,
           w_sigma: float = 0.02, seed: int = 0, outlier_frac: float = 0.0) -> LayerConfig:
    """An ad-hoc layer (ragged shapes for edge-case tests)."""
    return LayerConfig(name, d_out, d_in, d_seq, r, s, w_sigma, outlier_frac=outlier_frac, seed=seed)
