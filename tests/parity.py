"""Helpers shared by the GPU parity tests: device transfer, oracle pieces for
sampled checks at full size, and the floating-point tolerance of the products.

Tolerance of the GEMM outputs (bf16 in, fp32 accumulation, bf16 out) against
the float64 oracle on the same dequantised weights:
    max |Y - Y_ref| / max |Y_ref| <= 1e-2   and   ||Y - Y_ref||_F / ||Y_ref||_F <= 4e-3.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import nf4_oracle as O

MAX_REL = 1e-2
FRO_REL = 4e-3


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda", 0)


def to_gpu_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev())


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())
    return t.view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_f32(bf16_bits(t)).astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(got - ref)
    scale = np.max(np.abs(ref))
    max_rel = float(np.max(err) / scale) if scale > 0 else float(np.max(err))
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_rel <= MAX_REL and fro <= FRO_REL, f"{what}: max_rel={max_rel:.3e} fro={fro:.3e}"
    return max_rel, fro


class OracleLayer:
    """Oracle quantisation of W computed in pieces: all block constants, the mean
    and the second level in full (cheap), codes only for requested blocks."""

    def __init__(self, w: np.ndarray):
        self.d_out, self.d_in = w.shape
        self.blocks = O.to_blocks(w)
        self.absmax = O.block_absmax(self.blocks)
        self.mu = O.exact_mean_f32(self.absmax)
        self.qconst, self.qscale = O.dq_encode(self.absmax, self.mu)
        self.ahat = O.dq_decode(self.qconst, self.qscale, self.mu)

    def codes_of(self, blk: np.ndarray) -> np.ndarray:
        """Unpacked codes [len(blk), 64] of the given block indices."""
        return O.block_codes(self.blocks[blk], self.absmax[blk])

    def rows(self, rows: np.ndarray) -> np.ndarray:
        """W_hat rows as bf16 bits [len(rows), d_in] (d_in % 64 == 0)."""
        per = self.d_in // 64
        blk = (np.asarray(rows)[:, None] * per + np.arange(per)[None, :]).reshape(-1)
        vals = O.codebook()[self.codes_of(blk)]
        w = (vals * self.ahat[blk][:, None]).astype(np.float32)
        return O.f32_to_bf16_bits(w).reshape(len(rows), self.d_in)

    def col_blocks(self, cblocks: np.ndarray) -> np.ndarray:
        """W_hat columns of the given 64-wide column blocks, bf16 bits [d_out, 64*len]."""
        per = self.d_in // 64
        out = np.empty((self.d_out, 64 * len(cblocks)), np.uint16)
        for k, cb in enumerate(cblocks):
            blk = np.arange(self.d_out) * per + cb
            vals = O.codebook()[self.codes_of(blk)]
            w = (vals * self.ahat[blk][:, None]).astype(np.float32)
            out[:, 64 * k:64 * (k + 1)] = O.f32_to_bf16_bits(w)
        return out
