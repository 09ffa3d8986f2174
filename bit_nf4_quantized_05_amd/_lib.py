"""ctypes binding of libqlora_nf4.so (argument marshalling only).

Every function here checks tensor shapes, dtypes and devices, passes raw device
pointers and the current HIP stream to the C ABI declared in include/qlora_nf4.h,
and raises on a non-zero return. No arithmetic on the data happens in Python.
The library must be built (``python -m bit_nf4_quantized_05_amd.build``); a
missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/qlora_nf4.h
SIGNATURES = {
    "qn_version": (_c_int, []),
    "qn_last_error": (ctypes.c_char_p, []),
    "qn_codebook": (_c_int, [_c_vp]),
    "qn_nf4_sizes": (_c_int, [_c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "nf4_quantize_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
    "nf4_quantize": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "nf4_double_dequant": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "qlora_linear_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlora_linear_fwd_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlora_linear_bwd_x_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlora_linear_fwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_int, _c_float,
                                  _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp]),
    "qlora_linear_bwd_x": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_int, _c_float,
                                    _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp]),
    "qlora_lora_grads_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlora_lora_grads": (_c_int, [_c_vp, _c_vp, _c_int, _c_float, _c_vp, _c_i64, _c_vp, _c_i64, _c_i64, _c_i64,
                                  _c_i64, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "qn_nf4_sizes_ex": (_c_int, [_c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp]),
    "nf4_quantize_ex": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "nf4_double_dequant_ex": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp]),
    "qlora_set_fwd_gemm": (_c_int, [_c_int]),
    "qlora_set_ax_wait": (_c_int, [_c_int]),
    "qlora_linear_fwd_ex": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_int,
                                     _c_float, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp]),
    "qlora_linear_fwd_noalloc": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_int,
                                          _c_float, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp]),
    "qlora_linear_bwd_x_ex": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_int,
                                       _c_float, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp]),
    "int8_quantize": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "int8_dequant": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "qlr_linear_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlr_linear_fwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_int, _c_vp, _c_vp, _c_int,
                                _c_vp, _c_vp, _c_int, _c_float, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64,
                                _c_vp]),
    "qn_profile_enable": (_c_int, [_c_int]),
    "qn_profile_read": (_c_int, [_c_vp, _c_int, _c_vp, _c_vp, _c_int]),
    "qn_profile_durations": (_c_int, [ctypes.c_char_p, _c_vp, _c_int]),
}

# second-level formats: the QN_DQ_* codes of the header
DQ_CODES = {"int8": 0, "fp8": 1, "none": 2}

_lib = None


class QLoRAError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QLoRAError(f"{LIB_PATH} is missing: build it with `python -m bit_nf4_quantized_05_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().qn_last_error().decode(errors="replace")
        raise QLoRAError(f"{what} failed with {rc}: {msg}")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _rows(t: torch.Tensor, dtype, shape, name: str, device) -> int:
    """Checks a [rows, cols] activation that may be a view into a wider array: unit
    column stride, any row stride >= cols; returns the row stride (elements)."""
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    rows, cols = shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: the columns must be contiguous")
    ld = t.stride(0) if rows > 1 else cols
    if ld < cols:
        raise ValueError(f"{name}: row stride {ld} is smaller than the row length {cols}")
    return ld


def _need(t: torch.Tensor, dtype, shape, name: str, device) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")


@dataclass
class NF4Weight:
    """An NF4 weight with its block constants as produced by ``quantize``.

    dq names the second level: "int8" (default) or "fp8" (qconst holds E4M3 code
    bytes), both with qscale [n_g] and qmean [1]; or "none", where qscale [n_b]
    holds the float32 block absmax and qconst, qmean are empty."""
    codes: torch.Tensor    # uint8 [n_b * 32]
    qconst: torch.Tensor   # int8 [n_b] (empty for "none")
    qscale: torch.Tensor   # float32 [n_g] ([n_b] for "none")
    qmean: torch.Tensor    # float32 [1] (empty for "none")
    d_out: int
    d_in: int
    dq: str = "int8"

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.qconst, self.qscale, self.qmean))


def version() -> int:
    return lib().qn_version()


def codebook() -> list:
    buf = (ctypes.c_float * 16)()
    _check(lib().qn_codebook(ctypes.addressof(buf)), "qn_codebook")
    return list(buf)


def _dq_code(dq: str) -> int:
    if dq not in DQ_CODES:
        raise ValueError(f"dq must be one of {sorted(DQ_CODES)}, got {dq!r}")
    return DQ_CODES[dq]


def nf4_sizes(d_out: int, d_in: int, dq: str = "int8"):
    """(codes bytes, qconst entries, qscale entries) for format dq."""
    cb, nq, ns = _c_i64(), _c_i64(), _c_i64()
    _check(lib().qn_nf4_sizes_ex(d_out, d_in, _dq_code(dq), ctypes.addressof(cb), ctypes.addressof(nq),
                                 ctypes.addressof(ns)), "qn_nf4_sizes_ex")
    return cb.value, nq.value, ns.value


def quantize_workspace_bytes(d_out: int, d_in: int) -> int:
    return lib().nf4_quantize_workspace_bytes(d_out, d_in)


def linear_workspace_bytes(d_out: int, d_in: int, d_seq: int, r: int) -> int:
    """Bytes enough for both the forward and the input-gradient call."""
    return lib().qlora_linear_workspace_bytes(d_out, d_in, d_seq, r)


def linear_fwd_workspace_bytes(d_out: int, d_in: int, d_seq: int, r: int) -> int:
    return lib().qlora_linear_fwd_workspace_bytes(d_out, d_in, d_seq, r)


def linear_bwd_x_workspace_bytes(d_out: int, d_in: int, d_seq: int, r: int) -> int:
    return lib().qlora_linear_bwd_x_workspace_bytes(d_out, d_in, d_seq, r)


def alloc_weight(d_out: int, d_in: int, device, dq: str = "int8") -> NF4Weight:
    cb, nq, ns = nf4_sizes(d_out, d_in, dq)
    return NF4Weight(torch.empty(cb, dtype=torch.uint8, device=device),
                     torch.empty(nq, dtype=torch.int8, device=device),
                     torch.empty(ns, dtype=torch.float32, device=device),
                     torch.empty(0 if dq == "none" else 1, dtype=torch.float32, device=device), d_out, d_in, dq)


def quantize(W: torch.Tensor, out: NF4Weight | None = None, workspace: torch.Tensor | None = None,
             dq: str = "int8") -> NF4Weight:
    """nf4_quantize_ex on a float32 [d_out, d_in] CUDA tensor, second level dq."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [d_out, d_in]")
    d_out, d_in = W.shape
    _need(W, torch.float32, (d_out, d_in), "W", W.device)
    q = out if out is not None else alloc_weight(d_out, d_in, W.device, dq)
    if q.dq != dq:
        raise ValueError(f"out holds format {q.dq!r}, asked for {dq!r}")
    need = quantize_workspace_bytes(d_out, d_in)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=W.device)
    rc = lib().nf4_quantize_ex(_ptr(W), d_out, d_in, _dq_code(dq), _ptr(q.codes), _ptr(q.qconst), _ptr(q.qscale),
                               _ptr(q.qmean), _ptr(ws), ws.numel() * ws.element_size(), _stream(W.device))
    _check(rc, "nf4_quantize_ex")
    return q


def double_dequant(q: NF4Weight, out: torch.Tensor | None = None) -> torch.Tensor:
    """nf4_double_dequant_ex -> bfloat16 [d_out, d_in]."""
    o = out if out is not None else torch.empty(q.d_out, q.d_in, dtype=torch.bfloat16, device=q.device)
    _need(o, torch.bfloat16, (q.d_out, q.d_in), "out", q.device)
    rc = lib().nf4_double_dequant_ex(_ptr(q.codes), _ptr(q.qconst), _ptr(q.qscale), _ptr(q.qmean), q.d_out, q.d_in,
                                     _dq_code(q.dq), _ptr(o), _stream(q.device))
    _check(rc, "nf4_double_dequant_ex")
    return o


def _linear(fn_name: str, q: NF4Weight, A: torch.Tensor, B: torch.Tensor, s: float, inp: torch.Tensor,
            in_dim: int, out_dim: int, out: torch.Tensor | None, workspace: torch.Tensor | None,
            ws_bytes_fn) -> torch.Tensor:
    dev = q.device
    r = A.shape[0]
    _need(A, torch.bfloat16, (r, q.d_in), "A", dev)
    _need(B, torch.bfloat16, (q.d_out, r), "B", dev)
    if inp.dim() != 2 or inp.shape[1] != in_dim:
        raise ValueError(f"input must be [d_seq, {in_dim}]")
    d_seq = inp.shape[0]
    ld_in = _rows(inp, torch.bfloat16, (d_seq, in_dim), "input", dev)
    o = out if out is not None else torch.empty(d_seq, out_dim, dtype=torch.bfloat16, device=dev)
    ld_out = _rows(o, torch.bfloat16, (d_seq, out_dim), "out", dev)
    need = ws_bytes_fn(q.d_out, q.d_in, d_seq, r)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = getattr(lib(), fn_name)(_ptr(q.codes), _ptr(q.qconst), _ptr(q.qscale), _ptr(q.qmean), q.d_out, q.d_in,
                                 _dq_code(q.dq), _ptr(A), _ptr(B), r, float(s), _ptr(inp), ld_in, d_seq, _ptr(o),
                                 ld_out, _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, fn_name)
    return o


def linear_fwd(q: NF4Weight, A: torch.Tensor, B: torch.Tensor, s: float, X: torch.Tensor,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """qlora_linear_fwd: Y [d_seq, d_out] = X W_hat^T + s (X A^T) B^T. X and out may be
    row views of wider arrays (unit column stride)."""
    return _linear("qlora_linear_fwd_ex", q, A, B, s, X, q.d_in, q.d_out, out, workspace,
                   linear_fwd_workspace_bytes)


# forms of the forward product for more than 64 tokens (qlora_set_fwd_gemm)
FWD_GEMM_AUTO, FWD_GEMM_STAGED, FWD_GEMM_FUSED = 0, 1, 2


def set_fwd_gemm(form: int) -> int:
    """qlora_set_fwd_gemm: process-wide choice of how the forward GEMM meets W_hat (staged in
    the workspace or formed inside the GEMM); returns the previous choice."""
    rc = lib().qlora_set_fwd_gemm(int(form))
    if rc < 0:
        raise ValueError(f"unknown forward GEMM form {form}")
    return rc


def set_ax_wait(polls: int) -> int:
    """qlora_set_ax_wait: polls a persistent one-token GEMV workgroup makes for each
    published A x slice before forming the slices itself; returns the previous value."""
    rc = lib().qlora_set_ax_wait(int(polls))
    if rc < 0:
        raise ValueError(f"polls must be >= 0, got {polls}")
    return rc


def linear_fwd_noalloc(q: NF4Weight, A: torch.Tensor, B: torch.Tensor, s: float, X: torch.Tensor,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """qlora_linear_fwd_noalloc: the forward for 1..64 tokens with no workspace (the library's
    static per-device scratch instead). Calls that overlap on one device race."""
    dev = q.device
    r = A.shape[0]
    _need(A, torch.bfloat16, (r, q.d_in), "A", dev)
    _need(B, torch.bfloat16, (q.d_out, r), "B", dev)
    if X.dim() != 2 or X.shape[1] != q.d_in:
        raise ValueError(f"input must be [d_seq, {q.d_in}]")
    d_seq = X.shape[0]
    ldx = _rows(X, torch.bfloat16, (d_seq, q.d_in), "input", dev)
    o = out if out is not None else torch.empty(d_seq, q.d_out, dtype=torch.bfloat16, device=dev)
    ldy = _rows(o, torch.bfloat16, (d_seq, q.d_out), "out", dev)
    rc = lib().qlora_linear_fwd_noalloc(_ptr(q.codes), _ptr(q.qconst), _ptr(q.qscale), _ptr(q.qmean), q.d_out,
                                        q.d_in, _dq_code(q.dq), _ptr(A), _ptr(B), r, float(s), _ptr(X), ldx, d_seq,
                                        _ptr(o), ldy, _stream(dev))
    _check(rc, "qlora_linear_fwd_noalloc")
    return o


def linear_bwd_x(q: NF4Weight, A: torch.Tensor, B: torch.Tensor, s: float, dY: torch.Tensor,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """qlora_linear_bwd_x: dX [d_seq, d_in] = dY W_hat + s (dY B) A. dY and out may be row
    views of wider arrays."""
    return _linear("qlora_linear_bwd_x_ex", q, A, B, s, dY, q.d_out, q.d_in, out, workspace,
                   linear_bwd_x_workspace_bytes)


def lora_grads_workspace_bytes(d_out: int, d_in: int, d_seq: int, r: int) -> int:
    return lib().qlora_lora_grads_workspace_bytes(d_out, d_in, d_seq, r)


def lora_grads(A: torch.Tensor, B: torch.Tensor, s: float, X: torch.Tensor, dY: torch.Tensor,
               dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None):
    """qlora_lora_grads: (dA [r, d_in], dB [d_out, r]) float32 adapter gradients."""
    dev = A.device
    r, d_in = A.shape
    d_out = B.shape[0]
    _need(A, torch.bfloat16, (r, d_in), "A", dev)
    _need(B, torch.bfloat16, (d_out, r), "B", dev)
    if X.dim() != 2 or dY.dim() != 2 or X.shape[0] != dY.shape[0]:
        raise ValueError("X [d_seq, d_in] and dY [d_seq, d_out] must share d_seq")
    d_seq = X.shape[0]
    ldx = _rows(X, torch.bfloat16, (d_seq, d_in), "X", dev)
    lddy = _rows(dY, torch.bfloat16, (d_seq, d_out), "dY", dev)
    ga = dA if dA is not None else torch.empty(r, d_in, dtype=torch.float32, device=dev)
    gb = dB if dB is not None else torch.empty(d_out, r, dtype=torch.float32, device=dev)
    _need(ga, torch.float32, (r, d_in), "dA", dev)
    _need(gb, torch.float32, (d_out, r), "dB", dev)
    need = lora_grads_workspace_bytes(d_out, d_in, d_seq, r)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib().qlora_lora_grads(_ptr(A), _ptr(B), r, float(s), _ptr(X), ldx, _ptr(dY), lddy, d_out, d_in, d_seq,
                                _ptr(ga), _ptr(gb), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "qlora_lora_grads")
    return ga, gb


def profile_enable(on: bool = True) -> None:
    """Start (clearing old records) or stop per-kernel event timing in the library."""
    _check(lib().qn_profile_enable(1 if on else 0), "qn_profile_enable")


def profile_read(cap: int = 64) -> dict:
    """{kernel name: (launches, total ms)} of the kernels timed since profile_enable."""
    name_len = 96
    names = ctypes.create_string_buffer(name_len * cap)
    launches = (ctypes.c_int64 * cap)()
    total = (ctypes.c_double * cap)()
    n = lib().qn_profile_read(ctypes.addressof(names), name_len, ctypes.addressof(launches),
                              ctypes.addressof(total), cap)
    if n < 0:
        _check(n, "qn_profile_read")
    out = {}
    for i in range(min(n, cap)):
        nm = names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (int(launches[i]), float(total[i]))
    return out


def profile_durations(name: str, cap: int = 4096) -> list:
    """Milliseconds of each launch of kernel `name` timed since profile_enable, in order."""
    buf = (ctypes.c_float * cap)()
    n = lib().qn_profile_durations(name.encode(), ctypes.addressof(buf), cap)
    if n < 0:
        _check(n, "qn_profile_durations")
    return [float(buf[i]) for i in range(min(n, cap))]


# ---- quantised low-rank factors (W ~ Q + L R with L, R at 4 or 8 bits) ----------

@dataclass
class QFactor:
    """A low-rank factor [rows, cols] kept at 4 bits (NF4 codes, float32 a_j per block
    of 64) or 8 bits (absmax INT8 per block of 64, float32 a_j)."""
    bits: int
    codes: torch.Tensor    # uint8 [n_b * 32] (4 bits) or int8 [n_b * 64] (8 bits)
    scale: torch.Tensor    # float32 [n_b]
    rows: int
    cols: int


def int8_quantize(W: torch.Tensor):
    """int8_quantize on a float32 [rows, cols] CUDA tensor -> (q int8 [n_b*64], absmax float32 [n_b])."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    rows, cols = W.shape
    _need(W, torch.float32, (rows, cols), "W", W.device)
    n_b = -(-rows * cols // 64)
    q = torch.empty(n_b * 64, dtype=torch.int8, device=W.device)
    a = torch.empty(n_b, dtype=torch.float32, device=W.device)
    _check(lib().int8_quantize(_ptr(W), rows, cols, _ptr(q), _ptr(a), _stream(W.device)), "int8_quantize")
    return q, a


def int8_dequant(q: torch.Tensor, absmax: torch.Tensor, rows: int, cols: int) -> torch.Tensor:
    """int8_dequant -> bfloat16 [rows, cols]."""
    n_b = -(-rows * cols // 64)
    _need(q, torch.int8, (n_b * 64,), "q", q.device)
    _need(absmax, torch.float32, (n_b,), "absmax", q.device)
    o = torch.empty(rows, cols, dtype=torch.bfloat16, device=q.device)
    _check(lib().int8_dequant(_ptr(q), _ptr(absmax), rows, cols, _ptr(o), _stream(q.device)), "int8_dequant")
    return o


def quantize_factor(M: torch.Tensor, bits: int) -> QFactor:
    """A factor at 4 bits (nf4_quantize_ex without a second level) or 8 bits (int8_quantize)."""
    rows, cols = M.shape
    if bits == 4:
        q = quantize(M, dq="none")
        return QFactor(4, q.codes, q.qscale, rows, cols)
    if bits == 8:
        c, a = int8_quantize(M)
        return QFactor(8, c, a, rows, cols)
    raise ValueError("bits must be 4 or 8")


def dequant_factor(f: QFactor) -> torch.Tensor:
    """bfloat16 [rows, cols] of a quantised factor."""
    if f.bits == 4:
        empty_q = torch.empty(0, dtype=torch.int8, device=f.codes.device)
        empty_m = torch.empty(0, dtype=torch.float32, device=f.codes.device)
        return double_dequant(NF4Weight(f.codes, empty_q, f.scale, empty_m, f.rows, f.cols, "none"))
    return int8_dequant(f.codes, f.scale, f.rows, f.cols)


def qlr_linear_workspace_bytes(d_out: int, d_in: int, d_seq: int, r: int) -> int:
    return lib().qlr_linear_workspace_bytes(d_out, d_in, d_seq, r)


def qlr_linear_fwd(q: NF4Weight, Af: QFactor, Bf: QFactor, s: float, X: torch.Tensor,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """qlr_linear_fwd: Y [d_seq, d_out] = X Q_hat^T + s (X A_hat^T) B_hat^T with A [r, d_in]
    and B [d_out, r] quantised (W ~ Q + L R with B = R^T, A = L^T)."""
    dev = q.device
    r = Af.rows
    if (Af.rows, Af.cols) != (r, q.d_in) or (Bf.rows, Bf.cols) != (q.d_out, r):
        raise ValueError("factor shapes must be A [r, d_in] and B [d_out, r]")
    if X.dim() != 2 or X.shape[1] != q.d_in:
        raise ValueError(f"input must be [d_seq, {q.d_in}]")
    d_seq = X.shape[0]
    ldx = _rows(X, torch.bfloat16, (d_seq, q.d_in), "input", dev)
    o = out if out is not None else torch.empty(d_seq, q.d_out, dtype=torch.bfloat16, device=dev)
    ldy = _rows(o, torch.bfloat16, (d_seq, q.d_out), "out", dev)
    need = qlr_linear_workspace_bytes(q.d_out, q.d_in, d_seq, r)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib().qlr_linear_fwd(_ptr(q.codes), _ptr(q.qconst), _ptr(q.qscale), _ptr(q.qmean), q.d_out, q.d_in,
                              _dq_code(q.dq), Af.bits, _ptr(Af.codes), _ptr(Af.scale), Bf.bits, _ptr(Bf.codes),
                              _ptr(Bf.scale), r, float(s), _ptr(X), ldx, d_seq, _ptr(o), ldy, _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "qlr_linear_fwd")
    return o
