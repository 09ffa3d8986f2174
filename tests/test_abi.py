"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching a GPU. Also checks
that the library's independently built NF4 code book has the same float32 bits
as the oracle's (a host-side table query, no device work)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_nf4_quantized_05_amd as qn
from bit_nf4_quantized_05_amd import _lib
from oracle import nf4_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"nf4_quantize", "nf4_double_dequant", "qlora_linear_fwd", "qlora_linear_bwd_x"} <= set(names)
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must mirror the header"


def test_version_and_sizes():
    assert qn.version() >= 100
    assert qn.nf4_sizes(256, 256) == (32768, 1024, 4)
    assert qn.nf4_sizes(3, 50) == (3 * 32, 3, 1)
    assert qn.nf4_sizes(28672, 8192) == (28672 * 8192 // 2, 3670016, 14336)
    assert qn.quantize_workspace_bytes(4096, 4096) >= 262144 * 4
    assert qn.linear_workspace_bytes(4096, 4096, 4096, 16) >= 2 * 4096 * 4096
    # d_seq = 1: the forward streams the codes and needs only its A x partials, but the
    # input gradient still runs the dequantise + GEMM path; the shared query covers both
    assert qn.linear_fwd_workspace_bytes(4096, 4096, 1, 16) <= 64 * 1024
    assert qn.linear_bwd_x_workspace_bytes(4096, 4096, 1, 16) >= 2 * 4096 * 4096
    assert qn.linear_workspace_bytes(4096, 4096, 1, 16) == qn.linear_bwd_x_workspace_bytes(4096, 4096, 1, 16)
    # small batch (2..64 tokens): the forward keeps fp32 K-split partials, no W_hat
    assert qn.linear_fwd_workspace_bytes(28672, 8192, 64, 64) < 2 * 28672 * 8192 // 4
    assert qn.linear_fwd_workspace_bytes(4096, 4096, 16, 16) >= 4 * 8 * 16 * 4096
    # above 64 tokens both calls dequantise W into the workspace
    assert qn.linear_fwd_workspace_bytes(4096, 4096, 65, 16) >= 2 * 4096 * 4096
    # few output tiles: the GEMM splits K and keeps fp32 partials in the workspace
    # (2 tiles of the 200 x 512 forward -> 4 splits; a small K -> no split)
    base = qn.linear_fwd_workspace_bytes(512, 4096, 200, 16)
    assert base >= 2 * 512 * 4096 + 4 * 200 * 512 * 4
    assert qn.linear_workspace_bytes(320, 192, 300, 100) < 2 * 320 * 192 + 4 * 300 * 320 * 4 + (1 << 20)
    assert qn.quantize_workspace_bytes(0, 5) == 0
    assert qn.linear_workspace_bytes(64, 64, 1, 0) == 0
    assert qn.linear_fwd_workspace_bytes(64, 64, 0, 8) == 0
    for d_seq in (1, 2, 3, 16, 64, 65, 4096):
        both = qn.linear_workspace_bytes(1024, 2048, d_seq, 16)
        assert both == max(qn.linear_fwd_workspace_bytes(1024, 2048, d_seq, 16),
                           qn.linear_bwd_x_workspace_bytes(1024, 2048, d_seq, 16))


def test_library_code_book_bits_equal_oracle():
    lib_cb = np.array(qn.codebook(), dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), O.codebook().view(np.uint32))


FAKE = 1 << 20  # an aligned, never-dereferenced address: every call below fails validation first


def test_argument_validation_without_device_work():
    lib = _lib.lib()
    # null pointers -> -1
    assert lib.nf4_quantize(None, 4, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert b"null" in lib.qn_last_error()
    # non-positive sizes -> -1
    assert lib.nf4_quantize(FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    # misaligned weight pointer -> -1
    assert lib.nf4_quantize(FAKE + 4, 4, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    # workspace too small -> -3
    assert lib.nf4_quantize(FAKE, 4, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == -3
    # linear: codes, qconst, qscale, qmean, d_out, d_in, A, B, r, s, X, ldx, d_seq, Y, ldy, ws, ws_bytes, stream
    def lin(**kw):
        a = dict(d_out=64, d_in=64, r=8, ldx=64, d_seq=16, Y=FAKE, ldy=64, ws=1 << 30)
        a.update(kw)
        return [FAKE, FAKE, FAKE, FAKE, a["d_out"], a["d_in"], FAKE, FAKE, a["r"], 2.0, FAKE, a["ldx"], a["d_seq"],
                a["Y"], a["ldy"], FAKE, a["ws"], None]
    # d_in not a multiple of 64 -> -2
    assert lib.qlora_linear_fwd(*lin(d_in=96, ldx=96)) == -2
    assert lib.qlora_linear_bwd_x(*lin(d_in=96, ldy=96)) == -2
    # r out of range -> -1
    assert lib.qlora_linear_fwd(*lin(r=0)) == -1
    assert lib.qlora_linear_fwd(*lin(r=257)) == -1
    # workspace too small -> -3
    assert lib.qlora_linear_fwd(*lin(ws=16)) == -3
    assert lib.qlora_linear_bwd_x(*lin(ws=16)) == -3
    # null output -> -1
    assert lib.qlora_linear_fwd(*lin(Y=None)) == -1
    # leading dimensions: smaller than the row, or not a multiple of 8 -> -1; wider is fine
    assert lib.qlora_linear_fwd(*lin(ldx=56)) == -1
    assert b"leading dimension" in lib.qn_last_error()
    assert lib.qlora_linear_fwd(*lin(ldy=60)) == -1
    assert lib.qlora_linear_fwd(*lin(ldx=68)) == -1
    assert lib.qlora_linear_bwd_x(*lin(d_out=128, ldx=64)) == -1     # dY rows are d_out long
    assert lib.qlora_linear_bwd_x(*lin(d_in=128, ldy=64)) == -1      # dX rows are d_in long
    assert lib.qlora_linear_fwd(*lin(ldx=72, ldy=8192, ws=16)) == -3    # passes the ld checks
    # an operand reaching 4 GiB through its leading dimension -> -2
    assert lib.qlora_linear_fwd(*lin(d_seq=1 << 16, ldx=1 << 16)) == -2
    assert lib.nf4_double_dequant(FAKE, FAKE, FAKE, FAKE, 64, 64, None, None) == -1
    # adapter gradients: A, B, r, s, X, ldx, dY, lddy, d_out, d_in, d_seq, dA, dB, ws, ws_bytes, stream
    g = [FAKE, FAKE, 8, 2.0, FAKE, 64, FAKE, 64, 64, 64, 16, FAKE, FAKE, FAKE, 1 << 30, None]
    g[0] = None
    assert lib.qlora_lora_grads(*g) == -1                      # null pointer
    g[0] = FAKE
    g[9], g[5] = 96, 96
    assert lib.qlora_lora_grads(*g) == -2                      # d_in % 64 != 0
    g[9], g[5] = 64, 64
    g[2] = 0
    assert lib.qlora_lora_grads(*g) == -1                      # r < 1
    g[2] = 8
    g[11] = FAKE + 8
    assert lib.qlora_lora_grads(*g) == -1                      # misaligned dA
    g[11] = FAKE
    g[5] = 32
    assert lib.qlora_lora_grads(*g) == -1                      # ldx < d_in
    g[5] = 64
    g[7] = 68
    assert lib.qlora_lora_grads(*g) == -1                      # lddy not a multiple of 8
    g[7] = 64
    g[14] = 16
    assert lib.qlora_lora_grads(*g) == -3                      # workspace too small
    assert lib.qlora_lora_grads_workspace_bytes(64, 64, 16, 0) == 0
    assert lib.qlora_lora_grads_workspace_bytes(4096, 4096, 4096, 16) >= 2 * 2 * 4096 * 64


def test_second_level_formats_sizes_and_validation():
    assert qn.nf4_sizes(256, 256, "fp8") == (32768, 1024, 4)
    assert qn.nf4_sizes(256, 256, "none") == (32768, 0, 1024)     # a_j per block, no qconst
    assert qn.nf4_sizes(3, 50, "none") == (3 * 32, 0, 3)
    with pytest.raises(ValueError):
        qn.nf4_sizes(256, 256, "fp4")
    lib = _lib.lib()
    cb = ctypes.c_int64()
    assert lib.qn_nf4_sizes_ex(256, 256, 3, ctypes.addressof(cb), None, None) == -1
    # unknown format -> -1 on every entry point
    assert lib.nf4_quantize_ex(FAKE, 4, 64, 7, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.nf4_double_dequant_ex(FAKE, FAKE, FAKE, FAKE, 4, 64, -1, FAKE, None) == -1
    assert lib.qlora_linear_fwd_ex(FAKE, FAKE, FAKE, FAKE, 64, 64, 3, FAKE, FAKE, 8, 1.0, FAKE, 64, 4, FAKE, 64,
                                   FAKE, 1 << 30, None) == -1
    assert lib.qlora_linear_bwd_x_ex(FAKE, FAKE, FAKE, FAKE, 64, 64, 3, FAKE, FAKE, 8, 1.0, FAKE, 64, 4, FAKE, 64,
                                     FAKE, 1 << 30, None) == -1
    # the 8-bit formats need qconst and qmean; "none" does not (a too-small workspace
    # is the first thing it reports)
    for dq in (0, 1):
        assert lib.nf4_quantize_ex(FAKE, 4, 64, dq, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == -1
        assert lib.nf4_quantize_ex(FAKE, 4, 64, dq, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert lib.nf4_quantize_ex(FAKE, 4, 64, 2, FAKE, None, FAKE, None, FAKE, 1, None) == -3
    assert lib.nf4_quantize_ex(FAKE, 4, 64, 2, FAKE, None, None, None, FAKE, 1 << 20, None) == -1   # qscale needed
    assert lib.qlora_linear_fwd_ex(FAKE, None, FAKE, None, 64, 64, 2, FAKE, FAKE, 8, 1.0, FAKE, 64, 4, FAKE, 64,
                                   FAKE, 1, None) == -3
    assert lib.qlora_linear_fwd_ex(FAKE, None, FAKE, FAKE, 64, 64, 1, FAKE, FAKE, 8, 1.0, FAKE, 64, 4, FAKE, 64,
                                   FAKE, 1 << 30, None) == -1


def test_factor_entry_points_validation():
    lib = _lib.lib()
    assert lib.int8_quantize(None, 4, 64, FAKE, FAKE, None) == -1
    assert lib.int8_quantize(FAKE, 0, 64, FAKE, FAKE, None) == -1
    assert lib.int8_quantize(FAKE + 4, 4, 64, FAKE, FAKE, None) == -1          # misaligned W
    assert lib.int8_dequant(FAKE, None, 4, 64, FAKE, None) == -1
    assert lib.qlr_linear_workspace_bytes(64, 64, 4, 8) >= lib.qlora_linear_fwd_workspace_bytes(64, 64, 4, 8) + \
        2 * 8 * 64 * 2
    assert lib.qlr_linear_workspace_bytes(64, 64, 4, 0) == 0
    args = [FAKE, FAKE, FAKE, FAKE, 64, 64, 0]
    tail = [8, 1.0, FAKE, 64, 4, FAKE, 64, FAKE, 1 << 30, None]
    assert lib.qlr_linear_fwd(*args, 3, FAKE, FAKE, 4, FAKE, FAKE, *tail) == -1       # bits
    assert lib.qlr_linear_fwd(*args, 4, FAKE, FAKE, 16, FAKE, FAKE, *tail) == -1      # bits
    assert lib.qlr_linear_fwd(*args, 4, None, FAKE, 8, FAKE, FAKE, *tail) == -1       # null factor
    small = [8, 1.0, FAKE, 64, 4, FAKE, 64, FAKE, 1024, None]
    assert lib.qlr_linear_fwd(*args, 4, FAKE, FAKE, 8, FAKE, FAKE, *small) == -3      # workspace
    bad_shape = [FAKE, FAKE, FAKE, FAKE, 64, 96, 0]
    tail96 = [8, 1.0, FAKE, 96, 4, FAKE, 64, FAKE, 1 << 30, None]
    assert lib.qlr_linear_fwd(*bad_shape, 8, FAKE, FAKE, 8, FAKE, FAKE, *tail96) == -2
    assert lib.qlr_linear_fwd(*args, 8, FAKE, FAKE, 8, FAKE, FAKE, 8, 1.0, FAKE, 64, 4, FAKE, 32, FAKE, 1 << 30,
                              None) == -1                                          # ldy < d_out


def test_codebook_null_pointer():
    assert _lib.lib().qn_codebook(None) == -1


def test_profile_durations_validation():
    """Per-launch kernel timing: bad arguments are rejected and a kernel that was never
    recorded has no launches (no device work)."""
    lib = _lib.lib()
    # enabling creates the reusable events, which needs a device: 0 with one, -4 without
    assert lib.qn_profile_enable(1) in (0, -4)
    try:
        assert lib.qn_profile_durations(None, None, 0) == -1
        assert lib.qn_profile_durations(b"gemm_nt_kernel", None, 4) == -1
        assert lib.qn_profile_durations(b"gemm_nt_kernel", None, -1) == -1
        buf = (ctypes.c_float * 4)()
        assert lib.qn_profile_durations(b"gemm_nt_kernel", ctypes.addressof(buf), 4) == 0
        assert qn.profile_durations("never_launched") == []
    finally:
        assert lib.qn_profile_enable(0) == 0


def test_ax_wait_setter():
    """qlora_set_ax_wait returns the previous poll limit and rejects negative values."""
    prev = qn.set_ax_wait(7)
    try:
        assert prev >= 0
        assert qn.set_ax_wait(0) == 7
        assert _lib.lib().qlora_set_ax_wait(-1) == -1
        assert qn.set_ax_wait(prev) == 0
    finally:
        qn.set_ax_wait(prev)


def test_forward_form_switch():
    """qlora_set_fwd_gemm returns the previous form and rejects unknown values."""
    prev = qn.set_fwd_gemm(qn.FWD_GEMM_STAGED)
    try:
        assert prev in (qn.FWD_GEMM_AUTO, qn.FWD_GEMM_STAGED, qn.FWD_GEMM_FUSED)
        assert qn.set_fwd_gemm(qn.FWD_GEMM_FUSED) == qn.FWD_GEMM_STAGED
        assert qn.set_fwd_gemm(qn.FWD_GEMM_AUTO) == qn.FWD_GEMM_FUSED
        assert _lib.lib().qlora_set_fwd_gemm(3) == -1
        assert _lib.lib().qlora_set_fwd_gemm(-1) == -1
        assert qn.set_fwd_gemm(qn.FWD_GEMM_AUTO) == qn.FWD_GEMM_AUTO
    finally:
        qn.set_fwd_gemm(prev)


def test_missing_library_is_an_error(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(_lib.QLoRAError):
        _lib.lib()
    monkeypatch.undo()
    assert isinstance(_lib.lib(), ctypes.CDLL)


def test_calibration_library_exports_and_validation():
    """libqn_calibrate.so (the benchmark's streaming-read floor, include/qn_calibrate.h)
    exports what its header declares and rejects bad arguments before any device work."""
    path = os.path.join(ROOT, "bit_nf4_quantized_05_amd", "libqn_calibrate.so")
    cal = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qn_calibrate.h")).read(), flags=re.S)
    names = set(re.findall(r"^\s*int\s+([a-z][a-z0-9_]*)\s*\(", text, flags=re.M))
    assert names == {"qn_calibrate_code_stream", "qn_calibrate_read"}
    for n in names:
        assert hasattr(cal, n)
    f = cal.qn_calibrate_code_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 2
    assert f(None, FAKE, FAKE, 64, 64, FAKE, None) == -1
    assert f(FAKE, FAKE, FAKE, 64, 96, FAKE, None) == -1          # d_in % 64 != 0
    assert f(FAKE + 8, FAKE, FAKE, 64, 64, FAKE, None) == -1      # misaligned codes
    g = cal.qn_calibrate_read
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert g(FAKE, 24, 1, FAKE, None) == -1                       # not a multiple of 16
    assert g(FAKE, 4096, 0, FAKE, None) == -1                     # no workgroups
    assert g(None, 4096, 4, FAKE, None) == -1
