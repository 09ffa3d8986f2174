"""Resource use of the built gfx950 kernels, read from the library's own code objects
(the AMDGPU metadata note of each embedded gfx950 ELF): no kernel may use scratch
(private) memory or spill vector registers, which go to scratch (the few scalar
registers a kernel may spill are kept in vector-register lanes, not in memory).
A register array indexed at run time, for example, is silently placed in scratch,
and every access then becomes a round trip to memory: the transposed
dequantisation once moved 32 extra bytes per thread each way that way."""
import glob
import os
import shutil
import subprocess

import pytest
import yaml

from bit_nf4_quantized_05_amd import _lib

LLVM = "/opt/rocm/llvm/bin"
OBJDUMP = os.path.join(LLVM, "llvm-objdump")
READELF = os.path.join(LLVM, "llvm-readelf")

# kernels of every stage of the path (a substring of the mangled name each)
EXPECTED = ["quant_blocks", "dq_encode", "dequant_rows", "prologue_kernel", "prepass_reduce", "gemm_nt_kernel",
            "gemm_nt_split", "gemm_split_reduce", "gemv_nf4_kernel", "lora_ax_partial_kernel", "skinny_nf4",
            "skinny_reduce", "lora_grad_mfma", "lora_grad_reduce", "int8_quant_blocks", "int8_dequant_rows"]


def _kernels(tmp_path):
    if not (os.path.exists(OBJDUMP) and os.path.exists(READELF)):
        pytest.skip("ROCm LLVM tools not found")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    lib = tmp_path / "lib.so"
    shutil.copy(_lib.LIB_PATH, lib)
    # extracts the offload bundles next to the copy
    subprocess.run([OBJDUMP, "--offloading", str(lib)], cwd=tmp_path, check=True, capture_output=True)
    objs = glob.glob(str(tmp_path / "*amdgcn-amd-amdhsa--gfx950"))
    assert objs, "no gfx950 code object in the library"
    out = []
    for o in objs:
        text = subprocess.run([READELF, "--notes", o], check=True, capture_output=True, text=True).stdout
        doc = text[text.index("---"):]
        doc = doc[:doc.index("...")] if "..." in doc else doc
        meta = yaml.safe_load(doc)
        out += meta.get("amdhsa.kernels", [])
    return out


def test_no_scratch_and_no_vgpr_spills(tmp_path):
    ks = _kernels(tmp_path)
    names = [k[".name"] for k in ks]
    for e in EXPECTED:
        assert any(e in n for n in names), f"kernel {e} not found"
    bad = [(k[".name"], k.get(".private_segment_fixed_size"), k.get(".vgpr_spill_count"))
           for k in ks if k.get(".private_segment_fixed_size", 0) or k.get(".vgpr_spill_count", 0)]
    assert not bad, f"kernels with scratch or vector spills (name, scratch bytes, vgpr spills): {bad}"
