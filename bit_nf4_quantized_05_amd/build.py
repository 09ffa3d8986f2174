"""Builds libqlora_nf4.so (HIP, gfx950) in-tree with hipcc, and beside it
libqn_calibrate.so, the benchmark's streaming-read calibration kernels
(include/qn_calibrate.h), which are not part of the layer.

    python -m bit_nf4_quantized_05_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqlora_nf4.so")
CALIB_OUT = os.path.join(PKG, "libqn_calibrate.so")
CALIB_SOURCES = ["calibrate.hip"]
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "quantize.hip", "gemm_nt.hip", "gemm_nf4.hip", "prologue.hip", "gemv.hip", "skinny.hip", "lora_grads.hip", "factors.hip",
           "tables.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # bit-exact float32 steps: no contraction, correctly rounded division
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(CALIB_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + CALIB_SOURCES))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], CALIB_OUT)
    if verbose:
        print("built", OUT, "and", CALIB_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
