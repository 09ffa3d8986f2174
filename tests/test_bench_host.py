"""Host-side logic of bench.py, on the CPU: the algorithmic byte count of a decode call,
the GEMM launch plan the K-step bound is computed from, the check that a committed
counter summary still matches the sources it was measured with, the one-GPU guard, and
that no function of bench.py rebinds the name of one of its module-level functions."""
import ast
import hashlib
import importlib.util
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _cfg(d_out, d_in, r):
    return types.SimpleNamespace(d_out=d_out, d_in=d_in, r=r)


def test_decode_bytes_of_the_4096_layer(bench):
    # codes 8 388 608 + 8-bit constants 262 144 + group scales 4 096 + mean 4
    # + A and B (bf16, r = 16) 262 144 + x and y (bf16) 16 384
    assert bench.decode_bytes(_cfg(4096, 4096, 16)) == 8933380
    # without a second level: one float32 per 64-weight block instead of the 8-bit code,
    # group scales and mean
    assert bench.decode_bytes(_cfg(4096, 4096, 16), "none") == 8388608 + 4 * 262144 + 262144 + 16384
    # 64 tokens: x and y 64 times
    assert bench.decode_bytes(_cfg(4096, 4096, 16), "int8", 64) == 8933380 + 63 * 16384


def test_gemm_plan_of_the_mlp_pair(bench):
    # 11008 x 4096 at 2048 tokens: 8 x 43 = 344 tiles, one full round of 256 and 88 more
    # split two ways; the busiest CU runs a whole tile (64 + 1 K-steps) and half of one
    p = bench.gemm_plan(2048, 11008, 4096, 64)
    assert (p["tiles"], p["splits"], p["workgroups"], p["critical_steps"]) == (344, 2, 432, 65 + 32 + 1)
    # 4096 x 11008: 128 tiles split two ways, 86 main K-steps each plus the LoRA step
    p = bench.gemm_plan(2048, 4096, 11008, 64)
    assert (p["tiles"], p["splits"], p["workgroups"], p["critical_steps"]) == (128, 2, 256, 86 + 1)
    # 4096 x 4096 at 4096 tokens: exactly one round, no split
    p = bench.gemm_plan(4096, 4096, 4096, 64)
    assert (p["tiles"], p["splits"], p["workgroups"], p["critical_steps"]) == (256, 1, 256, 65)


def test_measured_traffic_follows_the_sources(bench, tmp_path, monkeypatch):
    csrc = tmp_path / "bit_nf4_quantized_05_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_bytes(b"kernel source\n")
    (csrc / "h.h").write_bytes(b"header\n")
    digest = hashlib.sha256(b"kernel source\n" + b"header\n").hexdigest()
    (tmp_path / "profiles" / "p.md").write_text(
        f"summary\n\ntraffic_bytes_per_launch: 123456\nsources_sha256: {digest}\n")
    monkeypatch.setattr(bench, "_ROOT", str(tmp_path))
    assert bench.measured_traffic(("p.md", ("k.hip", "h.h"))) == 123456
    # the same files hashed in another order, an edited source, a missing profile
    assert bench.measured_traffic(("p.md", ("h.h", "k.hip"))) is None
    (csrc / "h.h").write_bytes(b"header, edited\n")
    assert bench.measured_traffic(("p.md", ("k.hip", "h.h"))) is None
    assert bench.measured_traffic(("absent.md", ("k.hip", "h.h"))) is None


def test_committed_profiles_name_existing_sources(bench):
    for profile, files in (bench.GEMM_TRAFFIC, bench.DECODE_TRAFFIC):
        assert os.path.exists(os.path.join(ROOT, "profiles", profile)), profile
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "bit_nf4_quantized_05_amd", "csrc", f)), f


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120,
                         env=dict(os.environ, WORLD_SIZE="1"))
    assert out.returncode == 2
    assert "exactly one GPU" in out.stdout


def test_no_function_rebinds_a_module_function_name():
    """A local assignment to the name of a module-level function hides that function in
    the whole enclosing function (a call before or after the assignment then fails)."""
    tree = ast.parse(open(BENCH).read())
    funcs = {n.name for n in tree.body if isinstance(n, ast.FunctionDef)}
    clashes = []
    for fn in (n for n in tree.body if isinstance(n, ast.FunctionDef)):
        for node in ast.walk(fn):
            targets = []
            if isinstance(node, (ast.Assign, ast.AnnAssign, ast.AugAssign)):
                targets = node.targets if isinstance(node, ast.Assign) else [node.target]
            elif isinstance(node, (ast.For, ast.comprehension)):
                targets = [node.target]
            for t in targets:
                for name in ast.walk(t):
                    if isinstance(name, ast.Name) and isinstance(name.ctx, ast.Store) and name.id in funcs:
                        clashes.append(f"{fn.name}:{node.lineno}:{name.id}")
    assert not clashes, clashes
