"""Host-side sanitizer builds (CPU only).

The C oracle and the library's host plan arithmetic (workspace layout,
tiling, backward grid sizes) are compiled with the host compiler under
AddressSanitizer and UndefinedBehaviorSanitizer, with every report fatal,
and run on hostile inputs: index rows with negative, out-of-range and
repeated entries, counts outside [0, S], empty and one-token packed
sequences (oracle); sizes at and past the int32 range, S = 1024, G = 1024
(plans).  No GPU code is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_and_run(tmp_path, compiler, std, src, extra, out_name):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / out_name)
    cmd = [compiler, std, *SAN, *extra, os.path.join(NATIVE, src), "-o", exe]
    if compiler == "gcc":
        cmd.append("-lm")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{src} failed:\n{r.stdout}\n{r.stderr}"
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "gcc", "-std=c11", "oracle_check.c", [], "oracle_check")
    assert "oracle sanitizer check: ok" in out


def test_plan_arithmetic_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "block_index_sparse_amd", "csrc")]
    out = _build_and_run(tmp_path, "g++", "-std=c++17", "plan_check.cpp", inc, "plan_check")
    assert ", ok" in out
    fwd_ok, bwd_ok = (int(x) for x in out.split("dims, ")[1].split(" forward and ")[0:1] +
                      out.split(" forward and ")[1].split(" backward")[0:1])
    assert fwd_ok > 1000 and bwd_ok > 100, out
