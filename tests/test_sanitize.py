"""The host pattern code (csrc/pattern.cpp: builder, transpose, orders,
row-split planner, status strings) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by tests/c/pattern_sanitize.c over
many valid and refused inputs (block indices out of bounds are the first
failure the log-linear page's troubleshooting section names).  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "block_sparse_attention_csr_amd", "csrc", "pattern.cpp")
DRIVER = os.path.join(ROOT, "tests", "c", "pattern_sanitize.c")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_pattern_code_under_asan_and_ubsan(tmp_path):
    obj = tmp_path / "pattern.o"
    drv = tmp_path / "driver.o"
    exe = tmp_path / "pattern_sanitize"
    subprocess.run(["g++", "-std=c++17", *SAN, f"-I{INCLUDE}", "-c", SRC, "-o", str(obj)],
                   check=True)
    subprocess.run(["gcc", "-std=c11", *SAN, "-Wall", "-Wextra", f"-I{INCLUDE}", "-c", DRIVER,
                    "-o", str(drv)], check=True)
    subprocess.run(["g++", *SAN, str(obj), str(drv), "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert r.stdout.startswith("ok ") and "runtime error" not in r.stderr, r.stderr[-4000:]
