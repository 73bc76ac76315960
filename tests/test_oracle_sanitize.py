"""The C++ oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/oracle_sanitize_main.cpp drives oracle/onebit_ref.cpp on ragged sizes,
worker counts 1 to 9, special and extreme values, with buffers of exactly
their stated sizes; built with g++ and the sanitizers (host code only, no GPU
code involved), it must run clean and print "ok".
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_main.cpp")
ORACLE = os.path.join(ROOT, "oracle", "onebit_ref.cpp")


def test_cpp_oracle_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "oracle_sanitize")
    build = subprocess.run([cxx, "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
                            "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            "-static-libasan", "-static-libubsan",
                            "-o", exe, DRIVER, ORACLE], capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("the sanitizer runtime is not installed")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip().endswith("ok"), run.stdout
