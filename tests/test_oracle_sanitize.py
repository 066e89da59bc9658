"""The C oracle and a host build of the library's block coder, run under
AddressSanitizer and UndefinedBehaviorSanitizer over random, special-value
and corrupted inputs with exactly sized buffers (out-of-bounds reads or
writes, negative or oversized shifts and signed overflow abort the test
program).
Host code only: the GPU kernels are not built with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd_build, exe, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
                                UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert "done" in r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-ffp-contract=off", "-fno-fast-math", os.path.join(ROOT, "oracle", "oracle_codec.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe], exe, tmp_path)


def test_library_block_coder_host_build_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "block_driver")
    _run([hipcc, "--cuda-host-only", "-O1", "-g", "-std=c++17",
          "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
          os.path.join(HERE, "block_driver.hip"), "-o", exe], exe, tmp_path)
