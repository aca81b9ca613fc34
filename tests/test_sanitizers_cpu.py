"""The host code under the address and undefined-behaviour sanitizers (CPU
only, no GPU, no HIP runtime).

1. The host half of the C ABI (csrc/kda_host.cpp: validation, state_at,
   pool sizing, launch description, the block-to-tile map, error strings)
   compiled with plain g++ and -fsanitize=address,undefined into the test
   driver tests/host_abi_check.cpp, which runs the refusals of ROCm/ATOM
   PR #2945 (Changes and Testing) and random slot tables checked against the
   documented rules.  Any sanitizer report is fatal.
2. The oracle's pins (tests/test_oracle_pins.py, test_conv_oracle.py,
   test_prefill_oracle.py) run in a child Python process against a build of
   oracle/kda_oracle.c with the same sanitizers, their runtimes preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kda_gated_delta_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip("%s not available" % tool)


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("%s not found" % name)
    return path


def test_host_half_under_asan_ubsan(tmp_path):
    _need("g++")
    exe = tmp_path / "host_abi_check"
    cmd = ["g++", "-std=c++17", "-O1", *SAN, "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_abi_check.cpp"), os.path.join(CSRC, "kda_host.cpp"),
           "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                                UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.slow
def test_oracle_pins_under_asan_ubsan(tmp_path):
    _need("gcc")
    from oracle import build as oracle_build
    lib = oracle_build.build(out=str(tmp_path / "libkda_oracle_san.so"), sanitize=True)
    preload = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env = dict(os.environ, KDA_ORACLE_LIB=lib, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               PYTHONDONTWRITEBYTECODE="1")
    pins = [os.path.join(ROOT, "tests", f) for f in
            ("test_oracle_pins.py", "test_conv_oracle.py", "test_prefill_oracle.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *pins], capture_output=True, text=True, cwd=ROOT,
                       env=env, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
