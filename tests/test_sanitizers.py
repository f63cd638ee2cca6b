"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (plain C) is built with gcc and run by tests/sanitize/oracle_driver.c
  over every function, edge cases and refused arguments included.
* The library's C ABI is built from its sources with hipcc, the sanitizers on
  the host side only (the GPU code is compiled as usual and never launched),
  and run by tests/sanitize/abi_driver.cpp over the argument checks of every
  entry point that can be reached without a GPU.

Any sanitizer report aborts the driver (no recovery), so a zero exit status
and the driver's closing line are the whole check.  The two builds share
nothing: the oracle driver links only the oracle, the ABI driver only the
library sources.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "w8a8_rotated_int8_convrot_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    rc, out = run(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-o", exe,
                   os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "convrot_oracle.c"), "-lm"])
    assert rc == 0, out
    rc, out = run([exe], env=ENV, timeout=120)
    assert rc == 0 and "calls passed" in out, out


def test_abi_argument_paths_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_driver")
    srcs = [os.path.join(CSRC, s) for s in ("convrot_api.hip", "rotate_quant.hip", "gemm_i8.hip",
                                             "default_path.hip", "mfma_probe.hip")]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
           "-fhip-fp32-correctly-rounded-divide-sqrt",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-disable-promote-alloca-to-lds",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-o", exe, os.path.join(SAN, "abi_driver.cpp"), *srcs]
    rc, out = run(cmd, timeout=600)
    assert rc == 0, out
    rc, out = run([exe], env=ENV, timeout=120)
    assert rc == 0 and "checks passed" in out, out
