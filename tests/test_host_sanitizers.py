"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize/ are built with ``-fsanitize=address,undefined`` and run; any
sanitizer report, or a failed check, fails the test:

- ``oracle_driver.c`` with the oracle (oracle/oracle.c) and the input generators
  (synth/synth.c): every expert format through route, align (four block sizes) and the expert
  forward (full I and two slices), the decode tables, and degenerate routings;
- ``abi_driver.cpp`` with the C ABI's host code (the package's csrc/abi.cpp), linked against
  host stand-ins of the four HIP runtime calls it makes and of the kernel launchers
  (``host_stubs.cpp``, which also check the launch arguments): every entry point with valid
  arguments (reaching the launches) and with each class of invalid ones (rejected before any
  launch), on fake device addresses the host code must never dereference.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _build_and_run(cmd, exe, tmp_path):
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in report and "runtime error" not in report, \
        report[-6000:]
    return report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generators_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *FLAGS, "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth.c"),
           os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe]
    assert "oracle driver ok" in _build_and_run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "quantized_moe_expert_topk_amd", "csrc")
    cmd = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "abi.cpp"),
           os.path.join(SAN, "host_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    assert "abi driver ok" in _build_and_run(cmd, exe, tmp_path)
