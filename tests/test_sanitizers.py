"""The oracle and the C ABI's host-side argument checks, built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc/g++, host code only) and
run over their cases on the CPU.

- oracle_driver.c runs qmat_oracle.c's quantizers (every format, on random,
  tied, zero, subnormal-scale and extreme blocks), dequantization, the
  brute-force 4 x 64 products, the KV-cache write and its refused arguments.
- abi_driver.cpp runs qmat_api.cpp, the C ABI, with the launchers replaced by
  stubs that count calls (tests/host_check/launch_stub.cpp) and the few HIP
  runtime names it uses declared by a host-only stand-in header
  (tests/host_check/hip/hip_runtime.h): every rejected call must return its
  status without reaching a launcher, every accepted one must reach them.
Any sanitizer report aborts the driver (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "tests", "host_check")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _have(tool):
    return shutil.which(tool) is not None


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, f"{os.path.basename(exe)} failed:\n{r.stdout}\n{r.stderr}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.skipif(not _have("gcc"), reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drv")
    cmd = ["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fexcess-precision=standard",
           os.path.join(ROOT, "oracle", "qmat_oracle.c"), os.path.join(HC, "oracle_driver.c"),
           "-o", exe, "-lm"]
    assert "all cases ok" in _build_and_run(cmd, exe)


@pytest.mark.skipif(not _have("g++"), reason="g++ not available")
def test_abi_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_drv")
    csrc = os.path.join(ROOT, "block_quantized_weight_qmat_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, f"-I{HC}", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{csrc}", "-x", "c++", os.path.join(csrc, "qmat_api.cpp"),
           os.path.join(HC, "launch_stub.cpp"), os.path.join(HC, "abi_driver.cpp"), "-o", exe]
    assert "all cases ok" in _build_and_run(cmd, exe)
