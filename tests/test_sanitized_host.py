"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (gcc and
g++, CPU only): the oracle's C code driven through every layout, rounding,
block size and scale format on exactly sized heap buffers
(tests/sanitize/oracle_driver.c), and the C ABI's validation layer
(csrc/api.cpp, built for the host with the kernel launchers replaced by
checking stubs) driven through valid calls and every class of invalid
argument, including sizes at and past the 2^40 / 2^44 limits
(tests/sanitize/abi_driver.cpp). Any out-of-bounds access, overflow or
other undefined operation aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _build_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    out = _build_run(["gcc", "-std=gnu11", "-ffp-contract=off", "-frounding-math", *SAN,
                      os.path.join(ROOT, "oracle", "fp4q_oracle.c"),
                      os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe], exe)
    assert "oracle driver: ok" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "fp4_block_scaled_fp4q_amd", "csrc")
    out = _build_run(["g++", "-std=c++17", *SAN, "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                      "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "api.cpp"),
                      os.path.join(ROOT, "tests", "sanitize", "kernel_stubs.cpp"),
                      os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe], exe)
    assert "abi driver:" in out and "ok" in out
