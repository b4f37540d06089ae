"""The host half of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI layer (csrc/abi.cpp: argument checks, the fp64 frequency step,
workspace arithmetic) and the ring schedule (csrc/ring.cpp) are built with a
plain C++ compiler and -fsanitize=address,undefined, linked with stub kernel
launchers (tests/host/abi_sanitize_driver.cpp) that check the arguments they
receive.  The driver calls every entry point with valid and invalid arguments
and every ring partition and device count; it must return the expected
status everywhere with no sanitizer report.  No GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scaled_rope_tiled_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_and_ring_schedule_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "abi_sanitize_driver.cpp"),
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "ring.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "failures 0" in r.stdout
