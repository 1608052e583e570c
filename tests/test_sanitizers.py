"""The CPU oracle and the C-ABI host layer under AddressSanitizer and
UndefinedBehaviorSanitizer.

Each is built with gcc / g++ and `-fsanitize=address,undefined
-fno-sanitize-recover=all` into a standalone driver (tests/sanitize/) that
calls every entry point on small and invalid inputs.  A sanitizer report, a
failed check or a non-zero exit fails the test.  The host layer is built
host-only, its kernel launchers replaced by stubs, so no GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _build_and_run(tmp_path, cmd, exe):
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and ("asan" in r.stderr.lower() or "cannot find" in r.stderr):
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _build_and_run(tmp_path, ["gcc", "-std=c11", *FLAGS, os.path.join(HERE, "oracle_driver.c"),
                                    os.path.join(ROOT, "oracle", "gspn_oracle.c"), "-lm"], exe)
    assert "oracle driver: ok" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    csrc = os.path.join(ROOT, "spatial_line_scan_amd", "csrc")
    out = _build_and_run(tmp_path, ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__",
                                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                                    "-I", csrc, os.path.join(HERE, "host_driver.cpp"),
                                    os.path.join(csrc, "gspn_host.cpp")], exe)
    assert "host driver: ok" in out
