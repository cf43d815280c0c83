"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The C ABI's validation (csrc/gdn_api.cpp): built host-only with g++ and the
  launcher stubs of tests/sanitize/launch_stub.cpp, driven through every entry
  point with valid and invalid arguments by tests/sanitize/api_driver.cpp
  (fake device addresses, never dereferenced). This covers the extent and
  overflow arithmetic of the checks.
* The oracle (oracle/gdn_serial.c): built with gcc and OpenMP and run on
  small shapes that reach every indexing path by tests/sanitize/oracle_driver.c.

UBSan runs with -fno-sanitize-recover, so any report ends the program with a
non-zero status, as does any ASan report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "linear_attention_recurrence_chunked_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_api_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN +
         [os.path.join(CSRC, "gdn_api.cpp"), os.path.join(HERE, "launch_stub.cpp"),
          os.path.join(HERE, "api_driver.cpp"), "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "failures" in r.stdout and "0 failures" in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-fopenmp"] + SAN +
         [os.path.join(ROOT, "oracle", "gdn_serial.c"), os.path.join(HERE, "oracle_driver.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=300)
    assert "0 failures" in r.stdout, r.stdout
