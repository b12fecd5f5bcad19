"""The library's host side under AddressSanitizer and UndefinedBehaviorSanitizer.

A host-only build of every source (no device code, so no GPU is needed) is
linked with tests/host_checks.c, which drives each entry point's argument
checks, size queries and host-array validation: every mask family's
descriptor with its host arrays read in full, malformed descriptors, and
sizes past the library's limits, which must be refused rather than wrap.  A
sanitizer report aborts the driver, and the test fails on it.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "mask_aware_block_amd"))
import build as B  # noqa: E402

pytestmark = pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(B.CLANGXX)),
                                reason="hipcc / clang++ not available")


def test_host_side_under_asan_and_ubsan(tmp_path):
    lib = B.build_host_sanitized(str(tmp_path))
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([B.CLANGXX, "-x", "c", "-std=c11", "-g", "-O1", "-Wall", "-Werror",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_checks.c"),
                        "-x", "none", lib, f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "0 failed" in r.stdout, r.stdout
