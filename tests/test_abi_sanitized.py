"""The C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only, on the CPU): tests/c/abi_extremes.c calls every entry point with extreme
and invalid arguments; an out-of-bounds access or a signed overflow anywhere in
argument checking, launch planning, the cache model or the autotuner's checks
ends the run with a report.  About a minute: 40 s of compiling, 30 s of
calls."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))

import build_sanitized  # noqa: E402


@pytest.mark.skipif(not shutil.which("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_abi_extremes_under_sanitizers(tmp_path):
    exe = build_sanitized.build(str(tmp_path / "abi_extremes"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ABI EXTREMES OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
