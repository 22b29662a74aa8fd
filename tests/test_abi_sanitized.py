"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: every entry
point's validation paths (bad pointers, shapes, ranges, dtypes, segment tables, graph arguments)
driven from C, without a GPU.  Device code is built as usual and never launched."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_host_validation_under_sanitizers(tmp_path):
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    out = str(tmp_path / "asan")
    b = subprocess.run(["bash", os.path.join(HERE, "sanitize", "build.sh"), out], capture_output=True, text=True,
                       timeout=900)
    assert b.returncode == 0, b.stdout + b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([os.path.join(out, "abi_checks")], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    shutil.rmtree(out, ignore_errors=True)
