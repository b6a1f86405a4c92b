"""The oracle's pins, re-run against a build of the oracle with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only): an out-of-bounds access, a use of freed memory,
a signed overflow or a misaligned access anywhere in the oracle's loops aborts that run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_route.py", "test_oracle_layer.py", "test_oracle_layer_backward.py",
        "test_oracle_mx.py", "test_oracle_mx_bwd.py", "test_oracle_bias.py",
        "test_oracle_workload.py"]


def _libasan():
    try:
        out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_ubsan():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(force=True, sanitize=True)
    env = dict(os.environ, MOE_ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m",
           "not gpu"] + [os.path.join(ROOT, "tests", f) for f in PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
