"""The oracle's CPU pins run again against an AddressSanitizer +
UndefinedBehaviorSanitizer build of oracle/kv4_oracle.c (gcc, host code
only), in a child process with libasan preloaded: any out-of-bounds access,
use of freed memory, signed overflow, misaligned access or other undefined
behaviour in the oracle aborts the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_scalars.py", "tests/test_oracle_ties.py", "tests/test_oracle_cache.py",
        "tests/test_oracle_decode.py", "tests/test_oracle_budget.py", "tests/test_oracle_prefill_attn.py",
        "tests/test_oracle_kv8.py", "tests/test_oracle_mx.py"]


def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    from oracle import build
    lib = build.build(sanitize=True, out=str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ, LD_PRELOAD=asan, KV4_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        "-p", "no:xdist", *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
