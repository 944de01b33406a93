"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

tests/oracle_sanitize_driver.c calls every exported oracle function over
ordinary and edge inputs (zero, subnormal, huge, inf/NaN rows, NaN router
logits, every format byte) and prints a checksum of all results.  The
sanitized build must run clean (any report aborts it) and compute exactly
what the plain build computes.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE_C = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
DRIVER_C = os.path.join(HERE, "oracle_sanitize_driver.c")
BASE = ["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-builtin"]
SAN = ["-O1", "-g", "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _build_and_run(tmp_path, name, flags):
    exe = tmp_path / name
    r = subprocess.run(BASE + flags + [ORACLE_C, DRIVER_C, "-o", str(exe), "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("gcc build failed: " + r.stderr[:300])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    return out


def test_oracle_clean_under_asan_ubsan(tmp_path):
    plain = _build_and_run(tmp_path, "plain", ["-O2"])
    assert plain.returncode == 0, plain.stderr[-2000:]
    san = _build_and_run(tmp_path, "sanitized", SAN)
    assert san.returncode == 0, san.stderr[-4000:]
    assert "runtime error" not in san.stderr and "ERROR: AddressSanitizer" not in san.stderr, san.stderr[-4000:]
    assert san.stdout.strip() == plain.stdout.strip()
    assert len(plain.stdout.strip()) == 16
