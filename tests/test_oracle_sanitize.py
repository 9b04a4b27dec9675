"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/oracle_sanitize_driver.c calls every oracle entry point on small seeded inputs and
checks invariants that hold for any data (routing weights sum to one, the grouping is a
permutation with exclusive-scan offsets, ties go to the lower expert id, x = 0 gives y = 0,
closed forms of the dequantisation). Built here with gcc and both sanitizers, an
out-of-bounds access, a use of freed memory or undefined arithmetic in the oracle ends the
run with a report and a non-zero status. The oracle's own build (oracle/__init__.py) is not
involved: this test compiles the same C source into a separate executable.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")
ORACLE_C = os.path.join(ROOT, "oracle", "moe_oracle.c")


def _build(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"), "-o", exe, DRIVER, ORACLE_C, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr):
        pytest.skip("gcc here has no sanitizer runtime: " + r.stderr.strip()[-200:])
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_sanitizers(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ)
    # leak checking needs ptrace, which containers often forbid; every other check stays on
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
