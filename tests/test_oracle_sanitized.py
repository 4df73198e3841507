"""The oracle built under AddressSanitizer and UndefinedBehaviorSanitizer.

A C driver (tests/oracle_sanitize_driver.c) calls every oracle entry point:
table construction, compress and strict decompress of ragged chunks, all
65 536 patterns, truncated and mutated streams decoded with exactly their own
bytes readable, the slot-layout calls and the reduce-step sums.  Any
out-of-bounds access, use after free, leak or undefined operation (shift
overflow, signed overflow, misaligned load) ends the run with an error.
CPU only; gcc builds it (no GPU code is involved).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["gcc", "-O1", "-g", "-std=c99", "-Wall", "-Wextra", *SAN,
               "-I", os.path.join(ROOT, "oracle"),
               os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
               os.path.join(ROOT, "oracle", "zc_oracle.c"), "-lm", "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        assert b.returncode == 0, b.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
        assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
        assert "sanitized oracle run ok" in r.stdout
