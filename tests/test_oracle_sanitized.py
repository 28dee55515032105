"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a driver
that runs every oracle entry point over the pins' kinds of input with exactly
sized buffers (tests/oracle_sanitize_driver.c) is built with
-fsanitize=address,undefined (no recovery) and must run clean."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_runs_clean_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "driver")
        cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", DRIVER, "-o", exe, "-lm"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, r.stderr[-4000:]
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
        assert "oracle sanitize driver ok" in r.stdout
