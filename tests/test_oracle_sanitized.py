"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc) and driven by a standalone C program over every exported function on
small, ragged and degenerate shapes (tests/oracle_sanitize_driver.c): no
out-of-bounds access, leak or undefined behaviour, and the driver's invariant
checks hold.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "sol_oracle.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-o", exe, DRIVER, ORACLE_SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "OK", (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
