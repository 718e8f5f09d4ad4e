"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

`oracle_sanitize_driver.c` calls every oracle entry point on small problems
of each dtype combination (with and without router bias and shared expert,
k = E, one token, zero tokens) and the argument errors, with every buffer
its own heap block of the documented size.  Built with gcc's sanitizers and
no recovery, any out-of-bounds access, use after free, leak, signed
overflow or invalid shift ends the run with a report.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", ORACLE,
           os.path.join(ORACLE, "moe_oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("gcc sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr[-4000:]
