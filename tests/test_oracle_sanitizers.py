"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Compiles oracle/oracle.c with tests/oracle_sanitize_driver.c using gcc with
-fsanitize=address,undefined (no recovery) and runs every oracle entry point on
small ragged inputs.  A sanitizer report makes the program exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-O1", "-g", "-fopenmp", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("this gcc has no sanitizer runtime: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the sanitizer runtime need not be the first library
    # loaded (an environment may preload others)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok "), run.stdout
