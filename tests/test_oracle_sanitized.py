"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host only): oracle/sanitize_driver.c calls every exported oracle function
on small and degenerate shapes and on argument errors; built together with
oracle/mdn_oracle.c by gcc with -fsanitize=address,undefined and run as a
process of its own, it must exit cleanly.  No GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_runs_clean_under_address_and_undefined_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "mdn_oracle.c"),
           os.path.join(ROOT, "oracle", "sanitize_driver.c"), "-o", exe, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower():
        pytest.skip("the sanitizer runtime is not installed: " + res.stderr[-300:])
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert run.stdout.strip() == "ok"
