"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
only): every entry point on small problems with exactly-sized buffers, ragged
last mini-batches, b = 1, b > T, T = 0 and odd d (oracle/sanitize_check.c).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fopenmp", "-std=c11", os.path.join(ROOT, "oracle", "sanitize_check.c"),
         os.path.join(ROOT, "oracle", "ttt_oracle.c"), "-lm", "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
