"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/oracle_sanitize_driver.c calls every entry point of
oracle/stv_oracle.c on inputs that reach its edge cases (zero rows, empty
key ranges, forests, chains of 64, ragged appends, both cache formats,
commits, merges with empty splits, short and clamped histories) and checks
a few invariants on the way.  Any out-of-bounds access, leak-free misuse or
undefined behaviour aborts the run with the sanitizer's report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_sanitize"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "stv_oracle.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert "invariants hold" in r.stdout
