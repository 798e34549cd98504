"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc), driven
through every entry point by oracle/sanitize_check.c: no out-of-bounds access, leak or
undefined operation on the ring, CLOCK and resident paths, rollback, rounds on a given
selection and prefetch rounds."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "orc_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-I", ORACLE,
           os.path.join(ORACLE, "dsa_oracle.c"), os.path.join(ORACLE, "sanitize_check.c"), "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ran clean" in run.stdout
