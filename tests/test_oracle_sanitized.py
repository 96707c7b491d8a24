"""The plain-C oracle under gcc's address and undefined-behaviour sanitizers
(host code only): tests/c_oracle/oracle_driver.c calls every oracle entry
point on small ragged inputs (row counts that are not multiples of 64, int4
and int8, groups shorter than, equal to and longer than a superchunk, every
weight and scale type, the zero-point form, row subsets, top-K rescoring and
the embedding rows), with each buffer allocated to its exact length, so a read
or write past any of them, or undefined arithmetic, stops the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_oracle", "oracle_driver.c")
ORACLE = os.path.join(ROOT, "oracle", "lmh_oracle.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_runs_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", DRIVER, ORACLE, "-lm",
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all entry points ran clean" in r.stdout
