"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run on small shapes, both directions, with and
without the optional tensors, and the empty cases, by the C driver in
tests/sanitize/.  Any out-of-bounds access, use after free, leak or
undefined operation fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ROOT, "oracle", "lstm_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # (verify_asan_link_order=0: the run does not insist that the sanitizer
    # runtime be the first library the process maps)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    assert "ok" in r.stdout
