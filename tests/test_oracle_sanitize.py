"""The CPU oracle built under AddressSanitizer and UndefinedBehaviorSanitizer
(gcc), driven through every exported function on inputs that reach its edge
paths: lengths outside [0, N] and [0, pitch], empty rows, FP8 scoring of zero
and non-finite query rows, out-of-range key indices, e4m3fn specials."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-pthread",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_sanitize_main.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer run ok" in r.stdout
