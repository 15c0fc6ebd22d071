"""The oracle's C core under gcc's AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/csrc/asan_check.c calls every entry point of the core on small shapes,
edges included (one row, one column, empty, no L_O, a failing factorisation),
and checks that the naive and accumulator sweeps agree code for code. Built
here with gcc alone (host code; nothing in it runs on a GPU).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "oracle", "csrc")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_core_under_sanitizers(tmp_path):
    exe = str(tmp_path / "asan_check")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-o", exe, os.path.join(CSRC, "asan_check.c"),
           os.path.join(CSRC, "bakron_oracle.c"), "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "sanitize" in b.stderr:
        pytest.skip("gcc here has no sanitizer runtime: " + b.stderr.strip()[:200])
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "asan_check ok" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr
