"""Host-only planning code (plan.cpp: layouts, validation, decode work split) built with
AddressSanitizer and UndefinedBehaviorSanitizer and checked against its invariants (CPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_invariants_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "windowed_attention_amd", "csrc"),
           os.path.join(ROOT, "tests", "plan_host_check.cpp"),
           os.path.join(ROOT, "windowed_attention_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
