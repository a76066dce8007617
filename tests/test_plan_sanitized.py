"""The host-side planning and validation code (csrc/plan.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven over extreme and
random shapes by tests/plan_checks.cpp, whose results are checked against
128-bit arithmetic.  CPU only; g++ builds the host code on its own (no HIP)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_plan_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "plan_checks"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "decode_attention_kv_gqa_amd", "csrc"),
           os.path.join(ROOT, "tests", "plan_checks.cpp"),
           os.path.join(ROOT, "decode_attention_kv_gqa_amd", "csrc", "plan.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout
