"""The host runtime (validation, the phase-2 split planner, the extern "C"
entry points of csrc/star_host.cpp) built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer, against stub launchers, and driven through
every validation path and thousands of seeded plans (tests/host/
sanitize_driver.cpp). Host code only; no GPU and no HIP."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_runtime_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "sanitize_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "long_context_attention_phase1_amd", "csrc"),
           os.path.join(ROOT, "long_context_attention_phase1_amd", "csrc", "star_host.cpp"),
           os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
