"""The host-side metadata producer under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sched_stress.cpp drives csrc/sched.cpp through its C ABI with randomised request
streams (both cache policies, page sizes 1/4/16, small and large pools) and checks every
batch against the batch contract. Here it is built with g++ and both sanitizers (host
code only; the scheduler has no device code) and run: any out-of-bounds access, use
after free, leak or undefined behaviour aborts it with a report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_scheduler_stress_under_sanitizers(tmp_path):
    exe = tmp_path / "sched_stress"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "sched_stress.cpp"),
           os.path.join(ROOT, "paged_kv_attention_25_amd", "csrc", "sched.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-6000:])
    assert "SCHED_STRESS_OK" in run.stdout
