"""Host-side window planner of the prefill (kda_plan.h), compiled with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and run on random packed calls:
chunk coverage, empty sequences, window order lists and workspace sizing."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_window_planner(tmp_path):
    exe = tmp_path / "plan_check"
    # a clean environment (a sanitizer runtime preloaded into this process is not for them)
    env = {k: v for k, v in os.environ.items() if k not in ("LD_PRELOAD", "ASAN_OPTIONS", "UBSAN_OPTIONS")}
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(HERE, "host", "plan_check.cpp"),
                    "-o", str(exe)], check=True, env=env)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
