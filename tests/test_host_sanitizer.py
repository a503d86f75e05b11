"""The C ABI's host side (csrc/api.cpp: argument validation, workspace
layout, dispatch) built with AddressSanitizer and UndefinedBehaviorSanitizer
by the host compiler, against stand-ins for the device launchers, and driven
through every entry point's accepting and rejecting paths
(tests/host_sanitizer/). Needs g++ and the ROCm headers; no GPU."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC), reason="needs g++ and ROCm headers")
def test_abi_host_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "head_latent_attention_rmsnorm_amd", "csrc", "api.cpp"),
           os.path.join(HERE, "host_sanitizer", "stubs.cpp"), os.path.join(HERE, "host_sanitizer", "driver.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout
