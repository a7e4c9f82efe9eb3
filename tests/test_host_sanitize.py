"""The C ABI's host layer (argument validation and launch-descriptor
marshalling in attn_api.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, and driven through every validation path by
tests/helpers/abi_host_check.cpp. The kernel launchers are stubs there, so this
runs on the CPU only; any sanitizer report or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "exact_tiled_attention_20_amd", "csrc", "attn_api.cpp")
DRIVER = os.path.join(ROOT, "tests", "helpers", "abi_host_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", API, DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # The environment is passed on unchanged apart from the sanitizer options;
    # a library preloaded by the environment may precede the ASan runtime, so
    # the link-order check is relaxed rather than the preload touched.
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi host checks OK" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
