"""The C ABI layer (argument validation, derived launch sizes) built for the
host alone with g++ under AddressSanitizer and UndefinedBehaviorSanitizer,
the kernel launchers replaced by recording stubs (tests/abi_host), and
driven through every entry point with valid and invalid arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host")
    srcs = [os.path.join(ROOT, "mixed_precision_tiled_amd", "csrc", "lamp_api.cpp"),
            os.path.join(ROOT, "tests", "abi_host", "stubs.cpp"),
            os.path.join(ROOT, "tests", "abi_host", "driver.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, *srcs, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    # (verify_asan_link_order=0: the process environment may preload other
    # libraries ahead of the sanitizer runtime)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failed" in out and "runtime error" not in out and "ERROR: AddressSanitizer" not in out
