"""The C ABI's host code (argument validation, dispatch, quantise / pack /
unpack) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every entry point.  The device launchers are replaced by
host stand-ins (tests/sanitize/stub_launchers.cpp), so no GPU is involved;
any sanitizer report aborts the driver and fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_code_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.fail("g++ is required for the sanitizer build")
    exe = tmp_path / "abi_driver"
    srcs = [os.path.join(ROOT, p) for p in ("tests/sanitize/abi_driver.cpp", "tests/sanitize/stub_launchers.cpp",
                                            "w4a16_int4_weight_linear_amd/csrc/api.cpp",
                                            "w4a16_int4_weight_linear_amd/csrc/host_pack.cpp")]
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *srcs,
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "sanitize driver: ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
