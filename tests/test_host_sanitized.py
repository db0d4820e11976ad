"""The host half of libturbokv (argument checks, plane layouts, table
generation) built with g++ under AddressSanitizer and UBSan against stub
kernel launchers, and run on the CPU: every expectation in
tests/host/host_checks.cpp must hold with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_quantization_encode_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="needs g++ and the HIP runtime library to link the host code")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(CSRC, "tables.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(ROOT, "tests", "host", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "host", "host_checks.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failure(s)" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
