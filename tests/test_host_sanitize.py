"""The library's host code (plans, layouts, argument checks, the per-plan
constant tables, the host big-integer stage) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

    g++ -std=c++17 -O1 -g -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include
        -fsanitize=address,undefined -fno-omit-frame-pointer -fno-sanitize-recover=undefined
        tests/sanitize/host_checks.cpp tests/sanitize/stub_launchers.cpp
        exact_integer_gemm_amd/csrc/rns_host.cpp exact_integer_gemm_amd/csrc/rns_ratrec.cpp
        -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib -ldl -pthread

The launchers of the .hip sources are host stand-ins (tests/sanitize/stub_launchers.cpp)
that check the shapes they are handed; no device code is built or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["tests/sanitize/host_checks.cpp", "tests/sanitize/stub_launchers.cpp",
           "exact_integer_gemm_amd/csrc/rns_host.cpp", "exact_integer_gemm_amd/csrc/rns_ratrec.cpp"]
FLAGS = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
LINK = ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-ldl", "-pthread"]


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("g++ or the HIP host runtime is not available")
    exe = str(tmp_path / "host_checks")
    build = subprocess.run([gxx, *FLAGS, "-o", exe, *[os.path.join(ROOT, s) for s in SOURCES], *LINK],
                           capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    assert "host checks passed" in out
