"""The library's host code (scheduler, argument checks, JFA_VALIDATE, workspace
arithmetic) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven
by tests/host_abi_check.cpp, with the kernel launchers and HIP runtime calls
stubbed out (CPU only: no GPU, no HIP runtime)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_flash_jaggedfa_amd", "csrc")


def _compiler():
    for c in ("g++", "clang++"):
        if shutil.which(c):
            return shutil.which(c)
    return None


def test_host_code_under_sanitizers(tmp_path):
    cxx = _compiler()
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_abi_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_abi_check.cpp"), os.path.join(CSRC, "schedule.cpp"),
           os.path.join(CSRC, "api.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("JFA_VALIDATE", None)
    env.pop("JFA_LOG", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
