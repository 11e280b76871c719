"""The host library (argument validation, the dispatch rule, kernel choice,
grid sizing) built by g++ with AddressSanitizer and UndefinedBehaviorSanitizer
against the HIP stand-ins of tests/sanitize/hip_host_stubs.cpp, then driven by
the ABI tests (tests/test_abi.py) and the kernel-choice checks
(tests/sanitize/host_plan_checks.py) in a child process: any sanitizer report
fails the test.  CPU only: no device code is built or run."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_297_amd", "csrc")


def _hip_include() -> str:
    for d in (os.environ.get("ROCM_PATH", ""), "/opt/rocm"):
        if d and os.path.exists(os.path.join(d, "include", "hip", "hip_runtime.h")):
            return os.path.join(d, "include")
    pytest.skip("HIP headers not found")


def test_host_library_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    lib = str(tmp_path / "libpagedattn_host_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", _hip_include(), "-I", CSRC, "-w", "-shared", "-fPIC",
           os.path.join(CSRC, "pa_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "hip_host_stubs.cpp"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    asan_rt = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.exists(asan_rt), asan_rt
    env = dict(os.environ)
    # The sanitizer runtime must come first; whatever is preloaded already stays.
    env["LD_PRELOAD"] = " ".join(x for x in (asan_rt, os.environ.get("LD_PRELOAD", "")) if x)
    env.update(PA_LIB_PATH=lib, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
         "tests/test_abi.py", "tests/sanitize/host_plan_checks.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = run.stdout + run.stderr
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-6000:]
    assert run.returncode == 0, text[-6000:]
    assert " passed" in text and "skipped" not in text.splitlines()[-1], text[-2000:]
