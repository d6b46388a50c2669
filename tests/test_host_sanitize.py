"""The C ABI's host half under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_check.cpp is compiled with g++ together with the library's host
sources (validation, size queries, workspace layouts, argument marshalling,
tracing, side stream) and stand-ins for the kernel launchers, then run on the
CPU: every entry point with buffers of exactly the queried sizes, for every
benchmark shape and a set of edge shapes, with each array handed to a kernel
checked to lie inside a caller buffer. No GPU and no device code are used.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_sparse_ffn_03_amd", "csrc")
HOST_SOURCES = ["twell_api.hip", "side_stream.hip", "trace.hip", "twell_host.cpp"]


def _rocm():
    for p in (os.environ.get("ROCM_PATH"), "/opt/rocm"):
        if p and os.path.exists(os.path.join(p, "include", "hip", "hip_runtime.h")):
            return p
    return None


def test_host_half_under_sanitizers(tmp_path):
    gxx, rocm = shutil.which("g++"), _rocm()
    if gxx is None or rocm is None:
        pytest.skip("needs g++ and the ROCm headers / runtime library")
    exe = str(tmp_path / "host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-x", "c++"]
    cmd += [os.path.join(CSRC, s) for s in HOST_SOURCES]
    cmd += [os.path.join(ROOT, "tests", "host_check.cpp"), "-L", os.path.join(rocm, "lib"), "-lamdhip64",
            f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"host check failed (rc {r.returncode}):\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "host check ok" in r.stdout
