"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host part of libfsa (argument checks, schedules, the tap planner) is
rebuilt with both sanitizers into a temporary library (the kernels are built
as usual), and the plain-C test tests/c/abi_host.c, also built with them, runs
against it with leak detection on. Device code is not instrumented.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from static_pattern_sparse_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "static_pattern_sparse_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
KERNEL_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
INC = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]


def test_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm toolchain not found")
    d = str(tmp_path)
    jobs = [subprocess.Popen(
        [HIPCC, "-c", "-fPIC", "-O1", "-g", "-std=c++17",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         *INC, "-o", os.path.join(d, "api.o"), os.path.join(CSRC, "fsa_api.cpp")])]
    kernels = [os.path.splitext(n)[0] for n in build_lib.SOURCES if n.endswith(".hip")]
    for name in kernels:
        jobs.append(subprocess.Popen(
            [HIPCC, "-c", *KERNEL_FLAGS, *INC, "-o", os.path.join(d, name + ".o"),
             os.path.join(CSRC, name + ".hip")],
            stderr=subprocess.DEVNULL))
    assert all(j.wait(timeout=600) == 0 for j in jobs)
    lib = os.path.join(d, "libfsa.so")
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", lib,
                    *(os.path.join(d, n + ".o") for n in ["api", *kernels])],
                   check=True)
    exe = os.path.join(d, "abi_host")
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", d, "-lfsa",
                    f"-Wl,-rpath,{d}", "-lm", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("ok")
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr
