"""The C ABI from plain C: tests/c/abi_host.c is compiled with gcc against
include/fsa.h, linked to libfsa.so and run (host-only calls, no GPU)."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "static_pattern_sparse_amd")


def test_c_program_against_the_header(tmp_path):
    lib = os.path.join(PKG, "libfsa.so")
    if not os.path.exists(lib):
        pytest.skip("libfsa.so not built")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_host"
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", PKG, "-lfsa",
                    f"-Wl,-rpath,{PKG}", "-lm", "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("ok")
