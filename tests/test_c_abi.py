"""The C ABI from plain C: tests/c/abi_check.c is compiled with gcc against
include/moda.h, linked to libmoda.so, and run (validation paths only, no GPU)."""
import os
import shutil
import subprocess

import pytest

import depth_augmented_attention_amd as moda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_client(tmp_path):
    moda.load()   # the library must be built
    libdir = os.path.dirname(moda.LIB_PATH)
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe),
           "-L", libdir, "-lmoda", "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed" in r.stdout
