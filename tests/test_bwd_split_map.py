"""The row-split dK/dV map of the backward workspace path, checked on the CPU.

tests/c/split_map_check.cpp includes the map's header with the host compiler
alone and, over about 18000 (T, G, B * Hkv) shapes that split, compares the
closed forms the kernels use with plain loops over the key tiles, and checks
that every query block of every key tile is swept by exactly one chunk, that
the chunk slots the reduce kernel reads are the ones the dK/dV kernel wrote,
and that the remainder chunks come longest first.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GXX = shutil.which("g++")


@pytest.mark.skipif(GXX is None, reason="g++ not available")
def test_split_map(tmp_path):
    exe = tmp_path / "split_map_check"
    subprocess.run([GXX, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror", "-fsanitize=undefined",
                    "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "depth_augmented_attention_amd", "csrc"),
                    os.path.join(ROOT, "tests", "c", "split_map_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
