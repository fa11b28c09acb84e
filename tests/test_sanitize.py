"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; no GPU call is made).

libmoda.so is rebuilt into a temporary folder with the sanitizers on its host
code only (each -fsanitize= follows -Xarch_host; the GPU code is built as
usual), then
  * the plain-C clients tests/c/abi_check.c (documented error codes) and
    tests/c/abi_extremes.c (INT_MAX / INT_MIN sizes through every entry
    point, where the size arithmetic must neither overflow nor accept) are
    built with the same sanitizers and run, any report aborting the run;
  * the ctypes validation tests of tests/test_abi.py run against that build,
    with the sanitizer runtime preloaded into the Python process.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None or not os.path.exists(CLANG), reason="hipcc / clang not available")

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    lib = d / "libmoda.so"
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "depth_augmented_attention_amd", "csrc"),
           "-o", str(lib), os.path.join(ROOT, "depth_augmented_attention_amd", "csrc", "moda_api.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return lib


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


@pytest.mark.parametrize("client", ["abi_check", "abi_extremes"])
def test_c_client_sanitized(san_lib, client, tmp_path):
    exe = tmp_path / client
    cmd = [CLANG, "-std=c11", "-g", *SAN, "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", client + ".c"), "-o", str(exe), "-L", str(san_lib.parent), "-lmoda",
           "-Wl,-rpath," + str(san_lib.parent)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=_env())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_ctypes_validation_sanitized(san_lib):
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("sanitizer runtime not found")
    env = _env()
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] += ":verify_asan_link_order=0"
    env["MODA_LIB"] = str(san_lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, timeout=600,
                       env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
