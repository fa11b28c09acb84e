"""The kernel-source hash that ties the committed HBM-traffic counters to the
forward kernel's code: comments and spacing do not change it, code does
(CPU only)."""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_spacing():
    a = 'int a = 1;  // one\n/* block\n comment */ float b = 2.f;\n'
    b = 'int a = 1;\nfloat b = 2.f; // two'
    assert bench._code_only(a) == bench._code_only(b) == "int a = 1; float b = 2.f;"


def test_code_only_keeps_strings_and_code_changes():
    assert bench._code_only('s = "// not a comment";') == 's = "// not a comment";'
    assert bench._code_only('x = "a\\"//b"; // c') == 'x = "a\\"//b";'
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_more_than_one_gpu_exits_with_a_message():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so,
    before touching a GPU."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

