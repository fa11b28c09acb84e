"""Depth utilisation: the pages' worked figure, and the kernel's own tile geometry."""
import os

import pytest

from oracle import depth_utilisation

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "depth_utilisation.txt")


def _golden():
    rows = []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_golden_chunked():
    rows = [r for r in _golden() if r[0] == "chunked"]
    assert rows
    for _, C, G, u in rows:
        for (L, T) in [(1, 8), (3, 16), (24, 8)]:
            assert depth_utilisation(int(C), int(G), L, T, "chunked") == pytest.approx(float(u), abs=0)


def test_golden_naive():
    assert any(r[0] == "naive" and r[3] == "1/T" for r in _golden())
    for (G, L, T) in [(1, 1, 4), (8, 3, 8), (2, 5, 16)]:
        assert depth_utilisation(0, G, L, T, "naive") == pytest.approx(1.0 / T, abs=1e-15)
