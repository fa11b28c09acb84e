"""Oracle for 8-bit depth KV.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the plain CPU definition
that the GPU quantisation and the quantised forward are checked against.  Only
the tests, the smoke check and the CPU-baseline leg of the benchmark may
import it; it imports nothing from the product.

Source.  The mhpn.cn article "动态混合深度注意力机制MoDA技术解析", section 4.2
(memory optimisation), suggests 8-bit quantisation for the depth KV of models
deeper than 32 layers, without fixing a format.  Reading taken (the plainest
one): symmetric per-row int8 with one float32 scale per row, where a row is one
key (or value) vector of d elements -- one (b, t, slot, kv head):

    scale = max_i |x_i| / 127              (float32 division)
    code_i = rint(x_i / scale)             (float32 division, ties to even),
                                           clamped to [-127, 127]
    code_i = 0 for every i when scale == 0 (an all-zero row)
    dequantised x_i = scale * code_i

Codes and scales are decided in float32 (the precision of the inputs' upcast),
so that the GPU kernel, taking the same float32 steps, reproduces them bit for
bit.  The quantised forward is the MoDA forward (oracle.moda_forward) applied
to the dequantised depth KV, evaluated in float64.

Parity pins (tests/test_oracle_quant.py): the rounding bound
|x - dequantised x| <= scale / 2, the row maximum mapping to +-127 exactly,
exact codes for rows that are integer multiples of a power of two, sign
symmetry, the all-zero row, and a scalar pure-Python implementation of the
same float32 steps (Python's float rounded to float32 with struct).  None of
these functions is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def quantize_rows(x):
    """Quantise the last axis of x to int8 codes with one float32 scale per row.

    x: array of any float dtype, [..., d].  Returns (codes int8 [..., d],
    scales float32 [...]).  Decisions in float32 (see module docstring).
    """
    x32 = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x32), axis=-1)                              # float32
    scale = (absmax / np.float32(127.0)).astype(np.float32)            # float32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    r = np.rint(x32 / safe[..., None]).astype(np.float32)              # float32 division, ties to even
    r = np.clip(r, -127, 127)
    r = np.where(scale[..., None] > 0, r, 0)
    return r.astype(np.int8), scale


def dequantize_rows(codes, scales):
    """float64 scale * code, [..., d]."""
    return np.asarray(scales, dtype=np.float64)[..., None] * np.asarray(codes, dtype=np.float64)


def quantize_rows_scalar(rows):
    """The same definition with scalar Python loops, for tiny inputs only.

    rows: nested list (or array) [n][d].  Float32 rounding of every step is
    emulated with struct (IEEE-754 single, round to nearest even).
    Returns (codes [n][d] ints, scales [n] floats).
    """
    import struct

    def f32(v):
        return struct.unpack("<f", struct.pack("<f", v))[0]

    def rint_even(v):
        fl = int(v // 1)
        frac = v - fl
        if frac > 0.5 or (frac == 0.5 and fl % 2 == 1):
            return fl + 1
        return fl

    codes, scales = [], []
    for row in np.asarray(rows, dtype=np.float32).tolist():
        row = [f32(v) for v in row]
        m = 0.0
        for v in row:
            m = max(m, abs(v))
        s = f32(m / 127.0)
        if s == 0.0:
            codes.append([0] * len(row))
        else:
            codes.append([max(-127, min(127, rint_even(f32(v / s)))) for v in row])
        scales.append(s)
    return codes, scales
