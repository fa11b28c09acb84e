"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments before making any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import depth_augmented_attention_amd as moda
from depth_augmented_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moda.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moda_[a-z0-9_]+)\s*\(", src)))


def test_header_matches_binding():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_symbol():
    lib = moda.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moda_\w+)", out))
    assert set(_declared()) <= exported


def test_status_strings():
    for code in range(6):
        assert moda.status_string(code).startswith("MODA_")
    assert "unknown" in moda.status_string(99)


def test_packed_elems():
    lib = moda.load()
    assert lib.moda_depth_packed_elems(1, 128, 1, 64, 3) == 128 * 3 * 64
    assert lib.moda_depth_packed_elems(3, 77, 3, 128, 5) == 3 * 3 * 416 * 128   # 385 -> 416
    assert lib.moda_depth_packed_elems(1, 65536, 2, 128, 24) == 2 * 65536 * 24 * 128
    assert lib.moda_depth_packed_elems(1, 5, 1, 64, 0) == 0
    assert lib.moda_depth_packed_elems(0, 5, 1, 64, 1) == -1
    assert lib.moda_depth_packed_elems(1, 5, 1, 64, -1) == -1


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("args,code", [
    # q, k, v, kd, vd, out, lse, B, T, Hq, Hkv, d, L_d, dtype
    ((None, FAKE, FAKE, None, None, FAKE, None, 1, 4, 2, 1, 128, 0, 1), _lib.MODA_ERR_NULL),
    ((FAKE, FAKE, FAKE, None, None, None, None, 1, 4, 2, 1, 128, 0, 1), _lib.MODA_ERR_NULL),
    ((FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 1, 4, 2, 1, 128, 3, 1), _lib.MODA_ERR_NULL),
    ((FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 4, 3, 2, 128, 0, 1), _lib.MODA_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 0, 2, 1, 128, 0, 1), _lib.MODA_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, None, None, FAKE, None, 0, 4, 2, 1, 128, 0, 1), _lib.MODA_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 4, 2, 1, 128, -1, 1), _lib.MODA_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 4, 2, 1, 128, 0, 7), _lib.MODA_ERR_DTYPE),
    ((FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 4, 2, 1, 96, 0, 1), _lib.MODA_ERR_UNSUPPORTED),
])
def test_fwd_validation(args, code):
    lib = moda.load()
    assert lib.moda_fwd(*args, None) == code


def test_pack_validation():
    lib = moda.load()
    # L_d == 0: nothing to do, NULL pointers allowed, no HIP call
    assert lib.moda_pack_depth(None, None, None, None, 1, 4, 1, 128, 0, 1, None) == _lib.MODA_OK
    assert lib.moda_pack_depth(None, FAKE, FAKE, FAKE, 1, 4, 1, 128, 2, 1, None) == _lib.MODA_ERR_NULL
    assert lib.moda_pack_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 100, 2, 1, None) == _lib.MODA_ERR_UNSUPPORTED
    assert lib.moda_pack_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 2, 5, None) == _lib.MODA_ERR_DTYPE
    assert lib.moda_pack_depth(FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 128, 2, 1, None) == _lib.MODA_ERR_SHAPE


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moda.moda_fwd(q, k, k, None, None, 0)


def test_product_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "depth_augmented_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in src.lower(), f"{f} mentions the oracle"


def test_window_validation():
    lib = moda.load()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 1, 128)
    assert lib.moda_fwd_window(*args, 4, 0, 5, 1, None) == _lib.MODA_ERR_SHAPE    # hi > L_cap
    assert lib.moda_fwd_window(*args, 4, 3, 2, 1, None) == _lib.MODA_ERR_SHAPE    # lo > hi
    assert lib.moda_fwd_window(*args, 4, -1, 2, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_fwd_window(*args, -1, 0, 0, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_fwd_window(FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 1, 4, 2, 1, 128,
                               4, 1, 2, 1, None) == _lib.MODA_ERR_NULL
    assert lib.moda_fwd_window(*args, 4, 0, 2, 9, None) == _lib.MODA_ERR_DTYPE


def test_append_validation():
    lib = moda.load()
    assert lib.moda_append_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, 3, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_append_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 0, 0, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_append_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, -1, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_append_depth(None, FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, 1, 1, None) == _lib.MODA_ERR_NULL
    assert lib.moda_append_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 96, 3, 1, 1, None) == _lib.MODA_ERR_UNSUPPORTED
    assert lib.moda_append_depth(FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, 1, 4, None) == _lib.MODA_ERR_DTYPE


def test_bwd_validation():
    lib = moda.load()
    # q k v kd vd out lse dout dq dk dv dkd dvd work
    ok = [FAKE] * 14
    sizes = [1, 4, 2, 1, 128, 3, 1]

    def call(ptrs, sz):
        return lib.moda_bwd(*ptrs, *sz, None)

    for i in range(14):
        ptrs = list(ok)
        ptrs[i] = None
        assert call(ptrs, sizes) == _lib.MODA_ERR_NULL, f"pointer {i}"
    # with L_d == 0 the four depth pointers may be NULL (nothing else may)
    l0 = list(ok)
    for i in (3, 4, 11, 12):
        l0[i] = None
    bad = list(l0)
    bad[13] = None
    assert call(bad, [1, 4, 2, 1, 128, 0, 1]) == _lib.MODA_ERR_NULL
    assert call(ok, [1, 4, 3, 2, 128, 3, 1]) == _lib.MODA_ERR_SHAPE      # Hq % Hkv
    assert call(ok, [1, 0, 2, 1, 128, 3, 1]) == _lib.MODA_ERR_SHAPE
    assert call(ok, [1, 4, 2, 1, 128, -1, 1]) == _lib.MODA_ERR_SHAPE
    assert call(ok, [1, 4, 2, 1, 96, 3, 1]) == _lib.MODA_ERR_UNSUPPORTED
    assert call(ok, [1, 4, 2, 1, 128, 3, 2]) == _lib.MODA_ERR_DTYPE


def test_q8_validation():
    lib = moda.load()
    # pack: L_d == 0 is a no-op with NULL pointers; a NULL scale is rejected
    assert lib.moda_pack_depth_q8(None, None, None, None, None, None, 1, 4, 1, 128, 0, 1, None) == _lib.MODA_OK
    assert lib.moda_pack_depth_q8(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 128, 3, 1, None) == _lib.MODA_ERR_NULL
    assert lib.moda_pack_depth_q8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 100, 3, 1, None) == _lib.MODA_ERR_UNSUPPORTED
    assert lib.moda_pack_depth_q8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, 9, None) == _lib.MODA_ERR_DTYPE
    # forward: scales are required when slots are read
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.moda_fwd_q8(*args, None, FAKE, FAKE, None, 1, 4, 2, 1, 128, 3, 1, None) == _lib.MODA_ERR_NULL
    assert lib.moda_fwd_q8(*args, FAKE, FAKE, FAKE, None, 1, 4, 3, 2, 128, 3, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_fwd_q8(*args, FAKE, FAKE, FAKE, None, 1, 4, 2, 1, 128, -1, 1, None) == _lib.MODA_ERR_SHAPE


def test_window_q8_and_bwd_window_validation():
    lib = moda.load()
    a5 = (FAKE,) * 5
    # fwd_window_q8: window past the capacity, missing scales
    assert lib.moda_fwd_window_q8(*a5, FAKE, FAKE, FAKE, None, 1, 4, 2, 1, 128, 4, 0, 5, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_fwd_window_q8(*a5, None, FAKE, FAKE, None, 1, 4, 2, 1, 128, 4, 1, 3, 1, None) == _lib.MODA_ERR_NULL
    # append_q8: slot out of range, NULL scale
    assert lib.moda_append_depth_q8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, 3, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_append_depth_q8(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 4, 1, 128, 3, 1, 1, None) == _lib.MODA_ERR_NULL
    # bwd_window: empty window allows NULL depth pointers; a bad window is rejected
    ptrs = [FAKE] * 14
    assert lib.moda_bwd_window(*ptrs, 1, 4, 2, 1, 128, 4, 3, 2, 1, None) == _lib.MODA_ERR_SHAPE
    ptrs[11] = None
    assert lib.moda_bwd_window(*ptrs, 1, 4, 2, 1, 128, 4, 1, 3, 1, None) == _lib.MODA_ERR_NULL


def test_bwd_q8_validation():
    lib = moda.load()
    # q k v kq vq ks vs out lse dout dq dk dv dkd dvd work
    ok = [FAKE] * 16
    for i in (5, 6):                               # a NULL row scale with slots read
        ptrs = list(ok)
        ptrs[i] = None
        assert lib.moda_bwd_q8(*ptrs, 1, 4, 2, 1, 128, 3, 1, None) == _lib.MODA_ERR_NULL
    assert lib.moda_bwd_q8(*ok, 1, 4, 2, 1, 128, -1, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_bwd_q8(*ok, 1, 4, 2, 1, 96, 3, 1, None) == _lib.MODA_ERR_UNSUPPORTED
    assert lib.moda_bwd_window_q8(*ok, 1, 4, 2, 1, 128, 4, 3, 2, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_bwd_window_q8(*ok, 1, 4, 2, 1, 128, 4, 0, 5, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_bwd_window_q8(*ok, 1, 1 << 20, 2, 1, 128, 1 << 11, 0, 1, 1, None) == _lib.MODA_ERR_SHAPE


def test_packed_key_index_bound():
    # T * L_cap must leave the packed key index n = t * L_cap + slot (plus the
    # padding to 32) inside 31 bits: every entry point that takes a depth
    # capacity rejects a larger one before any HIP call
    lib = moda.load()
    T, cap = 1 << 20, 1 << 11                     # T * cap = 2^31
    a = (FAKE,) * 6
    assert lib.moda_fwd_window(*a, None, 1, T, 2, 1, 128, cap, 0, 1, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_fwd_window_q8(*(FAKE,) * 8, None, 1, T, 2, 1, 128, cap, 0, 1, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_append_depth(FAKE, FAKE, FAKE, FAKE, 1, T, 1, 128, cap, 0, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_append_depth_q8(*(FAKE,) * 6, 1, T, 1, 128, cap, 0, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_bwd_window(*(FAKE,) * 14, 1, T, 2, 1, 128, cap, 0, 1, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_pack_depth(FAKE, FAKE, FAKE, FAKE, 1, T, 1, 128, cap, 1, None) == _lib.MODA_ERR_SHAPE


def test_binding_rejects_mixed_devices():
    # every tensor of one call must live on one GPU: the library launches on
    # the current device (checked in the binding before any HIP call)
    from depth_augmented_attention_amd import ops
    a = torch.empty(0)
    assert ops._one_device(a, None, a) == a.device
    with pytest.raises(ValueError):
        ops._one_device(a, torch.empty(0, device="meta"))


def test_fwd_workspace_validation():
    lib = _lib.load()
    # small grids of the bf16 d = 128 kernel split their longest tiles: a
    # 4096-byte counter header + two 66 x 64 float states per (split tile, wave)
    units = 2 * 128 * 4                       # B = 1, T = 4096, G = 8, Hkv = 2: 128 split tiles per kv head
    assert lib.moda_fwd_workspace_bytes(1, 4096, 16, 2, 128, 1) == 4096 + units * 33792
    assert lib.moda_fwd_workspace_bytes(5, 1000, 8, 1, 128, 1) == 4096 + 5 * 31 * 4 * 33792
    assert lib.moda_fwd_workspace_bytes(1, 1000, 8, 1, 128, 1) == 0       # one round: split inside the workgroup
    assert lib.moda_fwd_workspace_bytes(1, 65536, 16, 2, 128, 1) == 0     # big grid: whole tiles
    assert lib.moda_fwd_workspace_bytes(1, 4096, 16, 2, 128, 0) == 0      # float32: generic kernel
    assert lib.moda_fwd_workspace_bytes(1, 4096, 16, 2, 64, 1) == 0       # d = 64: generic kernel
    assert lib.moda_fwd_workspace_bytes(1, 1, 2, 1, 128, 1) == 0          # one tile: nothing to split
    assert lib.moda_fwd_workspace_bytes(1, 4096, 16, 3, 128, 1) == -1     # Hq not a multiple of Hkv
    # no shape needs more than 512 workgroups' worth
    worst = max(lib.moda_fwd_workspace_bytes(B, T, Hq, 1, 128, 1)
                for B in (1, 2, 4) for T in (64, 257, 1000, 4096, 8191) for Hq in (1, 8, 32, 64))
    assert 0 < worst <= 4096 + 1024 * 33792
    need = lib.moda_fwd_workspace_bytes(1, 4096, 16, 2, 128, 1)
    a = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4096, 16, 2, 128, 24, 1)
    assert lib.moda_fwd_ws(*a, None, need, None) == _lib.MODA_ERR_WORKSPACE               # no workspace
    assert lib.moda_fwd_ws(*a, 4096, need - 1, None) == _lib.MODA_ERR_WORKSPACE           # too small
    assert lib.moda_fwd_ws(*a, 4096 + 64, need, None) == _lib.MODA_ERR_WORKSPACE          # misaligned
    assert lib.moda_fwd_ws(*a[:7], 1, 4096, 16, 3, 128, 24, 1, 4096, need, None) == _lib.MODA_ERR_SHAPE
    assert "workspace" in _lib.status_string(_lib.MODA_ERR_WORKSPACE)


def test_bwd_noalloc_validation():
    lib = _lib.load()
    # B * Hq * T = 2^22 + 64 rows: beyond the 32 MiB static scratch, rejected
    # before anything is enqueued (no GPU needed)
    args = [FAKE] * 11 + [None, None]
    assert lib.moda_bwd_noalloc(*args, 1, 65537, 64, 1, 128, 0, 1, None) == _lib.MODA_ERR_WORKSPACE
    assert lib.moda_bwd_noalloc(*args, 1, 65536, 64, 1, 128, -1, 1, None) == _lib.MODA_ERR_SHAPE
    assert lib.moda_bwd_noalloc(*([FAKE] * 10), None, None, None, 1, 64, 4, 1, 128, 0, 1, None) \
        == _lib.MODA_ERR_NULL
    assert lib.moda_bwd_noalloc(*args, 1, 64, 4, 1, 96, 0, 1, None) == _lib.MODA_ERR_UNSUPPORTED


def test_bwd_workspace_validation():
    lib = _lib.load()
    work = lambda B, T, Hq: (2 * B * Hq * T * 4 + 255) // 256 * 256
    # short sequences (bf16, d = 128): the work buffer + 128 KiB per chunk of
    # the row-split dK/dV, at most 256 + B * Hkv * ceil(T / 128) chunks
    for (B, T, Hq, Hkv) in ((1, 4096, 16, 2), (1, 1000, 8, 1), (2, 700, 12, 2), (1, 16384, 16, 2), (1, 257, 64, 1)):
        n = lib.moda_bwd_workspace_bytes(B, T, Hq, Hkv, 128, 1)
        extra = n - work(B, T, Hq)
        assert extra > 0 and extra % (131072 * B * Hkv) == 0, (B, T, Hq, Hkv, n)
        assert extra // 131072 <= 256 + B * Hkv * ((T + 127) // 128)
    # no split: grids that fill the GPU, one key tile, generic kernels
    for (B, T, Hq, Hkv, d, dt) in ((1, 65536, 16, 2, 128, 1), (2, 16384, 16, 2, 128, 1), (1, 100, 8, 1, 128, 1),
                                   (1, 4096, 16, 2, 128, 0), (1, 4096, 16, 2, 64, 1)):
        assert lib.moda_bwd_workspace_bytes(B, T, Hq, Hkv, d, dt) == work(B, T, Hq)
    assert lib.moda_bwd_workspace_bytes(1, 4096, 16, 3, 128, 1) == -1     # Hq not a multiple of Hkv
    assert lib.moda_bwd_workspace_bytes(1, 4096, 16, 2, 128, 9) == -1     # unknown dtype
    need = lib.moda_bwd_workspace_bytes(1, 4096, 16, 2, 128, 1)
    a = [FAKE] * 11 + [None, None, 1, 4096, 16, 2, 128, 0, 1]
    assert lib.moda_bwd_ws(*a, None, need, None) == _lib.MODA_ERR_WORKSPACE              # no workspace
    assert lib.moda_bwd_ws(*a, 4096, need - 1, None) == _lib.MODA_ERR_WORKSPACE          # too small
    assert lib.moda_bwd_ws(*a, 4096 + 64, need, None) == _lib.MODA_ERR_WORKSPACE         # misaligned
    a[15] = 3                                                                          # Hq % Hkv != 0
    assert lib.moda_bwd_ws(*a, 4096, need, None) == _lib.MODA_ERR_SHAPE
