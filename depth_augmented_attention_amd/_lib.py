"""ctypes loader for libmoda.so (the C ABI declared in include/moda.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MODA_LIB", os.path.join(_HERE, "libmoda.so"))

MODA_F32 = 0
MODA_BF16 = 1

MODA_OK = 0
MODA_ERR_NULL = 1
MODA_ERR_SHAPE = 2
MODA_ERR_DTYPE = 3
MODA_ERR_UNSUPPORTED = 4
MODA_ERR_HIP = 5
MODA_ERR_WORKSPACE = 6

# every symbol include/moda.h declares
EXPORTS = ("moda_depth_packed_elems", "moda_pack_depth", "moda_fwd", "moda_fwd_workspace_bytes", "moda_fwd_ws",
           "moda_fwd_window",
           "moda_append_depth", "moda_bwd", "moda_bwd_workspace_bytes", "moda_bwd_ws", "moda_bwd_noalloc", "moda_bwd_window", "moda_pack_depth_q8", "moda_fwd_q8",
           "moda_fwd_window_q8", "moda_append_depth_q8", "moda_bwd_q8", "moda_bwd_window_q8",
           "moda_status_string")


class ModaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m depth_augmented_attention_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_vp = ctypes.c_int, ctypes.c_void_p
    lib.moda_depth_packed_elems.argtypes = [c_int] * 5
    lib.moda_depth_packed_elems.restype = ctypes.c_longlong
    lib.moda_pack_depth.argtypes = [c_vp] * 4 + [c_int] * 6 + [c_vp]
    lib.moda_pack_depth.restype = c_int
    lib.moda_fwd.argtypes = [c_vp] * 6 + [c_vp] + [c_int] * 7 + [c_vp]
    lib.moda_fwd.restype = c_int
    lib.moda_fwd_workspace_bytes.argtypes = [c_int] * 6
    lib.moda_fwd_workspace_bytes.restype = ctypes.c_longlong
    lib.moda_fwd_ws.argtypes = [c_vp] * 6 + [c_vp] + [c_int] * 7 + [c_vp, ctypes.c_longlong, c_vp]
    lib.moda_fwd_ws.restype = c_int
    lib.moda_fwd_window.argtypes = [c_vp] * 6 + [c_vp] + [c_int] * 9 + [c_vp]
    lib.moda_fwd_window.restype = c_int
    lib.moda_append_depth.argtypes = [c_vp] * 4 + [c_int] * 7 + [c_vp]
    lib.moda_append_depth.restype = c_int
    lib.moda_bwd.argtypes = [c_vp] * 14 + [c_int] * 7 + [c_vp]
    lib.moda_bwd.restype = c_int
    lib.moda_bwd_workspace_bytes.argtypes = [c_int] * 6
    lib.moda_bwd_workspace_bytes.restype = ctypes.c_longlong
    lib.moda_bwd_ws.argtypes = [c_vp] * 13 + [c_int] * 7 + [c_vp, ctypes.c_longlong, c_vp]
    lib.moda_bwd_ws.restype = c_int
    lib.moda_bwd_noalloc.argtypes = [c_vp] * 13 + [c_int] * 7 + [c_vp]
    lib.moda_bwd_noalloc.restype = c_int
    lib.moda_pack_depth_q8.argtypes = [c_vp] * 6 + [c_int] * 6 + [c_vp]
    lib.moda_pack_depth_q8.restype = c_int
    lib.moda_fwd_q8.argtypes = [c_vp] * 9 + [c_int] * 7 + [c_vp]
    lib.moda_fwd_q8.restype = c_int
    lib.moda_bwd_window.argtypes = [c_vp] * 14 + [c_int] * 9 + [c_vp]
    lib.moda_bwd_window.restype = c_int
    lib.moda_fwd_window_q8.argtypes = [c_vp] * 9 + [c_int] * 9 + [c_vp]
    lib.moda_fwd_window_q8.restype = c_int
    lib.moda_append_depth_q8.argtypes = [c_vp] * 6 + [c_int] * 7 + [c_vp]
    lib.moda_append_depth_q8.restype = c_int
    lib.moda_bwd_q8.argtypes = [c_vp] * 16 + [c_int] * 7 + [c_vp]
    lib.moda_bwd_q8.restype = c_int
    lib.moda_bwd_window_q8.argtypes = [c_vp] * 16 + [c_int] * 9 + [c_vp]
    lib.moda_bwd_window_q8.restype = c_int
    lib.moda_status_string.argtypes = [c_int]
    lib.moda_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moda_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != MODA_OK:
        raise ModaError(status, what)
