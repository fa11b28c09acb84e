"""MoDA (mixture-of-depths attention) forward and backward for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
libmoda.so (include/moda.h); this package only marshals tensors into it.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MODA_BF16,
    MODA_F32,
    ModaError,
    load,
    status_string,
)
from .ops import (  # noqa: F401
    bwd_workspace,
    bwd_workspace_bytes,
    depth_packed_elems,
    fwd_workspace,
    fwd_workspace_bytes,
    moda_append_depth,
    moda_append_depth_q8,
    moda_bwd,
    moda_bwd_noalloc,
    moda_bwd_q8,
    moda_bwd_window,
    moda_bwd_window_q8,
    moda_fwd,
    moda_fwd_q8,
    moda_fwd_window,
    moda_fwd_window_q8,
    moda_pack_depth,
    moda_pack_depth_q8,
)
