"""Tensor-level binding of the C ABI: argument marshalling only.

Every step of the computation runs in the HIP kernels of libmoda.so; torch
provides device memory and the current stream.  There is no fallback path:
if the library is missing or the tensors are not on a GPU these calls raise.
"""
from __future__ import annotations

import torch

from ._lib import MODA_BF16, MODA_F32, check, load

_DT = {torch.float32: MODA_F32, torch.bfloat16: MODA_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")
    return _DT[t.dtype]


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _one_device(*tensors) -> torch.device:
    """The GPU that all (non-None) tensors of one call live on."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors of one call must be on one GPU, got {sorted(map(str, devs))}")
    return devs.pop()


def _call(device: torch.device, fn: str, stream, *args) -> int:
    """Call C entry point `fn` with `device` current (the library launches on
    the current device); the stream (default: that device's current stream)
    is the last argument."""
    with torch.cuda.device(device):
        return getattr(load(), fn)(*args, _stream(stream))


def depth_packed_elems(B: int, T: int, Hkv: int, d: int, L_d: int) -> int:
    n = load().moda_depth_packed_elems(B, T, Hkv, d, L_d)
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def moda_pack_depth(k_depth: torch.Tensor, v_depth: torch.Tensor,
                    k_packed: torch.Tensor | None = None, v_packed: torch.Tensor | None = None,
                    stream=None):
    """Repack depth KV [B,T,L_d,Hkv,d] into the fused kernel's layout.

    Returns (k_packed, v_packed), flat tensors of depth_packed_elems(...)
    elements each (allocated here when not given).
    """
    if k_depth.dim() != 5 or v_depth.shape != k_depth.shape or v_depth.dtype != k_depth.dtype:
        raise ValueError("k_depth / v_depth must both be [B,T,L_d,Hkv,d] of one dtype")
    B, T, L_d, Hkv, d = k_depth.shape
    n = depth_packed_elems(B, T, Hkv, d, L_d)
    if k_packed is None:
        k_packed = torch.empty(n, dtype=k_depth.dtype, device=k_depth.device)
    if v_packed is None:
        v_packed = torch.empty(n, dtype=k_depth.dtype, device=k_depth.device)
    if L_d == 0:
        return k_packed, v_packed
    for t, name in ((k_depth, "k_depth"), (v_depth, "v_depth"), (k_packed, "k_packed"), (v_packed, "v_packed")):
        _dev(t, name)
    if k_packed.numel() != n or v_packed.numel() != n or k_packed.dtype != k_depth.dtype \
            or v_packed.dtype != k_depth.dtype:
        raise ValueError(f"packed buffers must hold {n} elements of {k_depth.dtype}")
    dev = _one_device(k_depth, v_depth, k_packed, v_packed)
    st = _call(dev, "moda_pack_depth", stream,
        k_depth.data_ptr(), v_depth.data_ptr(), k_packed.data_ptr(),
        v_packed.data_ptr(), B, T, Hkv, d, L_d, _dtype_code(k_depth))
    check(st, "moda_pack_depth")
    return k_packed, v_packed


def moda_append_depth(k_new: torch.Tensor, v_new: torch.Tensor, k_packed: torch.Tensor,
                      v_packed: torch.Tensor, L_cap: int, slot: int, stream=None):
    """Write step: store this layer's K/V [B,T,Hkv,d] into slot `slot` of packed
    depth buffers with L_cap slots per position (in place)."""
    if k_new.dim() != 4 or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must both be [B,T,Hkv,d] of one dtype")
    B, T, Hkv, d = k_new.shape
    n = depth_packed_elems(B, T, Hkv, d, L_cap)
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (k_packed, "k_packed"), (v_packed, "v_packed")):
        _dev(t, name)
    if k_packed.numel() != n or v_packed.numel() != n or k_packed.dtype != k_new.dtype \
            or v_packed.dtype != k_new.dtype:
        raise ValueError(f"packed buffers must hold {n} elements of {k_new.dtype}")
    dev = _one_device(k_new, v_new, k_packed, v_packed)
    st = _call(dev, "moda_append_depth", stream,
        k_new.data_ptr(), v_new.data_ptr(), k_packed.data_ptr(),
        v_packed.data_ptr(), B, T, Hkv, d, L_cap, slot,
        _dtype_code(k_new))
    check(st, "moda_append_depth")
    return k_packed, v_packed


def moda_fwd(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor,
             k_depth: torch.Tensor | None, v_depth: torch.Tensor | None, L_d: int,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
             with_lse: bool = True, stream=None, work: torch.Tensor | None = None):
    """MoDA forward.  q [B,T,Hq,d]; k_seq, v_seq [B,T,Hkv,d]; k_depth, v_depth
    are the packed buffers from moda_pack_depth (None when L_d == 0).

    work: optional workspace from fwd_workspace(q, k_seq) -- the call then
    goes to moda_fwd_ws, which splits the key range of the longest query
    tiles on small grids (short sequences).

    Returns (out [B,T,Hq,d], lse [B,Hq,T] float32 or None).
    """
    if work is not None:
        return _fwd_call("moda_fwd_ws", q, k_seq, v_seq, k_depth, v_depth, L_d, 0, L_d, out, lse, with_lse,
                         stream, work=work)
    return _fwd_call("moda_fwd", q, k_seq, v_seq, k_depth, v_depth, L_d, 0, L_d, out, lse, with_lse, stream)


def fwd_workspace_bytes(B: int, T: int, Hq: int, Hkv: int, d: int, dtype: torch.dtype) -> int:
    n = load().moda_fwd_workspace_bytes(B, T, Hq, Hkv, d, _DT.get(dtype, -1))
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def fwd_workspace(q: torch.Tensor, k_seq: torch.Tensor) -> torch.Tensor:
    """A zero-filled workspace for moda_fwd(..., work=...) on these shapes
    (uint8 on q's device; at least one byte so that it has an address)."""
    B, T, Hq, d = q.shape
    n = fwd_workspace_bytes(B, T, Hq, k_seq.shape[2], d, q.dtype)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=q.device)


def moda_fwd_window(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor,
                    k_depth: torch.Tensor | None, v_depth: torch.Tensor | None,
                    L_cap: int, slot_lo: int, slot_hi: int,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                    with_lse: bool = True, stream=None):
    """MoDA forward reading depth slots [slot_lo, slot_hi) of packed buffers
    with L_cap slots per position.

    Returns (out [B,T,Hq,d], lse [B,Hq,T] float32 or None).
    """
    return _fwd_call("moda_fwd_window", q, k_seq, v_seq, k_depth, v_depth, L_cap, slot_lo, slot_hi, out, lse,
                     with_lse, stream)


def _fwd_call(fn, q, k_seq, v_seq, k_depth, v_depth, L_cap, slot_lo, slot_hi, out, lse, with_lse, stream,
              work=None):
    """Checks and the call of moda_fwd / moda_fwd_ws (L_cap slots, all read)
    or moda_fwd_window."""
    if q.dim() != 4 or k_seq.dim() != 4 or v_seq.shape != k_seq.shape:
        raise ValueError("q must be [B,T,Hq,d], k_seq / v_seq [B,T,Hkv,d]")
    B, T, Hq, d = q.shape
    Hkv = k_seq.shape[2]
    if k_seq.shape[:2] != (B, T) or k_seq.shape[3] != d:
        raise ValueError("k_seq shape does not match q")
    if k_seq.dtype != q.dtype or v_seq.dtype != q.dtype:
        raise ValueError("q, k_seq, v_seq must share one dtype")
    for t, name in ((q, "q"), (k_seq, "k_seq"), (v_seq, "v_seq")):
        _dev(t, name)
    kd_ptr = vd_ptr = None
    if slot_hi > slot_lo:
        if k_depth is None or v_depth is None:
            raise ValueError("packed depth buffers are required when slots are read")
        n = depth_packed_elems(B, T, Hkv, d, L_cap)
        for t, name in ((k_depth, "k_depth"), (v_depth, "v_depth")):
            _dev(t, name)
            if t.numel() != n or t.dtype != q.dtype:
                raise ValueError(f"{name} must be a packed buffer of {n} elements of {q.dtype}")
        kd_ptr, vd_ptr = k_depth.data_ptr(), v_depth.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have the shape and dtype of q")
    if with_lse and lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse")
        if lse.dtype != torch.float32 or lse.shape != (B, Hq, T):
            raise ValueError("lse must be float32 [B,Hq,T]")
    dev = _one_device(q, k_seq, v_seq, k_depth if kd_ptr else None, v_depth if vd_ptr else None, out, lse)
    slots = (L_cap, slot_lo, slot_hi) if fn == "moda_fwd_window" else (L_cap,)
    extra = ()
    if fn == "moda_fwd_ws":
        _dev(work, "work")
        if work.device != q.device:
            raise ValueError("work must be on q's device")
        extra = (work.data_ptr(), work.numel() * work.element_size())
    st = _call(dev, fn, stream,
        q.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(), kd_ptr, vd_ptr,
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, T, Hq, Hkv, d, *slots, _dtype_code(q), *extra)
    check(st, fn)
    return out, lse


def moda_bwd(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor,
             k_depth: torch.Tensor | None, v_depth: torch.Tensor | None, L_d: int,
             out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
             grads: tuple | None = None, work: torch.Tensor | None = None, stream=None,
             workspace: torch.Tensor | None = None):
    """Gradients of the MoDA forward.

    q, k_seq, v_seq and the packed depth buffers as for moda_fwd; out and lse
    are that forward's results; dout [B,T,Hq,d] is the gradient of out.
    Returns (dq [B,T,Hq,d], dk_seq [B,T,Hkv,d], dv_seq [B,T,Hkv,d],
    dk_depth [B,T,L_d,Hkv,d], dv_depth [B,T,L_d,Hkv,d]) -- the depth gradients
    in the logical depth layout (one slot per earlier layer), or None when
    L_d == 0.  `grads` may supply those five output tensors; `work` a float32
    [2,B,Hq,T] scratch tensor.

    workspace: optional workspace from bwd_workspace(q, k_seq) (instead of
    `work`) -- the call then goes to moda_bwd_ws, which splits each key
    tile's query rows over several workgroups on short sequences.
    """
    if workspace is not None:
        if work is not None:
            raise ValueError("pass either work or workspace")
        return _bwd_call("moda_bwd_ws", q, k_seq, v_seq, k_depth, v_depth, L_d, 0, L_d, out, lse, dout, grads,
                         False, stream, workspace=workspace)
    return _bwd_call("moda_bwd", q, k_seq, v_seq, k_depth, v_depth, L_d, 0, L_d, out, lse, dout, grads, work,
                     stream)


def bwd_workspace_bytes(B: int, T: int, Hq: int, Hkv: int, d: int, dtype: torch.dtype) -> int:
    n = load().moda_bwd_workspace_bytes(B, T, Hq, Hkv, d, _DT.get(dtype, -1))
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def bwd_workspace(q: torch.Tensor, k_seq: torch.Tensor) -> torch.Tensor:
    """A workspace for moda_bwd(..., workspace=...) on these shapes (uint8 on
    q's device, uninitialised: every byte the call reads it writes first)."""
    B, T, Hq, d = q.shape
    return torch.empty(bwd_workspace_bytes(B, T, Hq, k_seq.shape[2], d, q.dtype), dtype=torch.uint8,
                       device=q.device)


def moda_bwd_noalloc(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor,
                     k_depth: torch.Tensor | None, v_depth: torch.Tensor | None, L_d: int,
                     out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                     grads: tuple, stream=None):
    """moda_bwd through the C entry point that allocates nothing: the work
    buffer is the library's static per-GPU scratch (B * Hq * T <= 4M).  The
    five gradient tensors must be supplied (`grads`, as returned by moda_bwd);
    calls on one GPU must not overlap in time."""
    if grads is None:
        raise ValueError("moda_bwd_noalloc needs the gradient tensors (grads)")
    (B, T, Hq, Hkv, d, L), grads, _ = _bwd_common(q, k_seq, v_seq, 0, L_d, out, lse, dout, grads, False)
    kd_ptr = vd_ptr = None
    if L > 0:
        if k_depth is None or v_depth is None:
            raise ValueError("packed depth buffers are required when slots are read")
        n = depth_packed_elems(B, T, Hkv, d, L_d)
        for t, name in ((k_depth, "k_depth"), (v_depth, "v_depth")):
            _dev(t, name)
            if t.numel() != n or t.dtype != q.dtype:
                raise ValueError(f"{name} must be a packed buffer of {n} elements of {q.dtype}")
        kd_ptr, vd_ptr = k_depth.data_ptr(), v_depth.data_ptr()
    ptr = [g.data_ptr() if g is not None else None for g in grads]
    dev = _one_device(q, k_seq, v_seq, k_depth if kd_ptr else None, v_depth if vd_ptr else None, out, lse,
                      dout, *grads[:3], *(grads[3:] if L > 0 else ()))
    st = _call(dev, "moda_bwd_noalloc", stream,
        q.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(), kd_ptr, vd_ptr,
        out.data_ptr(), lse.data_ptr(), dout.data_ptr(), ptr[0], ptr[1], ptr[2],
        ptr[3], ptr[4], B, T, Hq, Hkv, d, L_d, _dtype_code(q))
    check(st, "moda_bwd_noalloc")
    return grads


def _bwd_common(q, k_seq, v_seq, slot_lo, slot_hi, out, lse, dout, grads, work):
    """Shape / dtype / device checks shared by the backward calls; allocates
    the gradients and the work buffer when not given."""
    if q.dim() != 4 or k_seq.dim() != 4 or v_seq.shape != k_seq.shape:
        raise ValueError("q must be [B,T,Hq,d], k_seq / v_seq [B,T,Hkv,d]")
    B, T, Hq, d = q.shape
    Hkv = k_seq.shape[2]
    if k_seq.shape[:2] != (B, T) or k_seq.shape[3] != d:
        raise ValueError("k_seq shape does not match q")
    for t, name in ((k_seq, "k_seq"), (v_seq, "v_seq"), (out, "out"), (dout, "dout")):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have the dtype of q")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have the shape of q")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, T):
        raise ValueError("lse must be float32 [B,Hq,T]")
    for t, name in ((q, "q"), (k_seq, "k_seq"), (v_seq, "v_seq"), (out, "out"), (lse, "lse"),
                    (dout, "dout")):
        _dev(t, name)
    L_d = slot_hi - slot_lo
    Ld = max(L_d, 0)
    shapes = [(B, T, Hq, d), (B, T, Hkv, d), (B, T, Hkv, d), (B, T, Ld, Hkv, d), (B, T, Ld, Hkv, d)]
    if grads is None:
        grads = tuple(torch.empty(s, dtype=q.dtype, device=q.device) if (i < 3 or L_d > 0) else None
                      for i, s in enumerate(shapes))
    grads = tuple(grads)
    for i, (g, s) in enumerate(zip(grads, shapes)):
        if i >= 3 and L_d <= 0:
            continue
        if g is None or tuple(g.shape) != s or g.dtype != q.dtype:
            raise ValueError(f"gradient {i} must be {q.dtype} {s}")
        _dev(g, f"gradient {i}")
    if work is False:          # the caller passes no work buffer (moda_bwd_noalloc)
        return (B, T, Hq, Hkv, d, L_d), grads, None
    if work is None:
        work = torch.empty(2, B, Hq, T, dtype=torch.float32, device=q.device)
    _dev(work, "work")
    if work.dtype != torch.float32 or work.shape != (2, B, Hq, T):
        raise ValueError("work must be float32 [2,B,Hq,T]")
    return (B, T, Hq, Hkv, d, L_d), grads, work


def moda_bwd_window(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor,
                    k_depth: torch.Tensor | None, v_depth: torch.Tensor | None,
                    L_cap: int, slot_lo: int, slot_hi: int,
                    out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                    grads: tuple | None = None, work: torch.Tensor | None = None, stream=None):
    """Gradients of moda_fwd_window(..., L_cap, slot_lo, slot_hi): as
    moda_bwd, with the depth gradients of slots slot_lo .. slot_hi-1
    ([B,T,slot_hi-slot_lo,Hkv,d])."""
    return _bwd_call("moda_bwd_window", q, k_seq, v_seq, k_depth, v_depth, L_cap, slot_lo, slot_hi, out, lse,
                     dout, grads, work, stream)


def _bwd_call(fn, q, k_seq, v_seq, k_depth, v_depth, L_cap, slot_lo, slot_hi, out, lse, dout, grads, work,
              stream, workspace=None):
    """Checks and the call of moda_bwd / moda_bwd_ws (L_cap slots, all read;
    work False and a workspace for moda_bwd_ws) or moda_bwd_window."""
    (B, T, Hq, Hkv, d, L_d), grads, work = _bwd_common(q, k_seq, v_seq, slot_lo, slot_hi, out, lse, dout,
                                                       grads, work)
    kd_ptr = vd_ptr = None
    if L_d > 0:
        if k_depth is None or v_depth is None:
            raise ValueError("packed depth buffers are required when slots are read")
        n = depth_packed_elems(B, T, Hkv, d, L_cap)
        for t, name in ((k_depth, "k_depth"), (v_depth, "v_depth")):
            _dev(t, name)
            if t.numel() != n or t.dtype != q.dtype:
                raise ValueError(f"{name} must be a packed buffer of {n} elements of {q.dtype}")
        kd_ptr, vd_ptr = k_depth.data_ptr(), v_depth.data_ptr()
    ptr = [g.data_ptr() if g is not None else None for g in grads]
    if fn == "moda_bwd_ws":
        _dev(workspace, "workspace")
        dev = _one_device(q, k_seq, v_seq, k_depth if kd_ptr else None, v_depth if vd_ptr else None, out, lse,
                          dout, workspace, *grads[:3], *(grads[3:] if L_d > 0 else ()))
        st = _call(dev, fn, stream,
            q.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(), kd_ptr, vd_ptr,
            out.data_ptr(), lse.data_ptr(), dout.data_ptr(), ptr[0], ptr[1], ptr[2],
            ptr[3], ptr[4], B, T, Hq, Hkv, d, L_cap, _dtype_code(q),
            workspace.data_ptr(), workspace.numel() * workspace.element_size())
        check(st, fn)
        return grads
    dev = _one_device(q, k_seq, v_seq, k_depth if kd_ptr else None, v_depth if vd_ptr else None, out, lse,
                      dout, work, *grads[:3], *(grads[3:] if L_d > 0 else ()))
    slots = (L_cap,) if fn == "moda_bwd" else (L_cap, slot_lo, slot_hi)
    st = _call(dev, fn, stream,
        q.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(), kd_ptr, vd_ptr,
        out.data_ptr(), lse.data_ptr(), dout.data_ptr(), ptr[0], ptr[1], ptr[2],
        ptr[3], ptr[4], work.data_ptr(), B, T, Hq, Hkv, d, *slots,
        _dtype_code(q))
    check(st, fn)
    return grads


def moda_bwd_window_q8(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor, packed_q8,
                       L_cap: int, slot_lo: int, slot_hi: int,
                       out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                       grads: tuple | None = None, work: torch.Tensor | None = None, stream=None):
    """Gradients of moda_fwd_window_q8(..., L_cap, slot_lo, slot_hi): as
    moda_bwd_window, the depth keys and values read from the four 8-bit
    buffers of moda_pack_depth_q8 / moda_append_depth_q8; the depth
    gradients are those of the dequantised keys and values."""
    (B, T, Hq, Hkv, d, L_d), grads, work = _bwd_common(q, k_seq, v_seq, slot_lo, slot_hi, out, lse, dout,
                                                       grads, work)
    ptrs = _check_q8(packed_q8, B, T, Hkv, d, L_cap) if L_d > 0 else [None] * 4
    ptr = [g.data_ptr() if g is not None else None for g in grads]
    dev = _one_device(q, k_seq, v_seq, *(packed_q8 if L_d > 0 else ()), out, lse, dout, work, *grads[:3],
                      *(grads[3:] if L_d > 0 else ()))
    st = _call(dev, "moda_bwd_window_q8", stream,
        q.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(), *ptrs,
        out.data_ptr(), lse.data_ptr(), dout.data_ptr(), ptr[0], ptr[1], ptr[2],
        ptr[3], ptr[4], work.data_ptr(), B, T, Hq, Hkv, d, L_cap, slot_lo, slot_hi,
        _dtype_code(q))
    check(st, "moda_bwd_window_q8")
    return grads


def moda_bwd_q8(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor, packed_q8, L_d: int,
                out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                grads: tuple | None = None, work: torch.Tensor | None = None, stream=None):
    """Gradients of moda_fwd_q8 (the four buffers of moda_pack_depth_q8)."""
    return moda_bwd_window_q8(q, k_seq, v_seq, packed_q8, L_d, 0, L_d, out, lse, dout,
                              grads=grads, work=work, stream=stream)


def moda_pack_depth_q8(k_depth: torch.Tensor, v_depth: torch.Tensor, stream=None, out=None):
    """8-bit packed depth KV: returns (k_q, v_q int8 flat buffers of
    depth_packed_elems(...) codes, k_scale, v_scale float32 [elems / d]),
    written into `out` (such a tuple) when it is given."""
    if k_depth.dim() != 5 or v_depth.shape != k_depth.shape or v_depth.dtype != k_depth.dtype:
        raise ValueError("k_depth / v_depth must both be [B,T,L_d,Hkv,d] of one dtype")
    B, T, L_d, Hkv, d = k_depth.shape
    n = depth_packed_elems(B, T, Hkv, d, L_d)
    dev = k_depth.device
    if out is not None:
        if len(out) != 4:
            raise ValueError("out must be (k_q, v_q, k_scale, v_scale)")
        _check_q8(out, B, T, Hkv, d, L_d)
        kq, vq, ks, vs = out
    else:
        kq = torch.empty(n, dtype=torch.int8, device=dev)
        vq = torch.empty(n, dtype=torch.int8, device=dev)
        ks = torch.empty(n // d, dtype=torch.float32, device=dev)
        vs = torch.empty(n // d, dtype=torch.float32, device=dev)
    if L_d == 0:
        return kq, vq, ks, vs
    for t, name in ((k_depth, "k_depth"), (v_depth, "v_depth")):
        _dev(t, name)
    dev = _one_device(k_depth, v_depth, kq, vq, ks, vs)
    st = _call(dev, "moda_pack_depth_q8", stream,
        k_depth.data_ptr(), v_depth.data_ptr(), kq.data_ptr(), vq.data_ptr(),
        ks.data_ptr(), vs.data_ptr(), B, T, Hkv, d, L_d,
        _dtype_code(k_depth))
    check(st, "moda_pack_depth_q8")
    return kq, vq, ks, vs


def _check_q8(packed_q8, B, T, Hkv, d, L_cap):
    kq, vq, ks, vs = packed_q8
    n = depth_packed_elems(B, T, Hkv, d, L_cap)
    for t, name, dt, cnt in ((kq, "k_q", torch.int8, n), (vq, "v_q", torch.int8, n),
                             (ks, "k_scale", torch.float32, n // d), (vs, "v_scale", torch.float32, n // d)):
        _dev(t, name)
        if t.dtype != dt or t.numel() != cnt:
            raise ValueError(f"{name} must hold {cnt} elements of {dt}")
    return [kq.data_ptr(), vq.data_ptr(), ks.data_ptr(), vs.data_ptr()]


def moda_append_depth_q8(k_new: torch.Tensor, v_new: torch.Tensor, packed_q8, L_cap: int, slot: int,
                         stream=None):
    """Write step into 8-bit packed buffers (the four of moda_pack_depth_q8
    built with L_cap slots per position), in place."""
    if k_new.dim() != 4 or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must both be [B,T,Hkv,d] of one dtype")
    B, T, Hkv, d = k_new.shape
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, name)
    ptrs = _check_q8(packed_q8, B, T, Hkv, d, L_cap)
    dev = _one_device(k_new, v_new, *packed_q8)
    st = _call(dev, "moda_append_depth_q8", stream,
        k_new.data_ptr(), v_new.data_ptr(), *ptrs, B, T, Hkv, d, L_cap, slot,
        _dtype_code(k_new))
    check(st, "moda_append_depth_q8")
    return packed_q8


def moda_fwd_window_q8(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor, packed_q8,
                       L_cap: int, slot_lo: int, slot_hi: int,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       with_lse: bool = True, stream=None):
    """MoDA forward over depth slots [slot_lo, slot_hi) of 8-bit packed
    buffers with L_cap slots per position."""
    if q.dim() != 4 or k_seq.dim() != 4 or v_seq.shape != k_seq.shape:
        raise ValueError("q must be [B,T,Hq,d], k_seq / v_seq [B,T,Hkv,d]")
    B, T, Hq, d = q.shape
    Hkv = k_seq.shape[2]
    if k_seq.shape[:2] != (B, T) or k_seq.shape[3] != d:
        raise ValueError("k_seq shape does not match q")
    if k_seq.dtype != q.dtype or v_seq.dtype != q.dtype:
        raise ValueError("q, k_seq, v_seq must share one dtype")
    for t, name in ((q, "q"), (k_seq, "k_seq"), (v_seq, "v_seq")):
        _dev(t, name)
    ptrs = _check_q8(packed_q8, B, T, Hkv, d, L_cap) if slot_hi > slot_lo else [None] * 4
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have the shape and dtype of q")
    if with_lse and lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse")
        if lse.dtype != torch.float32 or lse.shape != (B, Hq, T):
            raise ValueError("lse must be float32 [B,Hq,T]")
    dev = _one_device(q, k_seq, v_seq, *(packed_q8 if slot_hi > slot_lo else ()), out, lse)
    st = _call(dev, "moda_fwd_window_q8", stream,
        q.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(), *ptrs, out.data_ptr(),
        lse.data_ptr() if lse is not None else None, B, T, Hq, Hkv, d, L_cap,
        slot_lo, slot_hi, _dtype_code(q))
    check(st, "moda_fwd_window_q8")
    return out, lse


def moda_fwd_q8(q: torch.Tensor, k_seq: torch.Tensor, v_seq: torch.Tensor, packed_q8, L_d: int,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                with_lse: bool = True, stream=None):
    """MoDA forward over 8-bit depth KV (the four buffers of moda_pack_depth_q8)."""
    return moda_fwd_window_q8(q, k_seq, v_seq, packed_q8, L_d, 0, L_d, out=out, lse=lse,
                              with_lse=with_lse, stream=stream)
