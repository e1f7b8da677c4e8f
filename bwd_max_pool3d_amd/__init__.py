"""3-D max pooling over NCDHW tensors on AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of libmp3d.so (include/mp3d.h), with the same
names.  PyTorch supplies device memory and the current stream; every step
of the computation runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: if the library is missing every call raises ImportError.

  mp3d_forward(x, kernel, stride) -> (y, idx)        fixed windows, no padding
  amp3d_forward(x, out_size) -> (y, idx)             adaptive windows
      (indices=False: y only, no index written)
  mp3d_backward(gy, idx, in_shape, kernel=None, stride=None, overlap=-1) -> gx
      (overlap=2: ordered, bit-reproducible sums)
  mp3d_out_size(X, k, s) -> int
  mp3d_forward_ex(x, kernel, stride, padding, dilation, ceil_mode, index_dtype)
      -> (y, idx)                                    padding / dilation / ceil mode,
                                                     int32 or int64 idx
  mp3d_backward_ex(gy, idx, in_shape, kernel, stride, padding, dilation) -> gx
  mp3d_out_size_ex(X, k, s, pad, dilation, ceil_mode) -> int
  mp3d_backward_recompute(x, y, gy, kernel, stride, padding, dilation) -> gx
      index-free backward: the argmax recomputed from x and y

x, y, gy and gx are float32, float16, bfloat16 or float64; idx is int32 (int64 on
request: index_dtype=torch.int64), flat within each D*H*W plane.

The names of the three-call sketch are kept as aliases:
  max_pool3d(x, kernel, stride) = mp3d_forward,
  adaptive_max_pool3d(x, out_size) = amp3d_forward,
  max_pool3d_backward(gy, idx, in_shape, ..., overlap=None) = mp3d_backward
      (overlap None: the library picks; False: the gather; True: accumulate).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import Mp3dError  # noqa: F401

__all__ = ["mp3d_forward", "amp3d_forward", "mp3d_backward", "mp3d_out_size",
           "mp3d_forward_ex", "mp3d_backward_ex", "mp3d_out_size_ex",
           "mp3d_backward_recompute", "recompute_workspace_size",
           "mp3d_backward_workspace_bytes", "mp3d_time_next_call", "Mp3dError",
           "max_pool3d", "adaptive_max_pool3d", "max_pool3d_backward"]

_IDX = {torch.int32: _lib.MP3D_IDX_I32, torch.int64: _lib.MP3D_IDX_I64}

_DTYPE = {torch.float32: _lib.MP3D_F32, torch.float16: _lib.MP3D_F16,
          torch.bfloat16: _lib.MP3D_BF16, torch.float64: _lib.MP3D_F64}


def _triple(v) -> tuple[int, int, int]:
    if isinstance(v, int):
        return (v, v, v)
    v = tuple(int(a) for a in v)
    if len(v) != 3:
        raise ValueError("expected 3 values, got %r" % (v,))
    return v


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s" % t.dtype) from None


def _check_tensor(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous NCDHW" % name)
    if t.dim() != 5:
        raise ValueError("%s must be 5-D (N, C, D, H, W)" % name)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def mp3d_out_size(X: int, k: int, s: int) -> int:
    """(X - k) // s + 1, as the library computes it."""
    out = ctypes.c_int64()
    _lib.check(_lib.load().mp3d_out_size(X, k, s, ctypes.byref(out)))
    return out.value


def _outputs(x: torch.Tensor, shape, out, indices: bool, idx_dtype=torch.int32):
    if not indices:
        if out is None:
            return torch.empty(shape, dtype=x.dtype, device=x.device), None
        _check_tensor(out, "y")
        if tuple(out.shape) != shape or out.dtype != x.dtype:
            raise ValueError("out must be y of shape %s, dtype %s" % (shape, x.dtype))
        return out, None
    if out is None:
        return (torch.empty(shape, dtype=x.dtype, device=x.device),
                torch.empty(shape, dtype=idx_dtype, device=x.device))
    y, idx = out
    _check_tensor(y, "y")
    _check_tensor(idx, "idx")
    if (tuple(y.shape) != shape or tuple(idx.shape) != shape or y.dtype != x.dtype
            or idx.dtype != idx_dtype):
        raise ValueError("out must be (y, idx) of shape %s, dtypes (%s, %s)" % (
            shape, x.dtype, idx_dtype))
    return y, idx


def mp3d_forward(x: torch.Tensor, kernel, stride=None, out=None, indices: bool = True,
                 index_dtype=torch.int32):
    """Fixed-window forward: returns (y, idx), or y alone when ``indices``
    is False (no index is computed into memory).  ``out`` may supply a
    preallocated (y, idx) pair, or y.  ``index_dtype`` torch.int64 gives
    torch-style int64 indices (through mp3d_forward_ex)."""
    if index_dtype != torch.int32:
        return mp3d_forward_ex(x, kernel, stride, out=out, indices=indices,
                               index_dtype=index_dtype)
    lib = _lib.load()
    _check_tensor(x, "x")
    k = _triple(kernel)
    s = _triple(stride if stride is not None else kernel)
    N, C, D, H, W = x.shape
    o = tuple(mp3d_out_size(X, ka, sa) for X, ka, sa in zip((D, H, W), k, s))
    y, idx = _outputs(x, (N, C) + o, out, indices)
    _lib.check(lib.mp3d_forward(x.data_ptr(), y.data_ptr(), idx.data_ptr() if indices else None,
                                _code(x), N, C, D, H, W, *k, *s, _stream(x)))
    return (y, idx) if indices else y


def amp3d_forward(x: torch.Tensor, out_size, out=None, indices: bool = True,
                  index_dtype=torch.int32):
    """Adaptive-window forward: returns (y, idx), or y alone when
    ``indices`` is False.  ``out`` may supply a preallocated (y, idx) pair,
    or y.  ``index_dtype`` torch.int64 gives int64 indices."""
    lib = _lib.load()
    _check_tensor(x, "x")
    o = _triple(out_size)
    N, C, D, H, W = x.shape
    if index_dtype != torch.int32:
        if index_dtype not in _IDX:
            raise TypeError("index_dtype must be torch.int32 or torch.int64")
        y, idx = _outputs(x, (N, C) + o, out, indices, index_dtype)
        zero = _arr3((0, 0, 0))
        _lib.check(lib.mp3d_forward_ex(x.data_ptr(), y.data_ptr(),
                                       idx.data_ptr() if indices else None, _code(x),
                                       _IDX[index_dtype], N, C, D, H, W, *o, zero, zero, zero,
                                       _arr3((1, 1, 1)), _stream(x)))
        return (y, idx) if indices else y
    y, idx = _outputs(x, (N, C) + o, out, indices)
    _lib.check(lib.amp3d_forward(x.data_ptr(), y.data_ptr(), idx.data_ptr() if indices else None,
                                 _code(x), N, C, D, H, W, *o, _stream(x)))
    return (y, idx) if indices else y


def mp3d_backward(gy: torch.Tensor, idx: torch.Tensor, in_shape, kernel=None,
                  stride=None, overlap: int = -1, out: torch.Tensor | None = None):
    """Backward: gx of shape ``in_shape``.  ``kernel``/``stride`` None means
    adaptive windows; ``overlap`` -1 lets the library pick the gather path
    when the windows tile every axis, 0 forces it, 1 forces accumulation,
    2 asks for the ordered backward (each gx element the ascending-order
    binary32 sum, the same bits on every run).  ``out`` may supply a
    preallocated gx."""
    lib = _lib.load()
    _check_tensor(gy, "gy")
    _check_tensor(idx, "idx")
    if idx.dtype not in _IDX:
        raise TypeError("idx must be int32 or int64")
    if idx.shape != gy.shape or idx.device != gy.device:
        raise ValueError("idx and gy must have the same shape and device")
    N, C, D, H, W = (int(v) for v in in_shape)
    if gy.shape[:2] != (N, C):
        raise ValueError("gy's N, C do not match in_shape")
    if kernel is None:
        k = s = (0, 0, 0)
    else:
        k = _triple(kernel)
        s = _triple(stride if stride is not None else kernel)
    if idx.dtype == torch.int64:
        return mp3d_backward_ex(gy, idx, in_shape, k, s, 0, 1, overlap=overlap, out=out)
    if out is None:
        out = torch.empty((N, C, D, H, W), dtype=gy.dtype, device=gy.device)
    else:
        _check_tensor(out, "out")
        if out.shape != (N, C, D, H, W) or out.dtype != gy.dtype:
            raise ValueError("out must be a %s tensor of shape %s" % (gy.dtype, (N, C, D, H, W)))
    od, oh, ow = gy.shape[2:]
    _lib.check(lib.mp3d_backward(gy.data_ptr(), idx.data_ptr(), out.data_ptr(), _code(gy),
                                 N, C, D, H, W, od, oh, ow, *k, *s, int(overlap), _stream(gy)))
    return out


def mp3d_out_size_ex(X: int, k: int, s: int, pad: int = 0, dilation: int = 1,
                     ceil_mode: bool = False) -> int:
    """Output extent of a fixed axis with padding, dilation and ceil mode,
    as the library computes it."""
    out = ctypes.c_int64()
    _lib.check(_lib.load().mp3d_out_size_ex(X, k, s, pad, dilation, int(bool(ceil_mode)),
                                            ctypes.byref(out)))
    return out.value


def _arr3(v):
    return (ctypes.c_int32 * 3)(*v)


def mp3d_forward_ex(x: torch.Tensor, kernel, stride=None, padding=0, dilation=1,
                    ceil_mode: bool = False, index_dtype=torch.int32, out=None,
                    indices: bool = True):
    """Fixed-window forward with padding, dilation and ceil mode, and int32
    or int64 indices: returns (y, idx), or y alone when ``indices`` is
    False.  ``out`` may supply a preallocated (y, idx) pair, or y."""
    lib = _lib.load()
    _check_tensor(x, "x")
    if index_dtype not in _IDX:
        raise TypeError("index_dtype must be torch.int32 or torch.int64")
    k = _triple(kernel)
    s = _triple(stride if stride is not None else kernel)
    pd, dl = _triple(padding), _triple(dilation)
    N, C, D, H, W = x.shape
    o = tuple(mp3d_out_size_ex(X, *a, ceil_mode=ceil_mode)
              for X, a in zip((D, H, W), zip(k, s, pd, dl)))
    y, idx = _outputs(x, (N, C) + o, out, indices, index_dtype)
    _lib.check(lib.mp3d_forward_ex(x.data_ptr(), y.data_ptr(), idx.data_ptr() if indices else None,
                                   _code(x), _IDX[index_dtype], N, C, D, H, W, *o, _arr3(k),
                                   _arr3(s), _arr3(pd), _arr3(dl), _stream(x)))
    return (y, idx) if indices else y


def mp3d_backward_ex(gy: torch.Tensor, idx: torch.Tensor, in_shape, kernel, stride=None,
                     padding=0, dilation=1, overlap: int = -1, out: torch.Tensor | None = None):
    """Backward for mp3d_forward_ex: gx of shape ``in_shape`` from gy and
    idx (int32 or int64).  The ceil mode is read from gy's extents.
    ``overlap`` as for mp3d_backward."""
    lib = _lib.load()
    _check_tensor(gy, "gy")
    _check_tensor(idx, "idx")
    if idx.dtype not in _IDX:
        raise TypeError("idx must be int32 or int64")
    if idx.shape != gy.shape or idx.device != gy.device:
        raise ValueError("idx and gy must have the same shape and device")
    N, C, D, H, W = (int(v) for v in in_shape)
    if gy.shape[:2] != (N, C):
        raise ValueError("gy's N, C do not match in_shape")
    k = _triple(kernel)
    s = _triple(stride if stride is not None else kernel)
    pd, dl = _triple(padding), _triple(dilation)
    if out is None:
        out = torch.empty((N, C, D, H, W), dtype=gy.dtype, device=gy.device)
    else:
        _check_tensor(out, "out")
        if out.shape != (N, C, D, H, W) or out.dtype != gy.dtype:
            raise ValueError("out must be a %s tensor of shape %s" % (gy.dtype, (N, C, D, H, W)))
    od, oh, ow = gy.shape[2:]
    _lib.check(lib.mp3d_backward_ex(gy.data_ptr(), idx.data_ptr(), out.data_ptr(), _code(gy),
                                    _IDX[idx.dtype], N, C, D, H, W, od, oh, ow, _arr3(k),
                                    _arr3(s), _arr3(pd), _arr3(dl), int(overlap), _stream(gy)))
    return out


def mp3d_backward_workspace_bytes(dtype: torch.dtype, index_dtype, N: int, C: int,
                                  out_size) -> int:
    """Workspace bytes of a backward: 0 with an index array (index_dtype
    torch.int32 or torch.int64), the two-pass size for the index-free
    backward (index_dtype None)."""
    it = _lib.MP3D_IDX_NONE if index_dtype is None else _IDX[index_dtype]
    nbytes = ctypes.c_size_t()
    _lib.check(_lib.load().mp3d_backward_workspace_bytes(_DTYPE[dtype], it, N, C,
                                                         *_triple(out_size),
                                                         ctypes.byref(nbytes)))
    return nbytes.value


def mp3d_time_next_call(start_event: int | None, stop_event: int | None) -> None:
    """Arms kernel-time events (raw hipEvent_t handles) for the next call on
    this thread: the start of its first kernel and the end of its last.
    None, None disarms."""
    _lib.check(_lib.load().mp3d_time_next_call(start_event, stop_event))


def recompute_workspace_size(dtype: torch.dtype, N: int, C: int, out_size) -> int:
    """Bytes of workspace the two-pass index-free backward needs."""
    nbytes = ctypes.c_size_t()
    _lib.check(_lib.load().mp3d_recompute_workspace_size(_DTYPE[dtype], N, C,
                                                         *_triple(out_size),
                                                         ctypes.byref(nbytes)))
    return nbytes.value


def mp3d_backward_recompute(x: torch.Tensor, y: torch.Tensor, gy: torch.Tensor, kernel=None,
                            stride=None, padding=0, dilation=1, overlap: int = -1,
                            out: torch.Tensor | None = None, workspace=None):
    """Index-free backward: gx of x's shape, with each window's argmax
    recomputed from the forward's input ``x`` and output ``y`` (the first
    element of the window equal to y, the first NaN when y is NaN).
    ``kernel`` None means adaptive windows (y's extents); ``overlap`` as for
    mp3d_backward (2: ordered).  ``workspace``: None for the one-pass
    kernels; a contiguous uint8 device tensor of at least
    recompute_workspace_size(...) bytes, or True to allocate one, for the
    two-pass form (the forward into the workspace, its argmax checked
    against y)."""
    lib = _lib.load()
    for t, n in ((x, "x"), (y, "y"), (gy, "gy")):
        _check_tensor(t, n)
    if not (x.dtype == y.dtype == gy.dtype) or y.shape != gy.shape:
        raise ValueError("x, y and gy must share a dtype, and y and gy a shape")
    if x.shape[:2] != y.shape[:2] or x.device != y.device or x.device != gy.device:
        raise ValueError("x, y and gy must share N, C and device")
    N, C, D, H, W = x.shape
    if kernel is None:
        k = s = pd = (0, 0, 0)
        dl = (1, 1, 1)
    else:
        k = _triple(kernel)
        s = _triple(stride if stride is not None else kernel)
        pd, dl = _triple(padding), _triple(dilation)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_tensor(out, "out")
        if out.shape != x.shape or out.dtype != x.dtype:
            raise ValueError("out must match x")
    od, oh, ow = gy.shape[2:]
    if workspace is None or workspace is False:
        _lib.check(lib.mp3d_backward_recompute(x.data_ptr(), y.data_ptr(), gy.data_ptr(),
                                               out.data_ptr(), _code(gy), N, C, D, H, W, od, oh,
                                               ow, _arr3(k), _arr3(s), _arr3(pd), _arr3(dl),
                                               int(overlap), _stream(gy)))
        return out
    if workspace is True:
        workspace = torch.empty(recompute_workspace_size(x.dtype, N, C, (od, oh, ow)),
                                dtype=torch.uint8, device=x.device)
    if (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8
            or not workspace.is_cuda or not workspace.is_contiguous()
            or workspace.device != x.device):
        raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
    _lib.check(lib.mp3d_backward_recompute_ws(x.data_ptr(), y.data_ptr(), gy.data_ptr(),
                                              out.data_ptr(), _code(gy), N, C, D, H, W, od, oh,
                                              ow, _arr3(k), _arr3(s), _arr3(pd), _arr3(dl),
                                              int(overlap), workspace.data_ptr(),
                                              workspace.numel(), _stream(gy)))
    return out


def overlap_code(overlap) -> int:
    """The C ABI's overlap argument for the sketch's ``overlap``: None lets
    the library choose (-1), False asks for the gather (0), True for the
    accumulate path (1); an int is passed through (2: ordered)."""
    return -1 if overlap is None else int(overlap)


def max_pool3d(x: torch.Tensor, kernel, stride=None, out=None, indices: bool = True):
    """Alias of mp3d_forward under the sketch's name."""
    return mp3d_forward(x, kernel, stride, out=out, indices=indices)


def adaptive_max_pool3d(x: torch.Tensor, out_size, out=None, indices: bool = True):
    """Alias of amp3d_forward under the sketch's name."""
    return amp3d_forward(x, out_size, out=out, indices=indices)


def max_pool3d_backward(gy: torch.Tensor, idx: torch.Tensor, in_shape, kernel=None, stride=None,
                        overlap=None, out: torch.Tensor | None = None):
    """Alias of mp3d_backward under the sketch's name; ``overlap`` None,
    False or True (or the C ABI's integer codes)."""
    return mp3d_backward(gy, idx, in_shape, kernel, stride, overlap=overlap_code(overlap), out=out)
