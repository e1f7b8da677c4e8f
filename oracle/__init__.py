"""CPU oracle for 3-D max pooling: forward window max + int32 argmax (and,
for padded / dilated windows, int64 argmax), and the backward that routes
each output gradient to its argmax.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its Python binding) never imports or calls it, and the
two share no code: the oracle is plain C in ``mp3d_oracle.c`` (compiled with
gcc) driven through ctypes with numpy arrays.

Storage convention: float32 and float64 data are numpy float32 / float64
arrays; float16 and bfloat16 data are numpy uint16 arrays holding the raw
bit patterns.  dtype codes: 0 = float32, 1 = float16, 2 = bfloat16,
3 = float64.

The definitions followed (page titles and sections) are stated at the top
of ``mp3d_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, F16, BF16, F64 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mp3d_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_vp)


class Oracle:
    """ctypes front end over one compiled copy of ``mp3d_oracle.c``."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = LIBRARY
            if (not os.path.exists(path)
                    or os.path.getmtime(path) < os.path.getmtime(SOURCE)):
                build()
        lib = ctypes.CDLL(path)
        lib.oracle_window.argtypes = [_i64] * 5 + [ctypes.POINTER(_i64)] * 2
        lib.oracle_window.restype = None
        lib.oracle_fixed_out.argtypes = [_i64] * 3
        lib.oracle_fixed_out.restype = _i64
        lib.oracle_forward.argtypes = [_vp, _vp, _vp, ctypes.c_int] + [_i64] * 7 + [_vp, _vp]
        lib.oracle_forward.restype = None
        lib.oracle_fixed_out_ex.argtypes = [_i64] * 5 + [ctypes.c_int]
        lib.oracle_fixed_out_ex.restype = _i64
        lib.oracle_forward_ex.argtypes = ([_vp, _vp, _vp, ctypes.c_int] + [_i64] * 7
                                          + [_vp] * 4)
        lib.oracle_forward_ex.restype = None
        lib.oracle_argmax_from_output.argtypes = ([_vp, _vp, _vp, ctypes.c_int] + [_i64] * 7
                                                  + [_vp] * 4)
        lib.oracle_argmax_from_output.restype = None
        lib.oracle_backward.argtypes = [_vp, _vp, _vp, ctypes.c_int] + [_i64] * 7 + [_vp] * 4
        lib.oracle_backward.restype = None
        lib.oracle_widen_array.argtypes = [_vp, ctypes.c_int, _i64, _vp]
        lib.oracle_round_array.argtypes = [_vp, ctypes.c_int, _i64, _vp]
        self.lib = lib
        self.path = path

    # -- windows -------------------------------------------------------
    def window(self, X: int, O: int, k: int, s: int, o: int) -> tuple[int, int]:
        a, b = _i64(), _i64()
        self.lib.oracle_window(X, O, k, s, o, ctypes.byref(a), ctypes.byref(b))
        return a.value, b.value

    def fixed_out(self, X: int, k: int, s: int) -> int:
        return self.lib.oracle_fixed_out(X, k, s)

    def fixed_out_ex(self, X: int, k: int, s: int, pad: int = 0, dil: int = 1,
                     ceil_mode: bool = False) -> int:
        return self.lib.oracle_fixed_out_ex(X, k, s, pad, dil, int(bool(ceil_mode)))

    # -- conversions ---------------------------------------------------
    def widen(self, bits: np.ndarray, dtype: int) -> np.ndarray:
        src = np.ascontiguousarray(bits)
        out = np.empty(src.size, np.float64)
        self.lib.oracle_widen_array(_ptr(src), dtype, src.size, _ptr(out))
        return out.reshape(src.shape)

    def round16(self, f32: np.ndarray, dtype: int) -> np.ndarray:
        src = np.ascontiguousarray(f32, dtype=np.float32)
        out = np.empty(src.size, np.uint16)
        self.lib.oracle_round_array(_ptr(src), dtype, src.size, _ptr(out))
        return out.reshape(src.shape)

    # -- pooling -------------------------------------------------------
    @staticmethod
    def _check(x: np.ndarray, dtype: int):
        want = {F32: np.float32, F64: np.float64}.get(dtype, np.uint16)
        if x.dtype != want or not x.flags.c_contiguous:
            raise TypeError("oracle expects contiguous %s storage" % np.dtype(want))

    def forward(self, x: np.ndarray, dtype: int, out: tuple[int, int, int],
                k=(0, 0, 0), s=(0, 0, 0)):
        """x: (N, C, D, H, W) storage array.  out: (OD, OH, OW).  k/s per
        axis; an axis with k == 0 uses adaptive windows.  Returns (y, idx)."""
        self._check(x, dtype)
        N, C, D, H, W = x.shape
        OD, OH, OW = out
        y = np.empty((N, C, OD, OH, OW), x.dtype)
        idx = np.empty((N, C, OD, OH, OW), np.int32)
        k64 = np.asarray(k, np.int64)
        s64 = np.asarray(s, np.int64)
        self.lib.oracle_forward(_ptr(x), _ptr(y), _ptr(idx), dtype, N * C,
                                D, H, W, OD, OH, OW, _ptr(k64), _ptr(s64))
        return y, idx

    def forward_ex(self, x: np.ndarray, dtype: int, out: tuple[int, int, int],
                   k, s, pad=(0, 0, 0), dil=(1, 1, 1)):
        """Forward with padding and dilation; an axis with k == 0 uses
        adaptive windows.  Returns (y, idx) with idx int64 (-1 where a
        window has no tap inside the input)."""
        self._check(x, dtype)
        N, C, D, H, W = x.shape
        OD, OH, OW = out
        y = np.empty((N, C, OD, OH, OW), x.dtype)
        idx = np.empty((N, C, OD, OH, OW), np.int64)
        arrs = [np.asarray(v, np.int64) for v in (k, s, pad, dil)]
        self.lib.oracle_forward_ex(_ptr(x), _ptr(y), _ptr(idx), dtype, N * C,
                                   D, H, W, OD, OH, OW, *[_ptr(a) for a in arrs])
        return y, idx

    def argmax_from_output(self, x: np.ndarray, y: np.ndarray, dtype: int, k=(0, 0, 0),
                           s=(0, 0, 0), pad=(0, 0, 0), dil=(1, 1, 1)):
        """The first tap of each window equal to y (the first NaN when y is
        NaN), int64, -1 where none is; geometry as forward_ex, with the
        output extents taken from y."""
        self._check(x, dtype)
        self._check(y, dtype)
        N, C, D, H, W = x.shape
        OD, OH, OW = y.shape[2:]
        idx = np.empty(y.shape, np.int64)
        arrs = [np.asarray(v, np.int64) for v in (k, s, pad, dil)]
        self.lib.oracle_argmax_from_output(_ptr(x), _ptr(y), _ptr(idx), dtype, N * C,
                                           D, H, W, OD, OH, OW, *[_ptr(a) for a in arrs])
        return idx

    def backward(self, gy: np.ndarray, idx: np.ndarray, dtype: int,
                 in_shape: tuple[int, int, int, int, int], side: bool = True):
        """Returns a dict with gx (storage array), acc32, and when ``side``
        also ref64, abs64 and count, each shaped like the input."""
        self._check(gy, dtype)
        idx = np.ascontiguousarray(idx, np.int32)
        N, C, D, H, W = in_shape
        OD, OH, OW = gy.shape[2:]
        gx = np.empty(in_shape, gy.dtype)
        acc = np.empty(in_shape, np.float32)
        ref = np.empty(in_shape, np.float64) if side else None
        ab = np.empty(in_shape, np.float64) if side else None
        cnt = np.empty(in_shape, np.int32) if side else None
        self.lib.oracle_backward(_ptr(gy), _ptr(idx), _ptr(gx), dtype, N * C,
                                 D, H, W, OD, OH, OW, _ptr(acc), _ptr(ref),
                                 _ptr(ab), _ptr(cnt))
        res = {"gx": gx, "acc32": acc}
        if side:
            res.update(ref64=ref, abs64=ab, count=cnt)
        return res


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
