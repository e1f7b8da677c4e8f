"""The C ABI on the host: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented codes
before touching the GPU (none of these calls reaches a HIP API)."""
import ctypes
import os
import re

import pytest

import bwd_max_pool3d_amd as mp
from bwd_max_pool3d_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "mp3d.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for want in ("mp3d_forward", "amp3d_forward", "mp3d_backward"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(_lib.EXPORTS) == set(declared_functions())


def test_out_size():
    assert mp.mp3d_out_size(16, 2, 2) == 8
    assert mp.mp3d_out_size(112, 2, 2) == 56
    assert mp.mp3d_out_size(32, 3, 2) == 15
    assert mp.mp3d_out_size(56, 3, 2) == 27
    assert mp.mp3d_out_size(5, 5, 1) == 1
    for X, k, s in [(2, 3, 1), (5, 0, 1), (5, 2, 0), (5, -1, 1)]:
        with pytest.raises(mp.Mp3dError) as e:
            mp.mp3d_out_size(X, k, s)
        assert e.value.code == _lib.MP3D_EINVAL
    assert _lib.load().mp3d_out_size(5, 2, 2, None) == _lib.MP3D_EINVAL


FAKE = 0x1000   # never dereferenced: every call below fails validation


def fwd(*, x=FAKE, y=FAKE, idx=FAKE, dtype=0, shape=(1, 1, 4, 4, 4), k=(2, 2, 2), s=(2, 2, 2)):
    return _lib.load().mp3d_forward(x, y, idx, dtype, *shape, *k, *s, None)


def afwd(*, x=FAKE, dtype=0, shape=(1, 1, 4, 4, 4), out=(2, 2, 2)):
    return _lib.load().amp3d_forward(x, FAKE, FAKE, dtype, *shape, *out, None)


def bwd(*, gy=FAKE, dtype=0, shape=(1, 1, 4, 4, 4), out=(2, 2, 2), k=(0, 0, 0), s=(0, 0, 0),
        overlap=-1):
    return _lib.load().mp3d_backward(gy, FAKE, FAKE, dtype, *shape, *out, *k, *s, overlap, None)


def _a3(v):
    import ctypes
    return None if v is None else (ctypes.c_int32 * 3)(*v)


def fwdx(*, x=FAKE, dtype=0, it=0, shape=(1, 1, 6, 6, 6), out=(3, 3, 3), k=(3, 3, 3),
         s=(2, 2, 2), p=(1, 1, 1), d=(1, 1, 1)):
    return _lib.load().mp3d_forward_ex(x, FAKE, FAKE, dtype, it, *shape, *out, _a3(k), _a3(s),
                                       _a3(p), _a3(d), None)


def bwdx(*, gy=FAKE, dtype=0, it=0, shape=(1, 1, 6, 6, 6), out=(3, 3, 3), k=(3, 3, 3),
         s=(2, 2, 2), p=(1, 1, 1), d=(1, 1, 1), overlap=-1):
    return _lib.load().mp3d_backward_ex(gy, FAKE, FAKE, dtype, it, *shape, *out, _a3(k), _a3(s),
                                        _a3(p), _a3(d), overlap, None)


def outx(X, k, s, p=0, d=1, ceil=0):
    import ctypes
    v = ctypes.c_int64(-99)
    rc = _lib.load().mp3d_out_size_ex(X, k, s, p, d, ceil, ctypes.byref(v))
    return rc, v.value


@pytest.mark.parametrize("call,code", [
    (lambda: fwdx(it=2), _lib.MP3D_EDTYPE),
    (lambda: fwdx(dtype=4), _lib.MP3D_EDTYPE),
    (lambda: fwdx(x=None), _lib.MP3D_EINVAL),
    (lambda: fwdx(k=None), _lib.MP3D_EINVAL),
    (lambda: fwdx(p=(2, 1, 1)), _lib.MP3D_EINVAL),        # pad > kernel / 2
    (lambda: fwdx(p=(-1, 1, 1)), _lib.MP3D_EINVAL),
    (lambda: fwdx(d=(1, 0, 1)), _lib.MP3D_EINVAL),
    (lambda: fwdx(out=(5, 3, 3)), _lib.MP3D_EINVAL),      # floor 3, ceil 4: (6+2-3)/2 = 2.5
    (lambda: fwdx(out=(2, 3, 3)), _lib.MP3D_EINVAL),
    (lambda: fwdx(shape=(1, 1, 2, 6, 6), out=(1, 3, 3), k=(3, 3, 3), p=(0, 1, 1), d=(2, 1, 1)),
     _lib.MP3D_EINVAL),                                    # span 5 exceeds 2 + 0
    (lambda: fwdx(k=(0, 3, 3), s=(0, 2, 2), p=(1, 1, 1)), _lib.MP3D_EINVAL),  # adaptive with pad
    (lambda: bwdx(overlap=0), _lib.MP3D_ENOTDIV),          # padded windows never take the gather
    (lambda: bwdx(overlap=5), _lib.MP3D_EINVAL),
    (lambda: bwdx(it=-1), _lib.MP3D_EDTYPE),
    (lambda: bwdx(out=(9, 3, 3)), _lib.MP3D_EINVAL),
])
def test_validation_codes_ex(call, code):
    assert call() == code
    assert _lib.load().mp3d_last_error().decode() != ""


def test_out_size_ex():
    assert outx(10, 3, 2, 1) == (0, 5)
    assert outx(10, 3, 2, 1, 1, 1) == (0, 6)
    assert outx(6, 3, 2, 1, 1, 0) == (0, 3)
    assert outx(6, 3, 2, 1, 1, 1) == (0, 4)      # last window starts at 5 < 6 + 1
    assert outx(5, 2, 2, 1, 1, 1) == (0, 3)      # (5+2-2)/2 = 2.5 -> 3 + 1 = 4, but 3*2 >= 5+1
    assert outx(6, 2, 2, 1, 1, 1) == (0, 4)      # (6+2-2)/2 = 3 exactly: 4 windows
    assert outx(4, 2, 3, 1, 1, 1) == (0, 2)
    assert outx(2, 2, 1, 1, 3, 0) == (0, 1)
    assert outx(2, 3, 1, 0, 2, 0)[0] == _lib.MP3D_EINVAL
    assert outx(5, 2, 2, 0, 1, 2)[0] == _lib.MP3D_EINVAL
    assert outx(5, 0, 2)[0] == _lib.MP3D_EINVAL


def test_ex_empty_batch_is_a_no_op():
    assert fwdx(x=None, shape=(0, 2, 6, 6, 6)) == _lib.MP3D_OK
    assert bwdx(gy=None, shape=(3, 0, 6, 6, 6)) == _lib.MP3D_OK


@pytest.mark.parametrize("call,code", [
    (lambda: fwd(dtype=4), _lib.MP3D_EDTYPE),
    (lambda: fwd(dtype=-1), _lib.MP3D_EDTYPE),
    (lambda: fwd(x=None), _lib.MP3D_EINVAL),
    (lambda: fwd(y=None), _lib.MP3D_EINVAL),            # idx NULL is allowed: values only
    (lambda: fwd(k=(0, 2, 2)), _lib.MP3D_EINVAL),
    (lambda: fwd(s=(2, 2, -1)), _lib.MP3D_EINVAL),
    (lambda: fwd(k=(5, 2, 2)), _lib.MP3D_EINVAL),
    (lambda: fwd(shape=(1, 1, 0, 4, 4)), _lib.MP3D_EINVAL),
    (lambda: fwd(shape=(-1, 1, 4, 4, 4)), _lib.MP3D_EINVAL),
    (lambda: fwd(shape=(1, 1, 2048, 1024, 1024)), _lib.MP3D_EOVERFLOW),
    (lambda: fwd(shape=(1 << 40, 1 << 20, 4, 4, 4)), _lib.MP3D_EOVERFLOW),
    (lambda: afwd(out=(0, 2, 2)), _lib.MP3D_EINVAL),
    (lambda: afwd(x=None), _lib.MP3D_EINVAL),
    (lambda: afwd(out=(65536, 65536, 2)), _lib.MP3D_EOVERFLOW),
    (lambda: bwd(overlap=3), _lib.MP3D_EINVAL),
    (lambda: bwd(overlap=-2), _lib.MP3D_EINVAL),
    (lambda: bwd(gy=None), _lib.MP3D_EINVAL),
    (lambda: bwd(shape=(1, 1, 5, 5, 5), overlap=0), _lib.MP3D_ENOTDIV),
    (lambda: bwd(shape=(1, 1, 8, 8, 8), out=(2, 2, 2), k=(3, 3, 3), s=(3, 3, 3), overlap=0),
     _lib.MP3D_ENOTDIV),  # 8 % 2 == 0 but the windows [0,3), [3,6) do not tile
    (lambda: bwd(shape=(1, 1, 6, 6, 6), out=(3, 2, 2), k=(3, 3, 3), s=(3, 3, 3)), _lib.MP3D_EINVAL),
    (lambda: bwd(k=(2, 0, 2), s=(2, 2, 2)), _lib.MP3D_EINVAL),
    (lambda: bwd(dtype=5), _lib.MP3D_EDTYPE),
])
def test_validation_codes(call, code):
    assert call() == code
    assert _lib.load().mp3d_last_error().decode() != ""


def test_empty_batch_is_a_no_op():
    # N*C == 0: nothing to do, even with null pointers
    assert fwd(x=None, y=None, idx=None, shape=(0, 3, 4, 4, 4)) == _lib.MP3D_OK
    assert afwd(x=None, shape=(2, 0, 4, 4, 4)) == _lib.MP3D_OK
    assert bwd(gy=None, shape=(0, 0, 4, 4, 4)) == _lib.MP3D_OK


def test_strerror_covers_every_code():
    lib = _lib.load()
    texts = {lib.mp3d_strerror(c).decode() for c in range(7)}
    assert len(texts) == 7
    assert lib.mp3d_strerror(99).decode() == "unknown status"


def _ws_size(dtype, N, C, out):
    import ctypes
    v = ctypes.c_size_t(0)
    rc = _lib.load().mp3d_recompute_workspace_size(dtype, N, C, *out, ctypes.byref(v))
    return rc, v.value


def test_recompute_workspace_size():
    """The forward's maximum (storage bytes, rounded up to 256) then one
    int32 per output; host arithmetic only."""
    r256 = lambda b: (b + 255) // 256 * 256
    for dtype, es in ((_lib.MP3D_F32, 4), (_lib.MP3D_F16, 2), (_lib.MP3D_BF16, 2),
                      (_lib.MP3D_F64, 8)):
        for N, C, out in ((1, 1, (1, 1, 1)), (2, 3, (5, 7, 7)), (8, 128, (15, 27, 27)),
                          (0, 4, (2, 2, 2))):
            n = N * C * out[0] * out[1] * out[2]
            assert _ws_size(dtype, N, C, out) == (_lib.MP3D_OK, r256(n * es) + 4 * n)
    assert _ws_size(4, 1, 1, (1, 1, 1))[0] == _lib.MP3D_EDTYPE
    assert _ws_size(_lib.MP3D_F32, 1, 1, (0, 1, 1))[0] == _lib.MP3D_EINVAL
    assert _ws_size(_lib.MP3D_F32, -1, 1, (1, 1, 1))[0] == _lib.MP3D_EINVAL
    assert _ws_size(_lib.MP3D_F32, 1 << 40, 1 << 20, (4, 4, 4))[0] == _lib.MP3D_EOVERFLOW


def test_recompute_ws_empty_batch_and_checks():
    """Argument checks of the workspace form before any launch: an empty
    batch is a no-op (null pointers allowed), and a bad overlap or dtype is
    refused."""
    import ctypes
    lib = _lib.load()
    a3 = lambda v: (ctypes.c_int32 * 3)(*v)
    call = lambda dtype=_lib.MP3D_F32, shape=(0, 2, 6, 6, 6), overlap=-1: \
        lib.mp3d_backward_recompute_ws(None, None, None, None, dtype, *shape, 3, 3, 3,
                                       a3((2, 2, 2)), a3((2, 2, 2)), a3((0, 0, 0)),
                                       a3((1, 1, 1)), overlap, None, 0, None)
    assert call() == _lib.MP3D_OK
    assert call(overlap=3) == _lib.MP3D_EINVAL
    assert call(dtype=7) == _lib.MP3D_EDTYPE
    assert call(shape=(1, 2, 6, 6, 6)) == _lib.MP3D_EINVAL      # null tensors


def _bwd_ws(dtype, idx_type, N, C, out):
    v = ctypes.c_size_t(12345)
    rc = _lib.load().mp3d_backward_workspace_bytes(dtype, idx_type, N, C, *out, ctypes.byref(v))
    return rc, v.value


def test_backward_workspace_bytes():
    """The backward's workspace query: none for the index-array paths, the
    two-pass size for the index-free one; host arithmetic only."""
    for dtype in (_lib.MP3D_F32, _lib.MP3D_F16, _lib.MP3D_BF16, _lib.MP3D_F64):
        for N, C, out in ((1, 1, (1, 1, 1)), (8, 128, (15, 27, 27)), (0, 3, (2, 2, 2))):
            for it in (_lib.MP3D_IDX_I32, _lib.MP3D_IDX_I64):
                assert _bwd_ws(dtype, it, N, C, out) == (_lib.MP3D_OK, 0)
            assert _bwd_ws(dtype, _lib.MP3D_IDX_NONE, N, C, out) == _ws_size(dtype, N, C, out)
    assert _bwd_ws(_lib.MP3D_F32, 2, 1, 1, (1, 1, 1))[0] == _lib.MP3D_EDTYPE
    assert _bwd_ws(9, _lib.MP3D_IDX_I32, 1, 1, (1, 1, 1))[0] == _lib.MP3D_EDTYPE
    assert _bwd_ws(_lib.MP3D_F32, _lib.MP3D_IDX_I32, 1, 1, (0, 1, 1))[0] == _lib.MP3D_EINVAL
    assert _bwd_ws(_lib.MP3D_F32, _lib.MP3D_IDX_I32, -1, 1, (1, 1, 1))[0] == _lib.MP3D_EINVAL
    assert _lib.load().mp3d_backward_workspace_bytes(0, 0, 1, 1, 1, 1, 1, None) == _lib.MP3D_EINVAL


def test_time_next_call_arming():
    """The timing hook only stores the caller's events for the next call:
    disarming, and a start event without a stop event, need no GPU."""
    lib = _lib.load()
    assert lib.mp3d_time_next_call(None, None) == _lib.MP3D_OK
    assert lib.mp3d_time_next_call(FAKE, None) == _lib.MP3D_EINVAL
    # a failing call disarms the events it was given (nothing is launched)
    assert lib.mp3d_time_next_call(FAKE, FAKE) == _lib.MP3D_OK
    assert fwd(dtype=9) == _lib.MP3D_EDTYPE
    assert lib.mp3d_time_next_call(None, None) == _lib.MP3D_OK
