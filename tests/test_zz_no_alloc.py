"""The entry point that allocates nothing (mp3d_backward_recompute_static),
called through the C ABI: on two calls in a row, the second with a smaller
input, its results equal those of mp3d_backward_recompute_ws with a
workspace the caller allocated -- bit for bit on the ordered path, and both
within the accumulate path's bar against the oracle otherwise.  The
two-pass form is forced (MP3D_TWO_PASS=1), so that the library's static
scratch is what the forward writes into and the backward reads."""
import ctypes
import os

import pytest
import torch

import _gpu
import _pins
import bwd_max_pool3d_amd as mp
from bwd_max_pool3d_amd import _lib

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, shape, adaptive out or None, kernel, stride): a larger call, then a smaller one
    (torch.float16, (2, 8, 20, 18, 16), None, (3, 3, 3), (2, 2, 2)),
    (torch.bfloat16, (1, 3, 9, 10, 8), (4, 4, 3), None, None),
]


def _a3(v):
    return (ctypes.c_int32 * 3)(*v)


def _geometry(shape, out, k, s):
    if k is None:
        return out, (0, 0, 0), (0, 0, 0)
    o3 = tuple(mp.mp3d_out_size(X, ka, sa) for X, ka, sa in zip(shape[2:], k, s))
    return o3, k, s


def _call(fn, x, y, gy, gx, k, s, overlap, *ws):
    lib = _lib.load()
    N, C, D, H, W = x.shape
    od, oh, ow = gy.shape[2:]
    stream = torch.cuda.current_stream().cuda_stream
    return getattr(lib, fn)(x.data_ptr(), y.data_ptr(), gy.data_ptr(), gx.data_ptr(),
                            _gpu.CODE[x.dtype], N, C, D, H, W, od, oh, ow, _a3(k), _a3(s),
                            _a3((0, 0, 0)), _a3((1, 1, 1)), overlap, *ws, stream)


@pytest.fixture()
def two_pass():
    os.environ["MP3D_TWO_PASS"] = "1"
    yield
    del os.environ["MP3D_TWO_PASS"]


def test_static_scratch_matches_workspace(orc, two_pass):
    for i, (dtype, shape, out, kernel, stride) in enumerate(CASES):
        code = _gpu.CODE[dtype]
        x = _pins.from_storage(_pins.draw(shape, code, "normal", 40 + i), code)
        xd = x.cuda()
        o3, k, s = _geometry(shape, out, kernel, stride)
        if kernel is None:
            y, idx = mp.amp3d_forward(xd, o3)
        else:
            y, idx = mp.mp3d_forward(xd, kernel, stride)
        gy = _pins.from_storage(_pins.draw(tuple(y.shape), code, "normal", 50 + i), code)
        gyd = gy.cuda()
        need = mp.recompute_workspace_size(dtype, shape[0], shape[1], o3)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        for overlap in (2, -1):
            got = torch.full(shape, float("nan"), dtype=dtype, device="cuda")
            ref = torch.full(shape, float("nan"), dtype=dtype, device="cuda")
            assert _call("mp3d_backward_recompute_static", xd, y, gyd, got, k, s,
                         overlap) == _lib.MP3D_OK, _lib.load().mp3d_last_error()
            assert _call("mp3d_backward_recompute_ws", xd, y, gyd, ref, k, s, overlap,
                         ws.data_ptr(), need) == _lib.MP3D_OK, _lib.load().mp3d_last_error()
            torch.cuda.synchronize()
            what = "call %d overlap %d" % (i, overlap)
            if overlap == 2:
                assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), what
            for g in (got, ref):
                _gpu.check_backward(orc, gy, idx.cpu(), shape, g, exact=overlap == 2, what=what)


def test_static_scratch_too_small():
    """A call whose workspace exceeds the static scratch is refused before
    any launch, with its own status and a message naming the sizes."""
    x = torch.zeros((1, 1, 4, 4, 4), dtype=torch.float32, device="cuda")
    y = mp.amp3d_forward(x, (2, 2, 2), indices=False)
    gx = torch.full_like(x, 7.0)
    lib = _lib.load()
    # 4096 x 8192 planes of 2 x 2 x 2 float32 outputs: 1 GiB of workspace;
    # the shape is only described, never touched
    rc = lib.mp3d_backward_recompute_static(x.data_ptr(), y.data_ptr(), y.data_ptr(),
                                            gx.data_ptr(), _lib.MP3D_F32, 4096, 8192, 4, 4, 4,
                                            2, 2, 2, _a3((0, 0, 0)), _a3((0, 0, 0)),
                                            _a3((0, 0, 0)), _a3((1, 1, 1)), -1, None)
    assert rc == _lib.MP3D_EWORKSPACE
    assert "static scratch" in lib.mp3d_last_error().decode()
    torch.cuda.synchronize()
    assert bool((gx == 7.0).all())
