"""Seeded random geometries through the C ABI, against the oracle.

Each case draws, per axis, either adaptive windows or fixed windows with
their own kernel, stride, padding, dilation and rounding of the output
extent (floor or ceil), so that axes mix forms the hand-picked cases keep
apart; then a dtype, an index type, small N and C, and whether the
small-tensor kernels may run.  A share of the cases give every axis the
same kernel (2 or 3) and stride 2, with padding and rounding still drawn
per axis.  On each case: the forward (indices and
values only) must equal the oracle's y bits and idx; the backward from idx
(library's pick, accumulate, ordered) and the index-free backward (any
order, ordered; one-pass and through a workspace) must meet the bar of
the hand-picked cases.  The windows
follow the definitions of "Struct Maxpool3dForward" (teenygrad,
description) and the PR #308 page (Summary); padding, dilation and ceil
rounding follow the pooling output-size rule the oracle pins to torch.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import _gpu
import _pins
import bwd_max_pool3d_amd as mp
from bwd_max_pool3d_amd import _lib

N_CASES = 240
DTYPES = [torch.float32, torch.float16, torch.bfloat16, torch.float64]
KINDS = ["normal", "sparse_nan", "special", "zeros"]


def _axis(orc, rng, X):
    """One axis: (X, O, k, s, pad, dil); k == s == 0 is adaptive."""
    if rng.random() < 0.25:
        return X, int(rng.integers(1, min(2 * X, 30) + 1)), 0, 0, 0, 1
    k = int(rng.integers(1, 6))
    s = int(rng.integers(1, 5))
    dil = int(rng.choice([1, 1, 1, 2, 3]))
    pad = int(rng.integers(0, k // 2 + 1))
    X = max(X, (k - 1) * dil + 1 - 2 * pad)
    O = orc.fixed_out_ex(X, k, s, pad, dil, bool(rng.random() < 0.35))
    return X, O, k, s, pad, dil


def _cube_axis(orc, rng, X, k):
    """A fixed axis of the shared kernel k and stride 2, padding 0 or 1 and
    either rounding: the forms the row-vector kernel takes."""
    pad = int(rng.integers(0, 2))
    X = max(X, k - 2 * pad)
    return X, orc.fixed_out_ex(X, k, 2, pad, 1, bool(rng.random() < 0.5)), k, 2, pad, 1


def _case(orc, i):
    rng = np.random.default_rng(7000 + i)
    D = int(rng.integers(1, 20))
    H = int(rng.integers(1, 20))
    W = int(rng.choice([8, 16, 24, 40, 64, 72])) if rng.random() < 0.5 else int(rng.integers(1, 50))
    if rng.random() < 0.3:
        k = int(rng.choice([2, 3]))
        axes = [_cube_axis(orc, rng, X, k) for X in (D, H, W)]
    else:
        axes = [_axis(orc, rng, X) for X in (D, H, W)]
    return dict(
        shape=(int(rng.integers(1, 3)), int(rng.integers(1, 4))) + tuple(a[0] for a in axes),
        out=tuple(a[1] for a in axes),
        geo=tuple(tuple(a[j] for a in axes) for j in range(2, 6)),
        dtype=DTYPES[int(rng.integers(0, 4))],
        idx=torch.int64 if rng.random() < 0.3 else torch.int32,
        small=bool(rng.random() < 0.7),
        kind=KINDS[int(rng.integers(0, len(KINDS)))],
        seed=9000 + 16 * i,
    )


def _a3(v):
    return (ctypes.c_int32 * 3)(*v)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _forward(x, c, indices):
    lib = _lib.load()
    y = torch.empty(c["shape"][:2] + c["out"], dtype=x.dtype, device=x.device)
    idx = torch.empty(y.shape, dtype=c["idx"], device=x.device) if indices else None
    k, s, p, d = c["geo"]
    _lib.check(lib.mp3d_forward_ex(x.data_ptr(), y.data_ptr(), idx.data_ptr() if indices else None,
                                   _gpu.CODE[x.dtype], mp._IDX[c["idx"]], *c["shape"], *c["out"],
                                   _a3(k), _a3(s), _a3(p), _a3(d), _stream()))
    return y, idx


def _backward(gy, idx, c, overlap):
    lib = _lib.load()
    gx = torch.empty(c["shape"], dtype=gy.dtype, device=gy.device)
    k, s, p, d = c["geo"]
    _lib.check(lib.mp3d_backward_ex(gy.data_ptr(), idx.data_ptr(), gx.data_ptr(),
                                    _gpu.CODE[gy.dtype], mp._IDX[idx.dtype], *c["shape"],
                                    *c["out"], _a3(k), _a3(s), _a3(p), _a3(d), overlap,
                                    _stream()))
    return gx


def _recompute(x, y, gy, c, overlap, ws=None):
    lib = _lib.load()
    gx = torch.empty_like(x)
    k, s, p, d = c["geo"]
    geo = (_gpu.CODE[gy.dtype],) + c["shape"] + c["out"] + (_a3(k), _a3(s), _a3(p), _a3(d))
    if ws is None:
        _lib.check(lib.mp3d_backward_recompute(x.data_ptr(), y.data_ptr(), gy.data_ptr(),
                                               gx.data_ptr(), *geo, overlap, _stream()))
    else:
        _lib.check(lib.mp3d_backward_recompute_ws(x.data_ptr(), y.data_ptr(), gy.data_ptr(),
                                                  gx.data_ptr(), *geo, overlap, ws.data_ptr(),
                                                  ws.numel(), _stream()))
    return gx


def _name(c):
    k, s, p, d = c["geo"]
    return "shape %s out %s k %s s %s pad %s dil %s %s %s small=%d %s" % (
        c["shape"], c["out"], k, s, p, d, c["dtype"], c["idx"], c["small"], c["kind"])


def test_random_cases_are_varied(orc):
    """The draw reaches every form it is meant to mix (host only)."""
    cs = [_case(orc, i) for i in range(N_CASES)]
    k = np.array([c["geo"][0] for c in cs])
    assert ((k == 0).any(axis=1) & (k != 0).any(axis=1)).any()       # mixed axes
    assert (np.array([c["geo"][2] for c in cs]) > 0).any()            # padding
    assert (np.array([c["geo"][3] for c in cs]) > 1).any()            # dilation
    assert len({c["dtype"] for c in cs}) == 4 and len({c["idx"] for c in cs}) == 2
    ceil = [any(c["geo"][0][a] and c["out"][a] != orc.fixed_out_ex(
        c["shape"][2 + a], *(c["geo"][j][a] for j in range(4)), False) for a in range(3))
        for c in cs]
    assert any(ceil)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: "r%03d" % i)
def test_random_geometry(orc, i, monkeypatch):
    c = _case(orc, i)
    if not c["small"]:
        monkeypatch.setenv("MP3D_SMALL", "0")
    what = _name(c)
    code = _gpu.CODE[c["dtype"]]
    k, s, p, d = c["geo"]
    for j, kind in enumerate(("ties", c["kind"])):
        x = _pins.from_storage(_pins.draw(c["shape"], code, kind, c["seed"] + j), code).cuda()
        y, idx = _forward(x, c, True)
        yo, io = orc.forward_ex(_gpu.storage(x), code, c["out"], k, s, p, d)
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), io), "%s %s: idx" % (what, kind)
        assert np.array_equal(_gpu.storage(y).view(np.uint8), yo.view(np.uint8)), \
            "%s %s: y bits" % (what, kind)
        yv, _ = _forward(x, c, False)
        assert np.array_equal(_gpu.storage(yv).view(np.uint8), yo.view(np.uint8)), \
            "%s %s: values-only y bits" % (what, kind)
    gy = _pins.from_storage(_pins.draw(tuple(y.shape), code, "normal", c["seed"] + 9), code).cuda()
    idx32 = torch.from_numpy(io.astype(np.int32))
    for overlap, exact in ((-1, False), (1, False), (2, True)):
        gx = _backward(gy, idx, c, overlap)
        _gpu.check_backward(orc, gy.cpu(), idx32, c["shape"], gx, exact=exact,
                            what="%s backward overlap=%d" % (what, overlap))
    ia = orc.argmax_from_output(_gpu.storage(x), _gpu.storage(y), code, k, s, p, d)
    assert np.array_equal(ia, io), "%s: argmax from (x, y) differs from the forward's" % what
    ws = torch.empty(mp.recompute_workspace_size(x.dtype, *c["shape"][:2], c["out"]),
                     dtype=torch.uint8, device=x.device)
    monkeypatch.setenv("MP3D_TWO_PASS", "1")       # the two-pass form on these small shapes
    for overlap, exact in ((-1, False), (2, True)):
        for w in (None, ws):
            gx = _recompute(x, y, gy, c, overlap, w)
            _gpu.check_backward(orc, gy.cpu(), idx32, c["shape"], gx, exact=exact,
                                what="%s index-free overlap=%d%s" % (
                                    what, overlap, " workspace" if w is not None else ""))
