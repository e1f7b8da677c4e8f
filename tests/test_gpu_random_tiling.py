"""Seeded random geometries whose windows tile every axis, against the oracle.

With X = q * O on every axis and the windows [o*q, o*q + k) (fixed, k <= q)
or [o*q, (o+1)*q) (adaptive), every input lies in at most one window, so
the backward is the gather of the PR #308 page (Summary: the divisible
case needs no zero pass and no atomics) and must equal the oracle bit for
bit, whichever path the library takes (its pick, the gather forced with
overlap 0, the ordered path).  The draw favours row lengths that are whole
16-byte chunks (the chunk-column gather) and sometimes offsets gy, idx or gx
by one element from their allocation's alignment (the element-wise
fallbacks).  The forward must give the oracle's y bits and idx.
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

N_CASES = 96
DTYPES = [torch.float32, torch.float16, torch.bfloat16, torch.float64]


def _axis(rng, whole_chunks_of=0):
    """(X, O, k, s) of one tiling axis; k == s == 0 is adaptive."""
    q = int(rng.choice([1, 2, 2, 2, 3, 4, 8]))
    O = int(rng.integers(1, 11))
    if whole_chunks_of:
        # X * element size a multiple of 16 bytes
        while (q * O) % whole_chunks_of:
            O += 1
    X = q * O
    if rng.random() < 0.4:
        return X, O, 0, 0
    return X, O, int(rng.integers(1, q + 1)), q


def _case(i):
    rng = np.random.default_rng(11000 + i)
    dtype = DTYPES[int(rng.integers(0, 4))]
    es = torch.empty(0, dtype=dtype).element_size()
    rows16 = rng.random() < 0.7
    axes = [_axis(rng), _axis(rng), _axis(rng, 16 // es if rows16 else 0)]
    return dict(
        shape=(int(rng.integers(1, 3)), int(rng.integers(1, 4))) + tuple(a[0] for a in axes),
        out=tuple(a[1] for a in axes),
        k=tuple(a[2] for a in axes),
        s=tuple(a[3] for a in axes),
        dtype=dtype,
        idx=torch.int64 if rng.random() < 0.25 else torch.int32,
        small=bool(rng.random() < 0.3),
        shift=tuple(bool(rng.random() < 0.15) for _ in range(3)),   # gy, idx, gx
        seed=13000 + 16 * i,
    )


def _a3(v):
    return (ctypes.c_int32 * 3)(*v)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _shifted(shape, dtype, shift):
    """An uninitialised tensor of ``shape``, one element past its
    allocation's start when ``shift``."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 8, dtype=dtype, device="cuda")
    return buf[1:1 + n].view(shape) if shift else buf[:n].view(shape)


def _name(c):
    return "shape %s out %s k %s s %s %s %s small=%d shift=%s" % (
        c["shape"], c["out"], c["k"], c["s"], c["dtype"], c["idx"], c["small"], c["shift"])


def test_tiling_cases_are_varied():
    """The draw reaches what it is meant to (host only): adaptive and fixed
    axes with k < s, every dtype and index type, qd > 2, whole 16-byte rows
    and shifted pointers."""
    cs = [_case(i) for i in range(N_CASES)]
    k = np.array([c["k"] for c in cs])
    s = np.array([c["s"] for c in cs])
    assert (k == 0).any() and ((k > 0) & (k < s)).any()
    assert len({c["dtype"] for c in cs}) == 4 and len({c["idx"] for c in cs}) == 2
    assert any(c["shape"][2] // c["out"][0] > 2 for c in cs)
    assert any((c["shape"][4] * torch.empty(0, dtype=c["dtype"]).element_size()) % 16 == 0
               for c in cs)
    assert any(any(c["shift"]) for c in cs)
    for c in cs:
        for a in range(3):
            X, O = c["shape"][2 + a], c["out"][a]
            assert X % O == 0 and c["k"][a] <= c["s"][a]
            assert c["k"][a] == 0 or c["s"][a] == X // O


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: "t%03d" % i)
def test_random_tiling(orc, i, monkeypatch):
    c = _case(i)
    if not c["small"]:
        monkeypatch.setenv("MP3D_SMALL", "0")
    what = _name(c)
    code = _gpu.CODE[c["dtype"]]
    lib = _lib.load()
    k = tuple(v if v else 0 for v in c["k"])
    s = tuple(v if v else 0 for v in c["s"])
    zero, one = _a3((0, 0, 0)), _a3((1, 1, 1))
    x = _pins.from_storage(_pins.draw(c["shape"], code, "ties", c["seed"]), code).cuda()
    y = torch.empty(c["shape"][:2] + c["out"], dtype=x.dtype, device="cuda")
    idx = _shifted(y.shape, c["idx"], c["shift"][1])
    _lib.check(lib.mp3d_forward_ex(x.data_ptr(), y.data_ptr(), idx.data_ptr(), code,
                                   mp._IDX[c["idx"]], *c["shape"], *c["out"], _a3(k), _a3(s),
                                   zero, one, _stream()))
    yo, io = orc.forward_ex(_gpu.storage(x), code, c["out"], k, s, (0, 0, 0), (1, 1, 1))
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), io), "%s: idx" % what
    assert np.array_equal(_gpu.storage(y).view(np.uint8), yo.view(np.uint8)), "%s: y bits" % what
    gy0 = _pins.from_storage(_pins.draw(tuple(y.shape), code, "normal", c["seed"] + 9), code).cuda()
    gy = _shifted(y.shape, x.dtype, c["shift"][0])
    gy.copy_(gy0)
    idx32 = torch.from_numpy(io.astype(np.int32))
    for overlap in (-1, 0, 2):
        gx = _shifted(c["shape"], x.dtype, c["shift"][2])
        gx.fill_(float("nan"))
        _lib.check(lib.mp3d_backward_ex(gy.data_ptr(), idx.data_ptr(), gx.data_ptr(), code,
                                        mp._IDX[c["idx"]], *c["shape"], *c["out"], _a3(k),
                                        _a3(s), zero, one, overlap, _stream()))
        _gpu.check_backward(orc, gy0.cpu(), idx32, c["shape"], gx, exact=True,
                            what="%s backward overlap=%d" % (what, overlap))
