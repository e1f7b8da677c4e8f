"""The index-free backward (argmax recomputed from x and y) on the device,
through the C ABI, against the oracle: its argmax recovered from (x, y) fed
to its backward.  With y from the values-only forward this is the whole
index-free pipeline; y that disagrees with x drops those windows."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import _gpu
import _pins
import bwd_max_pool3d_amd as mp
from bwd_max_pool3d_amd import workloads

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16, torch.float64]
DT_ID = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.float64: "f64"}

# (shape, adaptive out or None, kernel, stride, pad, dilation, ceil_mode)
CASES = [
    ((2, 3, 8, 8, 8), (4, 4, 4), None, None, None, None, False),
    ((1, 2, 10, 10, 10), (8, 8, 8), None, None, None, None, False),
    ((1, 1, 7, 7, 7), (8, 8, 8), None, None, None, None, False),
    ((1, 2, 16, 32, 32), (5, 7, 7), None, None, None, None, False),
    ((2, 3, 8, 8, 8), None, (2, 2, 2), (2, 2, 2), (0, 0, 0), (1, 1, 1), False),
    ((1, 2, 9, 8, 7), None, (3, 3, 3), (2, 2, 2), (0, 0, 0), (1, 1, 1), False),
    ((2, 1, 6, 7, 13), None, (3, 3, 3), (1, 1, 1), (0, 0, 0), (1, 1, 1), False),
    ((2, 2, 9, 12, 13), None, (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), True),
    ((1, 1, 10, 11, 12), None, (3, 2, 3), (1, 2, 3), (1, 1, 0), (2, 3, 1), False),
    ((1, 1, 2, 3, 4), None, (2, 2, 2), (1, 1, 1), (1, 1, 1), (3, 2, 2), False),
    ((1, 1, 3, 200, 300), None, (3, 3, 3), (1, 2, 2), (1, 1, 1), (1, 1, 1), False),
    # the fused index-free kernel: 2, 4 and 8 windows per thread with the
    # looped scan (windows of 4 taps along h, w), 4 and 8 with the 3 x 3
    # scan, and windows up to 8 slices deep
    ((1, 2, 8, 48, 48), (5, 14, 14), None, None, None, None, False),
    ((1, 2, 8, 64, 64), (5, 20, 20), None, None, None, None, False),
    ((1, 2, 8, 64, 64), (5, 23, 23), None, None, None, None, False),
    ((1, 2, 8, 40, 40), (5, 20, 20), None, None, None, None, False),
    ((1, 2, 8, 40, 48), (5, 28, 24), None, None, None, None, False),
    ((1, 2, 20, 12, 16), (3, 5, 5), None, None, None, None, False),
    # slabs that no window reaches: the slices after the last window, and
    # gaps between windows (stride above the kernel)
    ((1, 2, 8, 8, 16), None, (3, 3, 3), (2, 2, 2), (0, 0, 0), (1, 1, 1), False),
    ((1, 2, 10, 8, 8), None, (1, 1, 1), (5, 5, 5), (0, 0, 0), (1, 1, 1), False),
]


def _cid(c):
    shape, out, k, s, p, d, cm = c
    j = lambda t: "".join(map(str, t))
    geo = "a%s" % "x".join(map(str, out)) if out else "k%ss%sp%sd%s%s" % (
        j(k), j(s), j(p), j(d), "-ceil" if cm else "")
    return "%s-%s" % ("x".join(map(str, shape)), geo)


def _forward_values(x, case):
    shape, out, k, s, p, d, cm = case
    if out is not None:
        return mp.amp3d_forward(x, out, indices=False)
    return mp.mp3d_forward_ex(x, k, s, p, d, cm, indices=False)


def _geom(case):
    shape, out, k, s, p, d, cm = case
    if out is not None:
        return dict(kernel=None)
    return dict(kernel=k, stride=s, padding=p, dilation=d)


def _oracle_argmax(orc, x, y, case):
    shape, out, k, s, p, d, cm = case
    code = _gpu.CODE[x.dtype]
    xs, ys = _gpu.storage(x), _gpu.storage(y)
    if out is not None:
        return orc.argmax_from_output(xs, ys, code)
    return orc.argmax_from_output(xs, ys, code, k, s, p, d)


@pytest.fixture(params=["one-pass", "two-pass"])
def ws(request, monkeypatch):
    """'two-pass': a workspace, and MP3D_TWO_PASS=1 so that the forward into
    it and the checked argmax run on every shape (the library keeps small
    tensors on the one-pass form by itself)."""
    if request.param == "one-pass":
        return False
    monkeypatch.setenv("MP3D_TWO_PASS", "1")
    return True


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DT_ID[d])
@pytest.mark.parametrize("case", CASES, ids=_cid)
def test_recompute_backward(orc, case, dtype, ws):
    """Both forms: the one-pass kernels, and the forward into a workspace
    with its argmax checked against y."""
    shape = case[0]
    code = _gpu.CODE[dtype]
    base = abs(hash(case)) % 10000
    for j, kind in enumerate(("normal", "ties", "zeros", "sparse_nan")):
        x = _pins.from_storage(_pins.draw(shape, code, kind, base + j), code).cuda()
        y = _forward_values(x, case)
        gy = _pins.from_storage(_pins.draw(tuple(y.shape), code, "normal", base + 10 + j), code).cuda()
        ia = _oracle_argmax(orc, x.cpu(), y.cpu(), case)
        ref_idx = torch.from_numpy(ia.astype(np.int32))
        for overlap, exact in ((-1, False), (2, True)):
            gx = mp.mp3d_backward_recompute(x, y, gy, overlap=overlap, workspace=ws,
                                            **_geom(case))
            _gpu.check_backward(orc, gy.cpu(), ref_idx, shape, gx, exact=exact,
                                what="%s %s overlap=%d" % (_cid(case), kind, overlap))


def test_recompute_y_not_from_forward(orc, ws):
    """Windows whose y matches no element of the window contribute nothing;
    the others route to the first match (with a workspace: the windows
    where y is not the forward's maximum take the scan)."""
    case = ((1, 2, 9, 8, 7), None, (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), False)
    x = _pins.from_storage(_pins.draw(case[0], 0, "ties", 77), 0).cuda()
    y = _forward_values(x, case).clone()
    flat = y.view(-1)
    flat[::3] = flat[::3] - 1.0          # integer data: often still present in the window
    flat[1::5] = 100.0                   # never present
    gy = _pins.from_storage(_pins.draw(tuple(y.shape), 0, "normal", 78), 0).cuda()
    ia = _oracle_argmax(orc, x.cpu(), y.cpu(), case)
    assert (ia < 0).sum() > 0 and (ia >= 0).sum() > 0
    ref_idx = torch.from_numpy(ia.astype(np.int32))
    for overlap, exact in ((-1, False), (1, False), (2, True)):
        gx = mp.mp3d_backward_recompute(x, y, gy, overlap=overlap, workspace=ws, **_geom(case))
        _gpu.check_backward(orc, gy.cpu(), ref_idx, case[0], gx, exact=exact,
                            what="perturbed y overlap=%d" % overlap)


@pytest.mark.parametrize("wl", [w for w in workloads.WORKLOADS if w.backward], ids=lambda w: w.name)
def test_recompute_full_size(orc, wl):
    """At full size the ordered index-free backward equals the ordered
    backward from the forward's idx bit for bit (both are the ascending
    fold of the same contributions; the idx path is checked against the
    oracle in test_gpu_parity).  The index-free backward in any order (the
    fused column-stage kernel where it applies) is checked against the
    oracle, fed the forward's idx, on every plane, and within the
    binary32-summation bound on every element."""
    xd = wl.make_x().cuda()
    if wl.adaptive:
        y, idx = mp.amp3d_forward(xd, wl.out)
        geo = dict(kernel=None)
    else:
        y, idx = mp.mp3d_forward(xd, wl.kernel, wl.stride)
        geo = dict(kernel=wl.kernel, stride=wl.stride)
    gy = wl.make_gy(tuple(y.shape)).cuda()
    ref = mp.mp3d_backward(gy, idx, wl.shape, kernel=wl.kernel, stride=wl.stride, overlap=2)
    got = mp.mp3d_backward_recompute(xd, y, gy, overlap=2, **geo)
    iv = torch.int32 if got.element_size() == 4 else torch.int16
    assert torch.equal(got.view(iv), ref.view(iv)), wl.name
    ws = torch.empty(mp.recompute_workspace_size(xd.dtype, *wl.shape[:2], tuple(y.shape[2:])),
                     dtype=torch.uint8, device=xd.device)
    got = mp.mp3d_backward_recompute(xd, y, gy, overlap=2, workspace=ws, **geo)
    assert torch.equal(got.view(iv), ref.view(iv)), wl.name + " workspace"
    os.environ["MP3D_TWO_PASS"] = "1"      # the two-pass form on every workload
    try:
        got = mp.mp3d_backward_recompute(xd, y, gy, overlap=2, workspace=ws, **geo)
        assert torch.equal(got.view(iv), ref.view(iv)), wl.name + " two-pass"
        gxw = mp.mp3d_backward_recompute(xd, y, gy, workspace=ws, **geo)
    finally:
        del os.environ["MP3D_TWO_PASS"]
    del ref, got
    gx = mp.mp3d_backward_recompute(xd, y, gy, **geo)
    torch.cuda.synchronize()
    gyc = gy.cpu()
    for g, form in ((gx, "one-pass"), (gxw, "two-pass")):
        _gpu.check_backward_all(orc, gyc, idx, wl.shape, g, exact=False,
                                what="%s index-free %s" % (wl.name, form))
    _gpu.full_backward_property(gy, idx, gx, wl.shape)
    _gpu.full_backward_property(gy, idx, gxw, wl.shape)


def test_recompute_workspace_too_small():
    """A workspace smaller than the size query, or not 16-byte aligned, is
    refused before any launch."""
    x = torch.zeros((1, 2, 6, 6, 6), dtype=torch.float32, device="cuda")
    y = mp.amp3d_forward(x, (3, 3, 3), indices=False)
    need = mp.recompute_workspace_size(torch.float32, 1, 2, (3, 3, 3))
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(mp.Mp3dError, match="workspace"):
        mp.mp3d_backward_recompute(x, y, torch.ones_like(y), workspace=ws)
    # an unaligned workspace of enough bytes is refused too
    ws = torch.empty(need + 16, dtype=torch.uint8, device="cuda")[1:]
    with pytest.raises(mp.Mp3dError, match="aligned"):
        mp.mp3d_backward_recompute(x, y, torch.ones_like(y), workspace=ws)
