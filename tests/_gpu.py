"""Helpers for the GPU parity tests: run the HIP path through the Python
binding (which calls the C ABI), run the CPU oracle on the same bits, and
compare them to the bar each path must meet.

  forward:                      y bits and idx equal, every dtype
  backward, gather path:        gx bits equal
  backward, accumulate path:    gx bits equal wherever at most two
                                contributions land (a + b is one correctly
                                rounded, commutative add); elsewhere float32
                                within 1e-6 of the sum of magnitudes, and
                                float16 / bfloat16 within one unit in the
                                last place of the oracle's float32-summed,
                                once-rounded value; any cell outside that is
                                settled exactly by checking that it equals
                                the rounded float32 fold of its own
                                contributions in some order (an atomic
                                scatter serialises the adds to one address).
NaN outputs match NaN outputs; their payload bits are not compared.
"""
from __future__ import annotations

import itertools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import _pins
import bwd_max_pool3d_amd as mp

CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3}
POISON = {torch.float32: float("nan"), torch.float16: float("nan"),
          torch.bfloat16: float("nan"), torch.float64: float("nan")}


def storage(t: torch.Tensor) -> np.ndarray:
    return _pins.to_storage(t.detach().cpu())


def out_shape(orc, shape, out=None, k=None, s=None):
    if k is None:
        return tuple(out)
    return tuple(orc.fixed_out(X, ka, sa) for X, ka, sa in zip(shape[2:], k, s))


def gpu_forward(x: torch.Tensor, out=None, k=None, s=None, poison=True, indices=True):
    """Run the forward on the device copy of ``x``.  With ``poison`` the
    outputs start filled with NaN / -7 so an unwritten element cannot pass.
    With ``indices`` False the values-only forward runs (idx NULL) and y
    alone is returned."""
    xd = x.cuda() if not x.is_cuda else x
    N, C = x.shape[:2]
    if k is None:
        o3 = tuple(out)
    else:
        o3 = tuple(mp.mp3d_out_size(X, ka, sa) for X, ka, sa in zip(x.shape[2:], k, s))
    pre = None
    if poison:
        pre = (torch.full((N, C) + o3, POISON[x.dtype], dtype=x.dtype, device=xd.device),
               torch.full((N, C) + o3, -7, dtype=torch.int32, device=xd.device))
        if not indices:
            pre = pre[0]
    if k is None:
        return mp.amp3d_forward(xd, o3, out=pre, indices=indices)
    return mp.mp3d_forward(xd, k, s, out=pre, indices=indices)


def oracle_forward(orc, x: torch.Tensor, out=None, k=None, s=None):
    code = CODE[x.dtype]
    o3 = out_shape(orc, x.shape, out, k, s)
    kk = tuple(k) if k is not None else (0, 0, 0)
    ss = tuple(s) if s is not None else (0, 0, 0)
    return orc.forward(storage(x), code, o3, kk, ss)


def assert_forward_match(y_gpu, idx_gpu, y_orc, idx_orc, what=""):
    yg = storage(y_gpu)
    ig = idx_gpu.cpu().numpy()
    bad = np.nonzero((ig != idx_orc).ravel())[0]
    assert bad.size == 0, "%s: %d idx mismatches, first at flat %d: gpu %d oracle %d" % (
        what, bad.size, bad[0], ig.ravel()[bad[0]], idx_orc.ravel()[bad[0]])
    assert np.array_equal(yg.view(np.uint8), y_orc.view(np.uint8)), "%s: y bits differ" % what


def gpu_backward(gy: torch.Tensor, idx: torch.Tensor, in_shape, k=None, s=None,
                 overlap=-1, poison=True):
    gyd = gy.cuda() if not gy.is_cuda else gy
    idd = idx.cuda() if not idx.is_cuda else idx
    pre = None
    if poison:
        pre = torch.full(tuple(in_shape), POISON[gy.dtype], dtype=gy.dtype, device=gyd.device)
    return mp.mp3d_backward(gyd, idd, in_shape, kernel=k, stride=s, overlap=overlap, out=pre)


def _key16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7fff), b)


def _round(acc32: np.ndarray, code: int) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(acc32, np.float32))
    return _pins.to_storage(t.to(_pins.TORCH_DT[code]))


def _nan_mask(st: np.ndarray, code: int) -> np.ndarray:
    return np.isnan(_pins.widen_torch(st, code))


def _fold_orders(contribs: np.ndarray, code: int):
    """Every rounded float32 fold of ``contribs`` from +0 (distinct orders)."""
    seen = set()
    outs = set()
    for perm in itertools.permutations(range(len(contribs))):
        key = tuple(contribs[list(perm)].view(np.uint32))
        if key in seen:
            continue
        seen.add(key)
        acc = np.float32(0.0)
        for i in perm:
            acc = np.float32(acc + contribs[i])
        outs.add(int(_round(np.array([acc], np.float32), code).view(
            np.uint32 if code == 0 else np.uint16)[0]))
    return outs


def check_backward(orc, gy: torch.Tensor, idx: torch.Tensor, in_shape, gx_gpu,
                   exact: bool, what=""):
    """Compare gx from the device with the oracle on the same gy and idx."""
    code = CODE[gy.dtype]
    check_backward_arrays(orc, storage(gy), idx.cpu().numpy(), storage(gx_gpu), code,
                          tuple(in_shape), exact, what)


def check_backward_arrays(orc, gys: np.ndarray, ids: np.ndarray, got: np.ndarray, code: int,
                          in_shape, exact: bool, what=""):
    """check_backward on host arrays: gy and gx in storage form, idx int32."""
    r = orc.backward(np.ascontiguousarray(gys), np.ascontiguousarray(ids), code, tuple(in_shape))
    want = r["gx"].reshape(-1)
    got = got.reshape(-1)
    ubits = {0: np.uint32, 3: np.uint64}.get(code, np.uint16)
    wb, gb = want.view(ubits), got.view(ubits)
    nan_w, nan_g = _nan_mask(want, code), _nan_mask(got, code)
    assert np.array_equal(nan_w, nan_g), "%s: NaN positions differ" % what
    same = (wb == gb) | nan_w
    if exact:
        bad = np.nonzero(~same)[0]
        assert bad.size == 0, "%s: %d gx mismatches, first at %d" % (what, bad.size, bad[0])
        return
    cnt = r["count"].reshape(-1)
    bad = np.nonzero(~same & (cnt <= 2))[0]
    assert bad.size == 0, "%s: %d cells with <= 2 contributions differ, first at %d" % (
        what, bad.size, bad[0])
    if code == 3:
        # binary64 folds of the same terms in two orders: each within
        # (n-1) * 2^-53 * sum|c| of the exact sum
        ab = r["abs64"].reshape(-1)
        bound = 2 * np.maximum(cnt - 1, 0) * 2.0**-53 * ab * 1.0001
        err = np.abs(got - want)
        out = np.nonzero(~same & ~(err <= bound))[0]
        assert out.size == 0, "%s: %d float64 cells outside the bound" % (what, out.size)
        return
    if code == 0:
        err = np.abs(got.astype(np.float64) - r["acc32"].reshape(-1).astype(np.float64))
        tol_ok = err <= 1e-6 * r["abs64"].reshape(-1)
    else:
        tol_ok = np.abs(_key16(gb) - _key16(wb)) <= 1
    out = np.nonzero(~same & ~tol_ok)[0]
    if out.size == 0:
        return
    # settle the rest exactly: some serial order of the cell's contributions
    assert out.size <= 2000, "%s: %d cells outside tolerance" % (what, out.size)
    N, C, D, H, W = in_shape
    plane_in = D * H * W
    g32 = _pins.widen_torch(gys, code).astype(np.float32).reshape(N * C, -1)
    ii = ids.reshape(N * C, -1)
    for cell in out:
        p, loc = divmod(int(cell), plane_in)
        contribs = g32[p][ii[p] == loc]
        assert len(contribs) <= 8, "%s: cell %d has %d contributions" % (what, cell, len(contribs))
        assert int(gb[cell]) in _fold_orders(contribs, code), \
            "%s: cell %d is no serial order of its contributions" % (what, cell)


# ---------------------------------------------------------------------------
# every plane of a full-size tensor against the oracle, plane ranges in
# parallel host threads (each oracle call releases the interpreter lock)
# ---------------------------------------------------------------------------

def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ranges(P: int, parts: int):
    cuts = np.linspace(0, P, max(1, min(parts, P)) + 1).astype(int)
    return [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def _each_range(P: int, fn, parts: int | None = None):
    parts = parts or 4 * _threads()
    with ThreadPoolExecutor(_threads()) as pool:
        list(pool.map(lambda r: fn(*r), _ranges(P, parts)))


def check_forward_all(orc, x: torch.Tensor, y, idx, out=None, k=None, s=None, what=""):
    """Every plane's y bits and idx against the oracle (x on the host; y and
    idx on the device)."""
    N, C, D, H, W = x.shape
    P = N * C
    code = CODE[x.dtype]
    o3 = out_shape(orc, x.shape, out, k, s)
    kk = tuple(k) if k is not None else (0, 0, 0)
    ss = tuple(s) if s is not None else (0, 0, 0)
    xs = storage(x).reshape(P, 1, D, H, W)
    yg = storage(y).reshape(P, -1)
    ig = idx.cpu().numpy().reshape(P, -1)
    ubits = {0: np.uint32, 3: np.uint64}.get(code, np.uint16)

    def run(a, b):
        yo, io = orc.forward(xs[a:b], code, o3, kk, ss)
        io = io.reshape(b - a, -1)
        bad = np.nonzero((io != ig[a:b]).ravel())[0]
        assert bad.size == 0, "%s: %d idx mismatches in planes %d..%d, first at plane %d" % (
            what, bad.size, a, b, a + bad[0] // io.shape[1])
        assert np.array_equal(yo.reshape(b - a, -1).view(ubits), yg[a:b].view(ubits)), \
            "%s: y bits differ in planes %d..%d" % (what, a, b)
    _each_range(P, run)


def check_backward_all(orc, gy: torch.Tensor, idx, in_shape, gx, exact: bool, what=""):
    """check_backward on every plane (gy on the host or the device; idx and
    gx on either)."""
    N, C, D, H, W = in_shape
    P = N * C
    code = CODE[gy.dtype]
    OD, OH, OW = gy.shape[2:]
    gys = storage(gy).reshape(P, 1, OD, OH, OW)
    ids = (idx.cpu() if isinstance(idx, torch.Tensor) else torch.as_tensor(idx)).numpy()
    ids = ids.reshape(P, 1, OD, OH, OW)
    gxs = storage(gx).reshape(P, -1)

    def run(a, b):
        check_backward_arrays(orc, gys[a:b], ids[a:b], gxs[a:b], code, (b - a, 1, D, H, W),
                              exact, "%s planes %d..%d" % (what, a, b))
    _each_range(P, run)


def sample_planes(P: int, n: int = 10, seed: int = 0):
    """Planes 0 and P - 1 and n seeded picks, sorted."""
    rng = np.random.default_rng(seed)
    picks = {0, P - 1} | set(int(v) for v in rng.integers(0, P, size=n))
    return sorted(picks)


def full_backward_property(gy, idx, gx, in_shape):
    """On every gx element: within the float32-summation bound (plus half a
    unit in the last place of the storage type) of the exact sum."""
    N, C, D, H, W = in_shape
    P, n = N * C, D * H * W
    ii = idx.view(P, -1).long()
    g64 = gy.view(P, -1).double()
    ref = torch.zeros(P, n, dtype=torch.float64, device="cuda").scatter_add_(1, ii, g64)
    ab = torch.zeros(P, n, dtype=torch.float64, device="cuda").scatter_add_(1, ii, g64.abs())
    cnt = torch.zeros(P, n, dtype=torch.float64, device="cuda").scatter_add_(
        1, ii, torch.ones_like(g64))
    half_ulp = {torch.float32: 0.0, torch.float16: 2.0**-11, torch.bfloat16: 2.0**-8}[gy.dtype]
    tiny = {torch.float32: 0.0, torch.float16: 2.0**-25, torch.bfloat16: 2.0**-134}[gy.dtype]
    bound = (cnt - 1).clamp(min=0) * 2.0**-24 * ab * 1.0001 + half_ulp * ref.abs() * 1.0001 + tiny
    err = (gx.view(P, -1).double() - ref).abs()
    assert bool((err <= bound).all()), "max excess %g" % float((err - bound).max())
    assert bool((gx.view(P, -1)[cnt == 0] == 0).all())
