"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with the fact it checks.  They are
kept apart from the tests so that the mutation test can run the same
battery against deliberately broken copies of the oracle.

Sources of truth used here, none of which is the oracle's own code:
  * IEEE 754 binary16 / bfloat16 layouts, checked against torch's own
    conversions for every 16-bit pattern and for every rounding midpoint;
  * the page facts on windows: with no padding the fixed-window extent is
    the largest O whose last window still fits ("Struct Maxpool3dForward",
    teenygrad, description), and adaptive windows tile the axis disjointly
    exactly when it divides evenly, overlapping otherwise ("Add
    adaptive_max_pool3d_backward Moore Threads specialized operator",
    Summary);
  * a second formulation of the forward (numpy's first-occurrence argmax
    over each C-ordered window block);
  * torch's CPU max_pool3d / adaptive_max_pool3d and their autograd
    backward, on tie-free data;
  * closed forms (ramps, constants, identity and global windows);
  * for padding, dilation and ceil mode (no page defines them for pooling):
    torch's CPU max_pool3d and its output shapes, and identities with the
    plain forward (subsampling for dilation, a -inf border for padding);
  * numpy's unbuffered ``add.at`` accumulation and ``bincount`` for the
    backward, and the exact ``math.fsum`` invariant for disjoint windows.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

F32, F16, BF16, F64 = 0, 1, 2, 3
TORCH_DT = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, F64: torch.float64}


# ---------------------------------------------------------------------------
# storage helpers (torch <-> oracle storage arrays)
# ---------------------------------------------------------------------------

def to_storage(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> the oracle's storage array (float32 or uint16 bits)."""
    t = t.contiguous()
    if t.dtype in (torch.float32, torch.float64):
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def from_storage(a: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == F32:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32))
    if dtype == F64:
        return torch.from_numpy(np.ascontiguousarray(a, np.float64))
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TORCH_DT[dtype])


def widen_torch(a: np.ndarray, dtype: int) -> np.ndarray:
    """Storage -> float64 through torch's conversion (not the oracle's)."""
    return from_storage(a, dtype).to(torch.float64).numpy()


def draw(shape, dtype: int, kind: str, seed: int) -> np.ndarray:
    """Seeded test data; float64 draws keep full binary64 precision."""
    g = torch.Generator().manual_seed(seed)
    n = int(np.prod(shape))
    fd = torch.float64 if dtype == F64 else torch.float32
    if kind == "normal":
        t = torch.randn(n, generator=g, dtype=fd)
    elif kind == "ties":
        t = torch.randint(-3, 4, (n,), generator=g).float()
    elif kind == "distinct":
        # a random permutation of 0..n-1: no two elements equal
        t = torch.randperm(n, generator=g).float() - n / 2
    elif kind == "zeros":
        # signed zeros among negatives: many windows whose maximum is a zero
        t = torch.tensor([-2.0, -1.0, -0.0, 0.0])[torch.randint(0, 4, (n,), generator=g)]
    elif kind == "sparse_nan":
        # few NaN and infinities: most windows hold none
        t = torch.randn(n, generator=g, dtype=fd)
        u = torch.rand(n, generator=g)
        t[u < 2e-3] = float("inf")
        t[(u >= 2e-3) & (u < 4e-3)] = -float("inf")
        t[u > 1 - 5e-4] = float("nan")
    elif kind == "special":
        t = torch.randn(n, generator=g, dtype=fd)
        pick = torch.randint(0, 12, (n,), generator=g)
        t[pick == 0] = float("nan")
        t[pick == 1] = float("inf")
        t[pick == 2] = -float("inf")
        t[pick == 3] = 0.0
        t[pick == 4] = -0.0
    else:
        raise ValueError(kind)
    return to_storage(t.reshape(shape).to(TORCH_DT[dtype]))


def adaptive_bounds(X: int, O: int, o: int) -> tuple[int, int]:
    """Adaptive window from exact rational floor/ceil (second formulation)."""
    return math.floor(Fraction(o * X, O)), math.ceil(Fraction((o + 1) * X, O))


def window_lists(shape5, out3, k3, s3):
    """Per-axis window lists for the brute-force formulation."""
    lists = []
    for a in range(3):
        X, O, k, s = shape5[2 + a], out3[a], k3[a], s3[a]
        if k:
            lists.append([(o * s, o * s + k) for o in range(O)])
        else:
            lists.append([adaptive_bounds(X, O, o) for o in range(O)])
    return lists


def brute_forward(x: np.ndarray, dtype: int, out3, k3, s3):
    """Forward by numpy: first-occurrence argmax of each C-ordered block."""
    xs = widen_torch(x, dtype)
    N, C, D, H, W = x.shape
    wd, wh, ww = window_lists(x.shape, out3, k3, s3)
    y = np.empty((N, C) + tuple(out3), x.dtype)
    idx = np.empty((N, C) + tuple(out3), np.int32)
    for n in range(N):
        for c in range(C):
            for i, (d0, d1) in enumerate(wd):
                for j, (h0, h1) in enumerate(wh):
                    for l, (w0, w1) in enumerate(ww):
                        blk = xs[n, c, d0:d1, h0:h1, w0:w1]
                        a = int(np.argmax(blk))
                        dd, hh, wq = np.unravel_index(a, blk.shape)
                        flat = ((d0 + dd) * H + h0 + hh) * W + w0 + wq
                        idx[n, c, i, j, l] = flat
                        y[n, c, i, j, l] = x[n, c].reshape(-1)[flat]
    return y, idx


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def _bits64(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(v, np.float64).view(np.uint64)


def pin_widen(orc):
    """Every binary16 and bfloat16 pattern widens to the value torch gives."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in (F16, BF16):
        mine = orc.widen(pats, dt)
        ref = widen_torch(pats, dt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan), "NaN classes differ"
        assert np.array_equal(_bits64(mine[~nan]), _bits64(ref[~nan])), \
            "16-bit widening differs from torch (dtype %d)" % dt


def _midpoints(dt: int) -> np.ndarray:
    """Every value halfway between two adjacent finite 16-bit numbers, plus
    the neighbours of each midpoint, as binary32 (all exactly representable)."""
    pats = np.arange(0, 0x7c00 if dt == F16 else 0x7f80, dtype=np.uint16)
    v = widen_torch(pats, dt)
    mid = (v[:-1] + v[1:]) / 2
    mid32 = mid.astype(np.float32)
    assert np.array_equal(mid32.astype(np.float64), mid)
    up = np.nextafter(mid32, np.float32(np.inf))
    dn = np.nextafter(mid32, np.float32(0))
    allv = np.concatenate([mid32, up, dn])
    return np.concatenate([allv, -allv])


def pin_round(orc):
    """binary32 -> binary16/bfloat16 rounds to nearest, ties to even, on
    every midpoint, its neighbours, and random bit patterns (vs torch)."""
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 2**32, 400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    extra = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0,
                      1e-8, 2.0**-25, 2.0**-24, 3 * 2.0**-26, 1e38, 3.4e38,
                      2.0**-127, 2.0**-133, 2.0**-134, 1.5 * 2.0**-133], np.float32)
    for dt in (F16, BF16):
        vals = np.concatenate([_midpoints(dt), rnd, extra, -extra])
        mine = orc.round16(vals, dt)
        ref = to_storage(torch.from_numpy(vals).to(TORCH_DT[dt]))
        nan = np.isnan(vals)
        assert np.array_equal(mine[~nan], ref[~nan]), \
            "rounding to dtype %d differs from torch" % dt
        # NaN stays NaN (payload conventions are not fixed by the pages)
        back = widen_torch(mine[nan], dt)
        assert np.isnan(back).all()


def pin_windows_adaptive(orc):
    """Adaptive windows, exhaustively for 1 <= X, O <= 64: non-empty,
    monotone, covering [0, X); disjoint tiling of width X/O exactly when O
    divides X, overlapping otherwise (PR #308 Summary); mirror symmetric;
    and equal to exact rational floor/ceil."""
    for X in range(1, 65):
        for O in range(1, 65):
            ws = [orc.window(X, O, 0, 0, o) for o in range(O)]
            assert ws[0][0] == 0 and ws[-1][1] == X
            for o, (a, b) in enumerate(ws):
                assert 0 <= a < b <= X, (X, O, o, a, b)
                assert (a, b) == adaptive_bounds(X, O, o)
                ma, mb = ws[O - 1 - o]
                assert a == X - mb and b == X - ma, "not mirror symmetric"
                assert b - a <= -(-X // O) + 1
                if o:
                    pa, pb = ws[o - 1]
                    assert pa <= a and pb <= b and a <= pb, "gap or disorder"
            overlap = any(ws[o][0] < ws[o - 1][1] for o in range(1, O))
            if X % O == 0:
                assert not overlap
                assert all(b - a == X // O for a, b in ws)
            else:
                assert overlap


def pin_windows_fixed(orc):
    """Fixed windows: O is the largest count whose last window fits without
    padding (teenygrad Maxpool3dForward description), O = 0 never, and a
    window never leaves the axis; matches torch's max_pool3d output size."""
    for k in range(1, 6):
        for s in range(1, 6):
            for X in range(1, 41):
                O = orc.fixed_out(X, k, s)
                if X < k:
                    assert O == -1
                    continue
                assert O >= 1
                assert (O - 1) * s + k <= X < O * s + k
                for o in range(O):
                    a, b = orc.window(X, O, k, s, o)
                    assert (a, b) == (o * s, o * s + k) and b <= X
    for X, k, s in [(7, 3, 2), (9, 2, 2), (16, 4, 3), (5, 5, 1)]:
        t = torch.zeros(1, 1, X, X, X)
        want = F.max_pool3d(t, k, s).shape[2]
        assert orc.fixed_out(X, k, s) == want
    # stated output shapes of the two fixed-window workloads
    assert [orc.fixed_out(X, 2, 2) for X in (16, 112, 112)] == [8, 56, 56]
    assert [orc.fixed_out(X, 3, 2) for X in (32, 56, 56)] == [15, 27, 27]


FORWARD_CASES = [
    # shape, out (adaptive) or None, k, s
    ((1, 2, 5, 6, 7), (3, 4, 2), (0, 0, 0), (0, 0, 0)),
    ((2, 1, 7, 7, 7), (8, 8, 8), (0, 0, 0), (0, 0, 0)),       # O > X
    ((1, 1, 10, 10, 10), (8, 8, 8), (0, 0, 0), (0, 0, 0)),
    ((1, 2, 8, 4, 6), (4, 2, 3), (0, 0, 0), (0, 0, 0)),       # divisible
    ((1, 2, 7, 9, 8), None, (3, 2, 3), (2, 2, 1)),
    ((2, 1, 9, 5, 11), None, (2, 3, 2), (3, 1, 2)),           # k < s skips
    ((1, 1, 6, 6, 6), None, (2, 2, 2), (2, 2, 2)),
    ((1, 2, 5, 8, 7), (2, 3, 0), (0, 0, 3), (0, 0, 2)),       # mixed axes
]


def _out_of(orc, shape, out, k, s):
    res = []
    for a in range(3):
        if k[a]:
            res.append(orc.fixed_out(shape[2 + a], k[a], s[a]))
        else:
            res.append(out[a])
    return tuple(res)


def pin_forward_brute(orc):
    """Forward equals the numpy first-occurrence argmax formulation on
    random, tie-heavy and special-value data in all three dtypes, and the
    argmax invariants hold."""
    seed = 11
    for shape, out, k, s in FORWARD_CASES:
        o3 = _out_of(orc, shape, out, k, s)
        for dt in (F32, F16, BF16, F64):
            for kind in ("normal", "ties", "special"):
                seed += 1
                x = draw(shape, dt, kind, seed)
                y, idx = orc.forward(x, dt, o3, k, s)
                by, bidx = brute_forward(x, dt, o3, k, s)
                assert np.array_equal(idx, bidx), (shape, dt, kind)
                assert np.array_equal(y.view(np.uint8), by.view(np.uint8))


def pin_forward_torch(orc):
    """Values and indices equal torch's CPU pooling on tie-free data, and
    values equal on tie-heavy data (torch's own tie rule is not relied on)."""
    seed = 101
    for shape, out, k, s in FORWARD_CASES:
        if any(k) and not all(k):
            continue  # torch has no mixed fixed/adaptive form
        o3 = _out_of(orc, shape, out, k, s)
        for dt in (F32, F16, BF16, F64):
            for kind in ("distinct", "ties"):
                seed += 1
                n = int(np.prod(shape))
                if kind == "distinct" and n > {F32: 1 << 24, F16: 4096, BF16: 512,
                                               F64: 1 << 53}[dt]:
                    continue  # the format cannot hold that many distinct integers
                x = draw(shape, dt, kind, seed)
                y, idx = orc.forward(x, dt, o3, k, s)
                xt = torch.from_numpy(widen_torch(x, dt))
                if k[0]:
                    ty, ti = F.max_pool3d(xt, k, s, return_indices=True)
                else:
                    ty, ti = F.adaptive_max_pool3d(xt, o3, return_indices=True)
                assert np.array_equal(widen_torch(y, dt), ty.numpy())
                if kind == "distinct":
                    assert np.array_equal(idx, ti.numpy().astype(np.int32))


def pin_forward_closed_forms(orc):
    """Ramps, constants, identity and global windows."""
    shape = (1, 1, 6, 5, 7)
    N, C, D, H, W = shape
    n = D * H * W
    ramp = np.arange(n, dtype=np.float32).reshape(shape)
    for out, k, s in [((4, 3, 5), (0, 0, 0), (0, 0, 0)),
                      (None, (3, 2, 3), (2, 1, 2))]:
        o3 = _out_of(orc, shape, out, k, s)
        wd, wh, ww = window_lists(shape, o3, k, s)
        _, up = orc.forward(ramp, F32, o3, k, s)
        _, down = orc.forward(np.ascontiguousarray(-ramp), F32, o3, k, s)
        _, const = orc.forward(np.full(shape, 2.5, np.float32), F32, o3, k, s)
        for i, (d0, d1) in enumerate(wd):
            for j, (h0, h1) in enumerate(wh):
                for l, (w0, w1) in enumerate(ww):
                    last = ((d1 - 1) * H + h1 - 1) * W + w1 - 1
                    first = (d0 * H + h0) * W + w0
                    assert up[0, 0, i, j, l] == last
                    assert down[0, 0, i, j, l] == first
                    assert const[0, 0, i, j, l] == first
    # identity: 1-wide windows of stride 1, and adaptive O == X
    x = draw(shape, F16, "ties", 5)
    for out, k, s in [(None, (1, 1, 1), (1, 1, 1)), ((D, H, W), (0, 0, 0), (0, 0, 0))]:
        y, idx = orc.forward(x, F16, (D, H, W), k, s)
        assert np.array_equal(y, x)
        assert np.array_equal(idx.reshape(-1), np.arange(n, dtype=np.int32))
    # one global window: the plane's max and first argmax
    x = draw((2, 3, 4, 3, 5), BF16, "ties", 6)
    y, idx = orc.forward(x, BF16, (1, 1, 1))
    xs = widen_torch(x, BF16).reshape(6, -1)
    assert np.array_equal(idx.reshape(-1), np.argmax(xs, axis=1).astype(np.int32))
    # -0 and +0 tie: the earlier one is kept, with its own sign bit
    z = np.zeros((1, 1, 1, 1, 4), np.float32)
    z[..., 0] = -0.0
    z[..., 3] = 0.0
    y, idx = orc.forward(z, F32, (1, 1, 1))
    assert idx.item() == 0 and np.signbit(y.item())


BACKWARD_CASES = [
    ((1, 2, 8, 4, 6), (4, 2, 3), (0, 0, 0), (0, 0, 0)),        # disjoint
    ((2, 1, 6, 6, 6), None, (2, 2, 2), (2, 2, 2)),              # disjoint
    ((1, 2, 10, 10, 10), (8, 8, 8), (0, 0, 0), (0, 0, 0)),     # overlap
    ((1, 2, 9, 8, 7), None, (3, 3, 3), (2, 2, 2)),              # overlap
    ((2, 1, 7, 7, 7), (8, 8, 8), (0, 0, 0), (0, 0, 0)),        # O > X
]


def pin_backward(orc):
    """Backward: contribution counts equal numpy bincount; the binary64 sum
    equals numpy's add.at; the binary32 accumulator equals numpy's
    sequential float32 add.at and lies within the recursive-summation bound
    of the exact sum; gx is that accumulator rounded by torch; untouched
    cells are +0; disjoint windows give gx as an exact permutation of gy
    (fsum invariant); out-of-range idx is ignored."""
    seed = 300
    for shape, out, k, s in BACKWARD_CASES:
        o3 = _out_of(orc, shape, out, k, s)
        N, C, D, H, W = shape
        P, n = N * C, D * H * W
        for dt in (F32, F16, BF16, F64):
            for kind in ("ties", "normal"):
                seed += 1
                x = draw(shape, dt, kind, seed)
                _, idx = orc.forward(x, dt, o3, k, s)
                gy = draw((N, C) + o3, dt, "normal", seed + 1000)
                r = orc.backward(gy, idx, dt, shape)
                g64 = widen_torch(gy, dt).reshape(P, -1)
                ii = idx.reshape(P, -1)
                for p in range(P):
                    cnt = np.bincount(ii[p], minlength=n)
                    assert np.array_equal(r["count"].reshape(P, -1)[p], cnt)
                    ref = np.zeros(n)
                    np.add.at(ref, ii[p], g64[p])
                    assert np.array_equal(r["ref64"].reshape(P, -1)[p], ref)
                    ab = np.zeros(n)
                    np.add.at(ab, ii[p], np.abs(g64[p]))
                    assert np.array_equal(r["abs64"].reshape(P, -1)[p], ab)
                    if dt == F64:
                        # float64: the binary64 fold in ascending order is gx itself
                        got = r["gx"].reshape(P, -1)[p]
                        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))
                        continue
                    acc = np.zeros(n, np.float32)
                    np.add.at(acc, ii[p], g64[p].astype(np.float32))
                    got = r["acc32"].reshape(P, -1)[p]
                    assert np.array_equal(got.view(np.uint32), acc.view(np.uint32))
                    m = np.maximum(cnt - 1, 0)
                    bound = m * 2.0**-24 * ab * 1.0001
                    assert (np.abs(got.astype(np.float64) - ref) <= bound).all()
                    assert (got[cnt == 0].view(np.uint32) == 0).all()
                if dt != F64:
                    gx_ref = to_storage(torch.from_numpy(r["acc32"]).to(TORCH_DT[dt]))
                    assert np.array_equal(r["gx"], gx_ref)
                disjoint = all(
                    (k[a] and k[a] == s[a]) or (not k[a] and shape[2 + a] % o3[a] == 0)
                    for a in range(3))
                if disjoint:
                    assert r["count"].max() <= 1
                    gxs = widen_torch(r["gx"], dt)
                    assert math.fsum(gxs.ravel()) == math.fsum(g64.ravel())
                    # closed form: gx[p] = 0 + gy[w] where idx[w] == p
                    want = np.zeros((P, n))
                    for p in range(P):
                        want[p, ii[p]] = g64[p] + 0.0   # +0 + (-0) is +0
                    assert np.array_equal(_bits64(gxs.reshape(P, n)), _bits64(want))
    # out-of-range idx entries are skipped, in-range ones still land
    gy = draw((1, 1, 2, 2, 2), F32, "normal", 9)
    idx = np.array([0, -1, 7, 8, 2**31 - 1, 3, -2**31, 7], np.int32).reshape(1, 1, 2, 2, 2)
    r = orc.backward(gy, idx, F32, (1, 1, 2, 2, 2))
    flat = gy.reshape(-1)
    want = np.zeros(8, np.float32)
    want[0] = flat[0]
    want[3] = flat[5]
    want[7] = np.float32(flat[2] + flat[7])
    assert np.array_equal(r["gx"].reshape(-1), want)


def pin_backward_torch(orc):
    """On tie-free data, the binary64 sum equals torch's autograd gradient
    of max_pool3d / adaptive_max_pool3d (computed in float64)."""
    seed = 500
    for shape, out, k, s in BACKWARD_CASES:
        o3 = _out_of(orc, shape, out, k, s)
        seed += 1
        x = draw(shape, F32, "distinct", seed)
        _, idx = orc.forward(x, F32, o3, k, s)
        gy = draw((shape[0], shape[1]) + o3, F32, "normal", seed + 1)
        r = orc.backward(gy, idx, F32, shape)
        xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
        if k[0]:
            yt = F.max_pool3d(xt, k, s)
        else:
            yt = F.adaptive_max_pool3d(xt, o3)
        yt.backward(torch.from_numpy(gy.astype(np.float64)))
        assert np.allclose(r["ref64"], xt.grad.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# padding, dilation and ceil mode (forward_ex)
# ---------------------------------------------------------------------------

# (shape, kernel, stride, pad, dilation, ceil_mode); every case is one torch
# accepts (pad <= kernel / 2, at least one window per axis)
EX_CASES = [
    ((1, 2, 7, 8, 9), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), False),
    ((1, 1, 7, 8, 9), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), True),
    ((2, 1, 6, 7, 5), (2, 2, 2), (2, 2, 2), (1, 0, 1), (1, 1, 1), True),
    ((1, 1, 9, 9, 9), (3, 2, 3), (1, 2, 3), (1, 1, 0), (2, 3, 1), False),
    ((1, 1, 9, 10, 11), (3, 3, 2), (2, 3, 2), (1, 1, 1), (2, 2, 3), True),
    ((1, 1, 5, 6, 7), (1, 1, 1), (2, 2, 2), (0, 0, 0), (1, 1, 1), True),
    ((1, 1, 4, 5, 6), (4, 5, 2), (3, 2, 1), (2, 2, 1), (1, 1, 2), True),
    ((1, 1, 2, 3, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (3, 2, 2), False),   # all-padding windows
]


def ex_out(orc, shape, k, s, pad, dil, ceil_mode):
    return tuple(orc.fixed_out_ex(X, *a, ceil_mode=ceil_mode)
                 for X, a in zip(shape[2:], zip(k, s, pad, dil)))


def pin_out_size_ex(orc):
    """Output extents with padding, dilation and ceil mode equal torch's
    pooling output shape over a grid of small axes (and -1 exactly where no
    window fits)."""
    for X in range(1, 11):
        for k in range(1, 5):
            for s in range(1, 4):
                for pad in range(0, k // 2 + 1):
                    for dil in range(1, 4):
                        for cm in (False, True):
                            got = orc.fixed_out_ex(X, k, s, pad, dil, cm)
                            if X + 2 * pad < (k - 1) * dil + 1:
                                assert got == -1, (X, k, s, pad, dil, cm)
                                continue
                            t = F.max_pool1d(torch.zeros(1, 1, X), k, s, pad, dil, ceil_mode=cm)
                            assert got == t.shape[-1], (X, k, s, pad, dil, cm, got, t.shape)


def pin_forward_ex_torch(orc):
    """Values and indices with padding, dilation and ceil mode equal torch's
    CPU max_pool3d on tie-free data (values on tie-heavy data); a window
    whose taps are all padding gives -inf and index -1 (torch's index there
    is not a position, so only its -inf is compared)."""
    seed = 1301
    for shape, k, s, pad, dil, cm in EX_CASES:
        o3 = ex_out(orc, shape, k, s, pad, dil, cm)
        for dt in (F32, F16, BF16, F64):
            for kind in ("distinct", "ties"):
                seed += 1
                n = int(np.prod(shape))
                if kind == "distinct" and n > {F32: 1 << 24, F16: 4096, BF16: 512,
                                               F64: 1 << 53}[dt]:
                    continue
                x = draw(shape, dt, kind, seed)
                y, idx = orc.forward_ex(x, dt, o3, k, s, pad, dil)
                xt = torch.from_numpy(widen_torch(x, dt))
                ty, ti = F.max_pool3d(xt, k, s, pad, dil, ceil_mode=cm, return_indices=True)
                assert tuple(ty.shape[2:]) == o3, (shape, k, s, pad, dil, cm)
                assert np.array_equal(widen_torch(y, dt), ty.numpy()), (shape, dt, kind)
                empty = idx < 0
                assert np.all(np.isneginf(widen_torch(y, dt)[empty]))
                if kind == "distinct":
                    assert np.array_equal(idx[~empty], ti.numpy()[~empty]), (shape, dt, kind)


def pin_forward_ex_identities(orc):
    """Identities that tie the padded / dilated forward to the plain one
    (itself pinned above): no padding and dilation 1 is the plain forward;
    stride = m * dilation with no padding is the plain forward with stride m
    over every dil-th element; padding is an explicit -inf border."""
    x = draw((2, 1, 9, 10, 11), F32, "ties", 1401)
    for k, s in [((3, 2, 2), (2, 1, 2)), ((1, 3, 2), (1, 2, 2))]:
        o3 = _out_of(orc, x.shape, None, k, s)
        y0, i0 = orc.forward(x, F32, o3, k, s)
        y1, i1 = orc.forward_ex(x, F32, o3, k, s)
        assert np.array_equal(y0, y1) and np.array_equal(i0.astype(np.int64), i1)
    # dilation 2 and 3, stride a multiple of it, offset 0
    D, H, W = x.shape[2:]
    for dil, k, m in [((2, 3, 2), (2, 2, 3), (1, 1, 2)), ((3, 2, 1), (3, 2, 2), (1, 2, 1))]:
        s = tuple(a * b for a, b in zip(dil, m))
        o3 = ex_out(orc, x.shape, k, s, (0, 0, 0), dil, False)
        y, idx = orc.forward_ex(x, F32, o3, k, s, (0, 0, 0), dil)
        sub = np.ascontiguousarray(x[:, :, ::dil[0], ::dil[1], ::dil[2]])
        so3 = _out_of(orc, sub.shape, None, k, m)
        sy, sidx = orc.forward(sub, F32, so3, k, m)
        assert o3 == tuple(min(a, b) for a, b in zip(o3, so3))
        sd, sh, sw = sub.shape[2:]
        sd_, rem = np.divmod(sidx, sh * sw)
        sh_, sw_ = np.divmod(rem, sw)
        full = ((sd_ * dil[0]) * H + sh_ * dil[1]) * W + sw_ * dil[2]
        sl = (slice(None), slice(None)) + tuple(slice(0, n) for n in o3)
        assert np.array_equal(y, sy[sl]) and np.array_equal(idx, full[sl].astype(np.int64))
    # padding: an explicit -inf border, then no padding
    for k, s, pad, dil, cm in [((3, 3, 2), (2, 1, 2), (1, 1, 1), (1, 2, 1), False),
                               ((2, 3, 3), (2, 2, 3), (1, 1, 1), (1, 1, 1), True)]:
        o3 = ex_out(orc, x.shape, k, s, pad, dil, cm)
        y, idx = orc.forward_ex(x, F32, o3, k, s, pad, dil)
        big = np.pad(x, [(0, 0), (0, 0)] + [(p, p + 2 * max(s)) for p in pad],
                     constant_values=-np.inf).astype(np.float32)
        by, bidx = orc.forward_ex(np.ascontiguousarray(big), F32, o3, k, s, (0, 0, 0), dil)
        BH, BW = big.shape[3:]
        bd, rem = np.divmod(bidx, BH * BW)
        bh, bw = np.divmod(rem, BW)
        back = ((bd - pad[0]) * H + (bh - pad[1])) * W + (bw - pad[2])
        assert np.array_equal(y, by) and np.array_equal(idx, back)


def pin_argmax_from_output(orc):
    """The argmax recovered from (x, y) is the forward's own argmax when y
    is the forward's output -- on tie-heavy, zero-signed and NaN data, for
    plain, adaptive, padded and dilated windows -- and otherwise the first
    element of the window (numpy's first-occurrence search over each
    window's taps) equal to y, or -1."""
    seed = 1501
    cases = [((2, 2, 7, 8, 9), (2, 2, 2), (2, 2, 2), (0, 0, 0), (1, 1, 1), False),
             ((1, 2, 9, 8, 7), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), True),
             ((1, 1, 9, 10, 11), (3, 2, 3), (1, 2, 3), (1, 1, 0), (2, 3, 1), False),
             ((1, 1, 2, 3, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (3, 2, 2), False)]
    for shape, k, s, pad, dil, cm in cases:
        o3 = ex_out(orc, shape, k, s, pad, dil, cm)
        for dt in (F32, F16, BF16, F64):
            for kind in ("ties", "zeros", "sparse_nan", "special"):
                seed += 1
                x = draw(shape, dt, kind, seed)
                y, idx = orc.forward_ex(x, dt, o3, k, s, pad, dil)
                got = orc.argmax_from_output(x, y, dt, k, s, pad, dil)
                assert np.array_equal(got, idx), (shape, dt, kind)
    # adaptive axes, and y that is not the forward's output
    x = draw((2, 1, 7, 6, 5), F32, "ties", 1601)
    y, idx = orc.forward(x, F32, (3, 4, 2))
    assert np.array_equal(orc.argmax_from_output(x, y, F32), idx.astype(np.int64))
    rng = np.random.default_rng(1602)
    y2 = y.copy()
    y2.reshape(-1)[::3] = rng.integers(-5, 6, y2.size)[::3].astype(np.float32)
    got = orc.argmax_from_output(x, y2, F32)
    wd, wh, ww = window_lists(x.shape, (3, 4, 2), (0, 0, 0), (0, 0, 0))
    for p_ in range(2):
        for i, (d0, d1) in enumerate(wd):
            for j, (h0, h1) in enumerate(wh):
                for l, (w0, w1) in enumerate(ww):
                    blk = x[p_, 0, d0:d1, h0:h1, w0:w1]
                    hit = np.flatnonzero(blk.reshape(-1) == y2[p_, 0, i, j, l])
                    want = -1
                    if hit.size:
                        bd, rem = divmod(int(hit[0]), (h1 - h0) * (w1 - w0))
                        bh, bw = divmod(rem, w1 - w0)
                        want = ((d0 + bd) * 6 + h0 + bh) * 5 + w0 + bw
                    assert got[p_, 0, i, j, l] == want


ALL_PINS = [pin_widen, pin_round, pin_windows_adaptive, pin_windows_fixed,
            pin_forward_brute, pin_forward_torch, pin_forward_closed_forms,
            pin_backward, pin_backward_torch, pin_out_size_ex, pin_forward_ex_torch,
            pin_forward_ex_identities, pin_argmax_from_output]
