"""The entry points under HIP graph capture.  The library allocates nothing
and only launches kernels on the caller's stream (no memset, no
synchronisation), so a forward + backward sequence can be captured once and
replayed.  Every replay, with new input values copied in and the outputs
poisoned between replays (eager work in between, as a caller would do), must
reproduce the eager calls bit for bit."""
from __future__ import annotations

import pytest
import torch

import bwd_max_pool3d_amd as mp

pytestmark = pytest.mark.gpu

# (shape, dtype, kernel, stride, adaptive out): the fixed workloads' row-vector
# forward with the slab backward, and the column forward with the slab backward
CASES = [
    ((2, 4, 16, 28, 28), torch.float16, (3, 3, 3), (2, 2, 2), None),
    ((2, 8, 16, 32, 32), torch.float32, None, None, (5, 7, 7)),
    ((2, 4, 8, 56, 56), torch.bfloat16, (2, 2, 2), (2, 2, 2), None),
]


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s" % ("x".join(map(str, c[0])),
                                                                 str(c[1]).split(".")[-1]))
@pytest.mark.parametrize("overlap", [2, -1], ids=["ordered", "any"])
def test_graph_replay(case, overlap):
    shape, dt, k, s, out = case
    g = torch.Generator().manual_seed(11)
    xs = [torch.randn(shape, generator=g).to(dt).cuda() for _ in range(3)]
    x = xs[0].clone()
    y, idx = (mp.mp3d_forward(x, k, s) if k else mp.amp3d_forward(x, out))
    gy = torch.randn(tuple(y.shape), generator=g).to(dt).cuda()
    gx = torch.empty_like(x)

    def step():
        if k:
            mp.mp3d_forward(x, k, s, out=(y, idx))
        else:
            mp.amp3d_forward(x, out, out=(y, idx))
        mp.mp3d_backward(gy, idx, shape, kernel=k, stride=s, overlap=overlap, out=gx)

    refs = []
    for xi in xs:
        x.copy_(xi)
        step()
        torch.cuda.synchronize()
        refs.append((y.clone(), idx.clone(), gx.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(xi)
            y.fill_(0)
            idx.fill_(-1)
            gx.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            ry, ri, rgx = refs[i]
            assert torch.equal(_bits(y), _bits(ry)), "replay %d input %d: y" % (rep, i)
            assert torch.equal(idx, ri), "replay %d input %d: idx" % (rep, i)
            if overlap == 2:
                assert torch.equal(_bits(gx), _bits(rgx)), "replay %d input %d: gx" % (rep, i)
            else:
                # any order: the same sums up to the order of the additions
                assert bool(torch.isfinite(gx.float()).all()), "replay %d input %d: gx" % (rep, i)
                torch.testing.assert_close(gx.float(), rgx.float(), rtol=1e-2, atol=1e-3)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s" % ("x".join(map(str, c[0])),
                                                                 str(c[1]).split(".")[-1]))
@pytest.mark.parametrize("form", ["one-pass", "two-pass"])
def test_graph_replay_index_free(case, form, monkeypatch):
    """The values-only forward and the index-free backward (one pass, or two
    through a workspace the caller allocated before capture) under capture:
    every replay equals the eager calls bit for bit (ordered mode)."""
    shape, dt, k, s, out = case
    if form == "two-pass":
        monkeypatch.setenv("MP3D_TWO_PASS", "1")
    g = torch.Generator().manual_seed(12)
    xs = [torch.randn(shape, generator=g).to(dt).cuda() for _ in range(3)]
    x = xs[0].clone()
    y = mp.mp3d_forward(x, k, s, indices=False) if k else mp.amp3d_forward(x, out, indices=False)
    gy = torch.randn(tuple(y.shape), generator=g).to(dt).cuda()
    gx = torch.empty_like(x)
    ws = None
    if form == "two-pass":
        ws = torch.empty(mp.recompute_workspace_size(dt, *shape[:2], tuple(y.shape[2:])),
                         dtype=torch.uint8, device="cuda")
    geo = dict(kernel=k, stride=s) if k else dict(kernel=None)

    def step():
        if k:
            mp.mp3d_forward(x, k, s, out=y, indices=False)
        else:
            mp.amp3d_forward(x, out, out=y, indices=False)
        mp.mp3d_backward_recompute(x, y, gy, overlap=2, out=gx, workspace=ws, **geo)

    refs = []
    for xi in xs:
        x.copy_(xi)
        step()
        torch.cuda.synchronize()
        refs.append((y.clone(), gx.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(xi)
            y.fill_(0)
            gx.fill_(float("nan"))
            if ws is not None:
                ws.fill_(0xFF)
            graph.replay()
            torch.cuda.synchronize()
            ry, rgx = refs[i]
            assert torch.equal(_bits(y), _bits(ry)), "replay %d input %d: y" % (rep, i)
            assert torch.equal(_bits(gx), _bits(rgx)), "replay %d input %d: gx" % (rep, i)
