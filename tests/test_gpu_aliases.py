"""The sketch's Python names give the same bits as the C-ABI names they
alias, on one fixed, one adaptive and one ordered case."""
import pytest
import torch

import _pins
import bwd_max_pool3d_amd as mp

pytestmark = pytest.mark.gpu


def _x(shape, seed):
    return _pins.from_storage(_pins.draw(shape, 1, "ties", seed), 1).cuda()   # float16


def test_fixed_alias():
    x = _x((2, 3, 9, 10, 11), 71)
    y, idx = mp.max_pool3d(x, 3, 2)
    y2, idx2 = mp.mp3d_forward(x, 3, 2)
    assert torch.equal(idx, idx2) and torch.equal(y.view(torch.int16), y2.view(torch.int16))
    gy = _x(tuple(y.shape), 72)
    for ov, code in ((None, -1), (True, 1), (2, 2)):
        a = mp.max_pool3d_backward(gy, idx, x.shape, 3, 2, overlap=ov)
        b = mp.mp3d_backward(gy, idx, x.shape, 3, 2, overlap=code)
        if code == 2 or ov is None:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        else:
            # accumulate: the sum order is free; cells of <= 2 terms are
            # exact either way, and small integer gradients sum exactly
            assert torch.equal(a.float(), b.float())


def test_adaptive_alias_and_gather():
    x = _x((1, 4, 8, 8, 8), 73)
    y, idx = mp.adaptive_max_pool3d(x, (4, 4, 4))
    y2, idx2 = mp.amp3d_forward(x, (4, 4, 4))
    assert torch.equal(idx, idx2) and torch.equal(y.view(torch.int16), y2.view(torch.int16))
    gy = _x(tuple(y.shape), 74)
    a = mp.max_pool3d_backward(gy, idx, x.shape, overlap=False)     # windows tile: the gather
    b = mp.mp3d_backward(gy, idx, x.shape, overlap=0)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
