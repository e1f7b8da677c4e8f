"""The sketch's Python names are aliases of the C-ABI names (host only:
nothing here touches the GPU)."""
import inspect

import bwd_max_pool3d_amd as mp


def test_aliases_exported():
    for name in ("max_pool3d", "adaptive_max_pool3d", "max_pool3d_backward"):
        assert name in mp.__all__
        assert callable(getattr(mp, name))


def test_overlap_codes():
    assert mp.overlap_code(None) == -1      # the library chooses
    assert mp.overlap_code(False) == 0      # the gather
    assert mp.overlap_code(True) == 1       # accumulate
    assert mp.overlap_code(2) == 2          # ordered
    assert mp.overlap_code(-1) == -1


def test_alias_signatures_follow_the_c_names():
    fwd = inspect.signature(mp.max_pool3d).parameters
    assert list(fwd)[:3] == ["x", "kernel", "stride"]
    afwd = inspect.signature(mp.adaptive_max_pool3d).parameters
    assert list(afwd)[:2] == ["x", "out_size"]
    bwd = inspect.signature(mp.max_pool3d_backward).parameters
    assert list(bwd)[:3] == ["gy", "idx", "in_shape"]
    assert bwd["overlap"].default is None
