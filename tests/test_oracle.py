"""The CPU oracle against its pins (see tests/_pins.py for what each pin
checks and where the fact comes from).  CPU only."""
import pytest

import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_on_pr308_shapes(orc):
    """The oracle's forward equals the numpy first-occurrence formulation on
    every shape printed on the PR #308 page (tests/golden/pr308_shapes.txt),
    including its output-larger-than-input case."""
    import numpy as np
    import _golden
    codes = {"float32": 0, "float16": 1, "bfloat16": 2}
    for i, (kind, dt, shape, out) in enumerate(_golden.pr308_cases()):
        code = codes[dt]
        x = _pins.draw(shape, code, "ties", 700 + i)
        y, idx = orc.forward(x, code, out)
        by, bidx = _pins.brute_forward(x, code, out, (0, 0, 0), (0, 0, 0))
        assert np.array_equal(idx, bidx), (kind, dt, shape, out)
        assert np.array_equal(y, by)
