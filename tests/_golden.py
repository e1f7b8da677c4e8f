"""Reader for the text fixtures under tests/golden/ (each file states the
page and section its values come from)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pr308_shapes():
    """[(kind, dtype, (N,C,D,H,W), (OD,OH,OW) or None)] from pr308_shapes.txt."""
    rows = []
    with open(os.path.join(GOLDEN, "pr308_shapes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if not line:
                continue
            kind, dt, *nums = line
            nums = [int(v) for v in nums]
            out = tuple(nums[5:8])
            rows.append((kind, dt, tuple(nums[:5]), out if any(out) else None))
    return rows


def pr308_cases():
    """Adaptive cases built from the fixture: each printed shape with the
    printed output size where there is one, else with one output size that
    divides every axis (the gather path) and one that does not (overlap)."""
    cases = []
    for kind, dt, shape, out in pr308_shapes():
        if out is not None:
            cases.append((kind, dt, shape, out))
            continue
        D, H, W = shape[2:]
        cases.append((kind, dt, shape, (max(D // 2, 1), max(H // 2, 1), max(W // 2, 1))))
        cases.append((kind, dt, shape, (3, 3, 3)))
    return cases
