import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_path(name):
    return os.path.join(GOLDEN, name)


def golden_rows(name):
    """Non-comment, non-empty lines of a golden file, split on whitespace
    (text after '#' is dropped)."""
    out = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def pack_cases():
    """Parse tests/golden/pack_examples.txt into a list of dicts."""
    import numpy as np
    cases, cur = [], None
    for tok in golden_rows("pack_examples.txt"):
        key = tok[0]
        if key == "case":
            cur = {"name": tok[1], "rows": {}, "scales": {}, "codes": {}, "dequant": {}}
        elif key == "override":
            cur["override"] = None if tok[1] == "none" else float(tok[1])
        elif key == "shape":
            cur["N"], cur["K"] = int(tok[1]), int(tok[2])
        elif key == "row":
            cur["rows"][int(tok[1])] = [float(v) for v in tok[2:]]
        elif key == "expect_g":
            cur["g"] = float(tok[1])
        elif key == "expect_scales":
            cur["scales"][int(tok[1])] = [int(v, 16) for v in tok[2:]]
        elif key == "expect_codes":
            cur["codes"][int(tok[1])] = [int(v, 16) for v in tok[2:]]
        elif key == "expect_dequant":
            cur["dequant"][int(tok[1])] = [float(v) for v in tok[2:]]
        elif key == "end":
            N, K = cur["N"], cur["K"]
            cur["W"] = np.array([cur["rows"][n] for n in range(N)], np.float32)
            cur["exp_scales"] = np.array([cur["scales"][n] for n in range(N)], np.uint8)
            cur["exp_codes"] = np.array([cur["codes"][n] for n in range(N)], np.uint8)
            cur["exp_dequant"] = np.array([cur["dequant"][n] for n in range(N)], np.float32)
            assert cur["W"].shape == (N, K)
            assert cur["exp_codes"].shape == (N, K // 2)
            assert cur["exp_scales"].shape == (N, K // 16)
            cases.append(cur)
            cur = None
    return cases


@pytest.fixture(scope="session")
def oracle():
    import oracle as _o
    _o.lib()
    return _o
