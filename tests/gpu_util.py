"""Helpers for the GPU parity tests: device transfer and the tolerance check.
Expected values come only from the oracle (oracle/), never from the GPU."""
import numpy as np
import torch

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_x(x_bits: np.ndarray) -> torch.Tensor:
    """bf16 device tensor holding the given bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(
        torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_tol(y, y_ref, absdot, what=""):
    """|y - y_ref| <= 1e-3 * sum|w x| + 1e-6, elementwise (fp32 y, fp64 ref).
    Returns the largest error as a fraction of the bound."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    tol = 1e-3 * absdot + 1e-6
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)}: y={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} "
                             f"tol={tol[tuple(i)]!r}")
    return float((err / tol).max()) if err.size else 0.0


def say(*a):
    print(*a, flush=True)
