"""Test-side NVFP4 decode, independent of the oracle's C code: E2M1 values
come from the hand-enumerated golden table, E4M3 values from torch's
float8_e4m3fn conversion. Used to brute-force the oracle's GEMV and MoE."""
import numpy as np
import torch

from conftest import golden_rows

E2M1 = np.zeros(16, np.float64)
for _c, _v in golden_rows("e2m1_values.txt"):
    E2M1[int(_c, 16)] = float(_v)
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(
    torch.float32).numpy().astype(np.float64)


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e2m1 * s (no tensor scale) as fp64 [N, K]."""
    N = codes.shape[0]
    K = codes.shape[1] * 2
    nib = np.empty((N, K), np.uint8)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    return E2M1[nib] * np.repeat(E4M3[scales], 16, axis=1)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
