"""Pins for the oracle's GEMV (CPU only): brute force against a numpy fp64
matmul of the test-side decode, closed forms and invariants."""
import numpy as np
import pytest

import workloads
from refdecode import bf16_value, decode

ONE_BF16 = 0x3F80


@pytest.mark.parametrize("M,N,K", [(1, 7, 32), (3, 16, 64), (8, 33, 96), (5, 64, 48),
                                   (17, 9, 160), (128, 5, 64)])
def test_gemv_brute_force(oracle, M, N, K):
    W = workloads.normal_weights(1, 10 + M, 0, N, K)
    codes, scales, g = oracle.pack(W)
    x = workloads.x_bf16(1, 10 + M, 0, M, K)
    y, ad = oracle.gemv(codes, scales, g, x)
    Wd = decode(codes, scales)                 # fp64 e2m1*s
    xv = bf16_value(x)                         # fp64
    ref = float(g) * (xv @ Wd.T)               # library matmul
    aref = float(g) * (np.abs(xv) @ np.abs(Wd).T)
    assert y.shape == (M, N)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * aref.max() + 1e-300)
    np.testing.assert_allclose(ad, aref, rtol=1e-12)


def test_gemv_closed_form_all_ones(oracle):
    N, K = 5, 4096
    codes = np.full((N, K // 2), 0x22, np.uint8)     # every element 1.0
    scales = np.full((N, K // 16), 0x38, np.uint8)   # every scale 1.0
    x = np.full((2, K), ONE_BF16, np.uint16)
    y, ad = oracle.gemv(codes, scales, 1.0, x)
    assert np.all(y == K) and np.all(ad == K)
    y, _ = oracle.gemv(codes, scales, 0.25, x)
    assert np.all(y == K / 4)


def test_gemv_single_weight(oracle):
    N, K = 3, 64
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    codes[1, 37 // 2] = 0xD << 4                     # element 37 = -3.0
    scales[1, 37 // 16] = 0x3A                       # 1.25
    x = np.zeros((1, K), np.uint16)
    x[0, 37] = 0x4040                                # 3.0
    y, _ = oracle.gemv(codes, scales, 2.0, x)
    assert y[0, 1] == -3.0 * 1.25 * 3.0 * 2.0
    assert y[0, 0] == 0 and y[0, 2] == 0


def test_gemv_alternating_signs_cancel(oracle):
    N, K = 4, 512
    codes = np.full((N, K // 2), 0xA2, np.uint8)     # +1, -1, +1, -1, ...
    scales = np.full((N, K // 16), 0x40, np.uint8)
    x = np.full((3, K), 0x3FC0, np.uint16)           # 1.5
    y, ad = oracle.gemv(codes, scales, 1.0, x)
    assert np.all(y == 0) and np.all(ad == K * 2 * 1.5)


def test_gemv_row_subset_matches_full(oracle):
    N, K, M = 50, 128, 4
    W = workloads.normal_weights(1, 20, 0, N, K)
    codes, scales, g = oracle.pack(W)
    x = workloads.x_bf16(1, 20, 0, M, K)
    y, ad = oracle.gemv(codes, scales, g, x)
    rows = np.array([49, 0, 17, 17, 3])
    ys, ads = oracle.gemv(codes, scales, g, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(ads, ad[:, rows])
    with pytest.raises(ValueError):
        oracle.gemv(codes, scales, g, x, rows=[N])


def test_gemv_rows_are_independent_of_m(oracle):
    N, K = 20, 64
    W = workloads.normal_weights(1, 21, 0, N, K)
    codes, scales, g = oracle.pack(W)
    x = workloads.x_bf16(1, 21, 0, 6, K)
    y, _ = oracle.gemv(codes, scales, g, x)
    for m in range(6):
        y1, _ = oracle.gemv(codes, scales, g, x[m:m + 1])
        assert np.array_equal(y1[0], y[m])
