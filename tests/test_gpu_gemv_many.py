"""GPU GEMV at 9 <= M <= 128 tokens (the many-token matrix-core kernel; at
9 <= M <= 16 below 2^17 rows with K a multiple of 256, the eight-token
kernel in two token groups) against the oracle within
|y - y_ref| <= 1e-3 sum|w x| + 1e-6: the stress and
LM-head shapes at M in {9, 12, 16, 24, 32, 64, 128} (sampled rows where the
oracle would take long), ragged token counts, rows and K, arbitrary codes and
scales, segments, the W4A4 path at many tokens, and determinism."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu

MANY = [9, 12, 16, 24, 32, 64, 128]


def sample_rows(N, n, seed):
    """n random rows plus the first and last rows and both sides of the
    tile boundaries at the start."""
    if N <= n:
        return None
    fixed = [r for r in (0, 15, 16, 31, 32, 63, 64, N - 17, N - 16, N - 1) if 0 <= r < N]
    return np.unique(np.concatenate([fixed, np.random.default_rng(seed).choice(N, n, replace=False)]))


def compare(y, c, s, g, x, rows, what):
    y_ref, ad = oracle.gemv(c, s, g, x, rows=rows)
    r = check_tol(y if rows is None else y[:, rows], y_ref, ad, what)
    say(f"  {what}: max err / tol = {r:.3e}")


@pytest.fixture(scope="module")
def stress_packed():
    """The stress workload's two matrices (Student-t, 1% zero blocks), packed
    by the oracle and by the GPU (byte-identical)."""
    out = []
    for i, (_, N, K) in enumerate(workloads.WORKLOADS[5]["mats"]):
        W = workloads.dense_weights(5, 0, i, N, K)
        h = oracle.pack(W)
        d = nv.pack(dev(W))
        assert np.array_equal(host(d[0]), h[0]) and np.array_equal(host(d[1]), h[1])
        out.append((h, d, N, K))
    return out


@pytest.mark.parametrize("M", MANY)
def test_stress_shapes_many_tokens(stress_packed, M):
    for j, ((c0, s0, g0), (c1, s1, g1), N, K) in enumerate(stress_packed):
        say(f"[gemv-many] stress {N}x{K} M={M}")
        x = workloads.x_bf16(5, 1, 10 * M + j, M, K)
        y = host(nv.gemv(c1, s1, g1, dev_x(x)))
        rows = sample_rows(N, 1500, M) if M > 16 else None
        compare(y, c0, s0, g0, x, rows, f"{N}x{K} M={M}")


@pytest.fixture(scope="module")
def lm_head_packed():
    W = workloads.dense_weights(3, 0, 0, 151936, 4096)
    return oracle.pack(W), nv.pack(dev(W))


@pytest.mark.parametrize("M", MANY)
def test_lm_head_many_tokens(lm_head_packed, M):
    N, K = 151936, 4096
    say(f"[gemv-many] LM head {N}x{K} M={M}")
    (c0, s0, g0), (c1, s1, g1) = lm_head_packed
    x = workloads.x_bf16(3, 2, M, M, K)
    y = host(nv.gemv(c1, s1, g1, dev_x(x)))
    compare(y, c0, s0, g0, x, sample_rows(N, 600, M), f"LM head M={M}")


@pytest.mark.parametrize("M", [9, 13, 17, 31, 33, 47, 100, 127, 128])
@pytest.mark.parametrize("N,K", [(1, 32), (15, 96), (37, 160), (130, 4096), (513, 2080),
                                 (64, 12288), (2000, 1024)])
def test_ragged_shapes(M, N, K):
    """Token counts that leave a partial group of 16, rows that leave a
    partial tile, K with a partial last 128-k step (32 and 96 and 160 and
    2080 are not multiples of 128), one row, and a K split in which some
    wavefronts get no step at all (K = 32, 96)."""
    say(f"[gemv-many] ragged M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(11, M, N * 5 + K, N, K)
    x = workloads.x_bf16(11, M, N * 5 + K, M, K)
    g = np.float32(0.017)
    y = run(codes, scales, g, x)
    compare(y, codes, scales, g, x, None, f"M={M} N={N} K={K}")


def run(codes, scales, g, x):
    return host(nv.gemv(dev(codes), dev(scales), dev(np.array([g], np.float32)), dev_x(x)))


@pytest.mark.parametrize("M", [16, 128])
def test_subnormal_and_max_scales_many(M):
    N, K = 300, 1024
    for lo, hi in [(0x00, 0x07), (0x78, 0x7E)]:
        codes, scales = workloads.random_nvfp4(12, M, lo, N, K, lo, hi)
        x = workloads.x_bf16(12, M, lo, M, K)
        y = run(codes, scales, 1.0, x)
        compare(y, codes, scales, 1.0, x, None, f"M={M} scales {lo:#x}-{hi:#x}")


def test_closed_form_all_ones_many():
    """Every weight 1 (code 0x2, scale 0x38, g = 1) and x = 1: y = K exactly."""
    for M, K in [(9, 32), (16, 4096), (128, 12288)]:
        N = 77
        codes = np.full((N, K // 2), 0x22, np.uint8)
        scales = np.full((N, K // 16), 0x38, np.uint8)
        x = np.full((M, K), 0x3F80, np.uint16)
        y = run(codes, scales, 1.0, x)
        assert np.all(y == K), (M, K, y.min(), y.max())


@pytest.mark.parametrize("M", [12, 40, 128])
def test_segments_many_tokens(M):
    """q|k|v-like segments of ragged sizes in one launch at many tokens, each
    output checked against the oracle."""
    K = 512
    Ns = [300, 77, 77, 1]
    mats, host_mats = [], []
    for i, N in enumerate(Ns):
        c, s = workloads.random_nvfp4(13, M, i, N, K)
        g = np.float32(0.01 * (i + 1))
        host_mats.append((c, s, g))
        mats.append((dev(c), dev(s), dev(np.array([g], np.float32))))
    x = workloads.x_bf16(13, M, 99, M, K)
    ys = nv.gemv_segments(mats, dev_x(x))
    for (c, s, g), y in zip(host_mats, ys):
        compare(host(y), c, s, g, x, None, f"segment N={c.shape[0]} M={M}")


@pytest.mark.parametrize("M", [9, 64, 128])
def test_w4a4_many_tokens(M):
    """W4A4 at many tokens: the activations quantized with a static scale,
    decoded once into the workspace and multiplied by the many-token kernel."""
    N, K = 700, 2048
    W = workloads.normal_weights(14, M, 0, N, K)
    (cw, sw, gw), (dcw, dsw, dgw) = oracle.pack(W), nv.pack(dev(W))
    xb = workloads.x_bf16(14, M, 1, M, K)
    calib = workloads.x_bf16(14, M + 1, 1, M, K)
    gx = np.float32(np.abs((calib.astype(np.uint32) << 16).view(np.float32)).max() / 2688.0)
    dgx = dev(np.array([gx], np.float32))
    cx, sx = nv.quantize_act(dev_x(xb), dgx)
    hcx, hsx = oracle.quantize_act(xb, gx)
    assert np.array_equal(host(cx), hcx) and np.array_equal(host(sx), hsx)
    y = host(nv.gemv_w4a4(dcw, dsw, dgw, cx, sx, dgx))
    y_ref, ad = oracle.gemv_w4a4(cw, sw, gw, hcx, hsx, gx)
    r = check_tol(y, y_ref, ad, f"w4a4 M={M}")
    say(f"  w4a4 M={M}: max err / tol = {r:.3e}")


def test_deterministic_many_tokens():
    """The same call twice gives bit-identical outputs (fixed reduction order)."""
    M, N, K = 64, 4096, 4096
    codes, scales = workloads.random_nvfp4(15, 0, 0, N, K)
    x = dev_x(workloads.x_bf16(15, 0, 0, M, K))
    c, s, g = dev(codes), dev(scales), dev(np.array([0.02], np.float32))
    a = host(nv.gemv(c, s, g, x))
    b = host(nv.gemv(c, s, g, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
