"""GPU GEMV at 2 <= M <= 8 on very tall single matrices (2^17 rows and more,
K a multiple of 256 up to 4096), where the wavefronts split the rows (two or
three whole 16-row tiles each) and x sits once per workgroup in LDS, against
the oracle within |y - y_ref| <= 1e-3 sum|w x| + 1e-6: the LM head at every
token count (every output), and ragged shapes whose last tile is partial or
whose launch needs more than one workgroup per CU (rows sampled at the first
and last rows, around the first wavefronts' row boundaries and at random)."""
import numpy as np
import pytest

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


def wave_first_rows(N, waves):
    """First rows of wavefronts 0 .. waves - 1 in the launch: 16 wavefronts
    per workgroup, at least 256 workgroups, at most three tiles per
    wavefront; wavefront v takes tiles [v T / W, (v + 1) T / W)."""
    T = -(-N // 16)
    grid = max(256, -(-T // 48))
    W = 16 * grid
    return [16 * (v * T // W) for v in range(waves)]


def sample_rows(N, n, seed):
    fixed = [0, 1, 15, 16, 31, 32]
    for b in wave_first_rows(N, 6)[1:] + wave_first_rows(N, 300)[-2:]:
        fixed += [b - 1, b, b + 1, b + 15, b + 16]
    fixed += [N - 17, N - 16, N - 2, N - 1]
    fixed = [r for r in fixed if 0 <= r < N]
    return np.unique(np.concatenate([fixed, np.random.default_rng(seed).choice(N, n, replace=False)]))


def compare(y, c, s, g, x, rows, what):
    y_ref, ad = oracle.gemv(c, s, g, x, rows=rows)
    r = check_tol(y[:, rows], y_ref, ad, what)
    say(f"  {what}: max err / tol = {r:.3e}")


@pytest.fixture(scope="module")
def lm_head_packed():
    W = workloads.dense_weights(3, 0, 0, 151936, 4096)
    return oracle.pack(W), nv.pack(dev(W))


@pytest.mark.parametrize("M", [2, 3, 4, 5, 6, 7, 8])
def test_lm_head_up_to_eight_tokens(lm_head_packed, M):
    """Every output of the LM head against the oracle."""
    N, K = 151936, 4096
    say(f"[gemv-tall] LM head {N}x{K} M={M}")
    (c0, s0, g0), (c1, s1, g1) = lm_head_packed
    x = workloads.x_bf16(3, 3, M, M, K)
    y = host(nv.gemv(c1, s1, g1, dev_x(x)))
    y_ref, ad = oracle.gemv(c0, s0, g0, x)
    r = check_tol(y, y_ref, ad, f"LM head M={M}")
    say(f"  LM head M={M}: max err / tol = {r:.3e}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("M,N,K", [(8, 131072, 256), (3, 131073, 1024), (5, 200003, 4096),
                                   (8, 393217, 512), (7, 150001, 2304), (2, 140007, 3072)])
def test_tall_ragged_shapes(M, N, K):
    """Two tiles per wavefront exactly (131072 rows), a last tile of one row
    (131073, 150001), 261 workgroups at 2.99 tiles per wavefront (200003),
    513 workgroups (two per CU and more), K = 2304 (9 slices: the ring's
    last round half empty), and two tokens with a last tile of 7 rows."""
    say(f"[gemv-tall] ragged M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(17, M, N % 1000 + K, N, K)
    x = workloads.x_bf16(17, M, N % 1000 + K, M, K)
    g = np.float32(0.0123)
    y = host(nv.gemv(dev(codes), dev(scales), dev(np.array([g], np.float32)), dev_x(x)))
    compare(y, codes, scales, g, x, sample_rows(N, 600, N), f"{N}x{K} M={M}")
    assert np.all(np.isfinite(y))


def test_tall_deterministic(lm_head_packed):
    """Two calls give the same bits."""
    _, (c1, s1, g1) = lm_head_packed
    x = dev_x(workloads.x_bf16(3, 4, 0, 8, 4096))
    a = host(nv.gemv(c1, s1, g1, x))
    b = host(nv.gemv(c1, s1, g1, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
