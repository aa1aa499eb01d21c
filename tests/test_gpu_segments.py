"""GPU fused multi-projection GEMV (nvfp4_gemv_segments) against the oracle:
every segment of one launch within |y - y_ref| <= 1e-3 sum|w x| + 1e-6, on
the decode layer's q|k|v and gate|up groups, on ragged row counts and K that
take each kernel (vector ALU for M <= 2, the matrix-core kernels for K % 512
== 0 and otherwise), the eight-segment maximum, empty segments and
determinism."""
import numpy as np
import pytest

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


def random_mats(seed, Ns, K):
    mats = []
    for i, N in enumerate(Ns):
        codes, scales = workloads.random_nvfp4(11, seed, i, N, K)
        g = np.float32(0.01 * (i + 1))
        mats.append((codes, scales, g))
    return mats


def run_and_check(mats, x, what):
    dmats = [(dev(c), dev(s), dev(np.array([g], np.float32))) for c, s, g in mats]
    ys = [host(y) for y in nv.gemv_segments(dmats, dev_x(x))]
    worst = 0.0
    for i, ((c, s, g), y) in enumerate(zip(mats, ys)):
        y_ref, ad = oracle.gemv(c, s, g, x)
        worst = max(worst, check_tol(y, y_ref, ad, f"{what} segment {i}"))
    return ys, worst


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("Ns,K", [((333, 16, 1000), 96), ((257, 31, 64), 2048),
                                  ((130, 1, 515, 48), 4096), ((5, 700), 2080)])
def test_ragged_segments(M, Ns, K):
    say(f"[segments] M={M} Ns={Ns} K={K}")
    mats = random_mats(M * 31 + K, Ns, K)
    x = workloads.x_bf16(11, M, K, M, K)
    run_and_check(mats, x, f"M={M} K={K}")


@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_decode_layer_groups(M):
    """q|k|v (4096 + 1024 + 1024 rows) and gate|up (2 x 12288 rows), K = 4096,
    packed from the decode-layer workload's weights."""
    names = dict((n, (N, K)) for n, N, K in workloads.DECODE_LAYER)
    for group in (("q", "k", "v"), ("gate", "up")):
        mats = []
        for name in group:
            si = [n for n, _, _ in workloads.DECODE_LAYER].index(name)
            N, K = names[name]
            mats.append(oracle.pack(workloads.dense_weights(2, 0, si, N, K)))
        x = workloads.x_bf16(2, 0, 100 + M, M, 4096)
        say(f"[segments] decode layer {'|'.join(group)} M={M}")
        _, worst = run_and_check(mats, x, "|".join(group))
        say(f"  max err / tol = {worst:.3e}")


def test_eight_segments_and_empty():
    K, M = 512, 4
    Ns = (16, 0, 17, 3, 0, 64, 1, 100)
    mats = random_mats(77, Ns, K)
    x = workloads.x_bf16(11, 77, 0, M, K)
    ys, _ = run_and_check([m for m, N in zip(mats, Ns)], x, "eight segments")
    assert [y.shape for y in ys] == [(M, N) for N in Ns]


def test_matches_separate_calls_and_is_deterministic():
    K, M = 4096, 5
    mats = random_mats(5, (4096, 1024, 1024), K)
    x = workloads.x_bf16(11, 5, 1, M, K)
    dmats = [(dev(c), dev(s), dev(np.array([g], np.float32))) for c, s, g in mats]
    xd = dev_x(x)
    a = [host(y) for y in nv.gemv_segments(dmats, xd)]
    b = [host(y) for y in nv.gemv_segments(dmats, xd)]
    for ya, yb in zip(a, b):
        assert np.array_equal(ya, yb)
    for (c, s, g), (hc, hs, hg), ya in zip(dmats, mats, a):
        y1 = host(nv.gemv(c, s, g, xd))
        # the same definition in a different launch shape (summation order):
        # the two agree within twice the bound of one
        _, ad = oracle.gemv(hc, hs, hg, x)
        assert np.all(np.abs(ya.astype(np.float64) - y1) <= 2e-3 * ad + 2e-6)
