"""Weights larger than 4 GiB: every GEMV path, the segmented GEMV, W4A4 and
the MoE reach rows and experts whose byte offsets lie past 2^32 (codes) and
2^31 (scales). The weight bytes are drawn on the device from a seeded
generator (every row distinct, so a wrapped offset reads the wrong row); the
oracle gets the sampled rows and the routed experts copied back, and checks
the output within |y - y_ref| <= 1e-3 sum|w x| + 1e-6."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


def device_nvfp4(seed, N, K, lo=0x30, hi=0x48):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    c = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    s = torch.randint(lo, hi, (N, K // 16), dtype=torch.uint8, device="cuda", generator=g)
    return c, s


def sample_rows(N, K, seed):
    """First, last and random rows, and the rows on both sides of every
    power-of-two byte offset from 2^31 up, in the codes and in the scales."""
    rows = [0, 1, N - 2, N - 1]
    for per_row in (K // 2, K // 16):
        p = 31
        while (1 << p) // per_row < N:
            b = (1 << p) // per_row
            rows += [b - 1, b] if b > 0 else [b]
            p += 1
    rows += list(np.random.default_rng(seed).choice(N, 120, replace=False))
    return np.unique(np.array(rows, np.int64))


def rows_to_host(t, rows):
    return host(t[torch.from_numpy(rows).to("cuda")])


def release():
    """Return the device memory of tensors the caller has deleted."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_k256():
    """2.2 M rows x K = 16384: 18 GB of codes, 2.25 GB of scales."""
    N, K = 2_200_000, 16384
    say(f"[large] drawing {N}x{K} on the device")
    c, s = device_nvfp4(11, N, K)
    rows = sample_rows(N, K, 5)
    yield c, s, N, K, rows, rows_to_host(c, rows), rows_to_host(s, rows)
    del c, s
    release()


@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_large_gemv_vector_alu_and_split_k(big_k256, M):
    """M <= 2: the vector-ALU kernel (four rows per wavefront); M >= 3: the
    split-K matrix-core kernel streaming x (64 slices)."""
    c, s, N, K, rows, hc, hs = big_k256
    say(f"[large] gemv M={M} N={N} K={K}")
    g = np.float32(0.0091)
    x = workloads.x_bf16(9, 500 + M, 0, M, K)
    y = nv.gemv(c, s, dev(np.array([g], np.float32)), dev_x(x))
    y_rows = host(y[:, torch.from_numpy(rows).to("cuda")])
    y_ref, ad = oracle.gemv(hc, hs, g, x)
    check_tol(y_rows, y_ref, ad, f"large gemv M={M}")
    assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("M", [3, 8])
def test_large_tall_eight_tokens(M):
    """2.2 M rows x K = 4096 (4.5 GB of codes): the row-split matrix-core
    kernel for 3 <= M <= 8, whose wavefronts take two or three whole tiles
    from 45840 (2865 workgroups), with rows on both sides of the 2^31 and
    2^32 byte offsets of the codes."""
    N, K = 2_200_000, 4096
    say(f"[large] tall gemv M={M} N={N} K={K}")
    c, s = device_nvfp4(13, N, K)
    rows = sample_rows(N, K, 7)
    hc, hs = rows_to_host(c, rows), rows_to_host(s, rows)
    g = np.float32(0.0077)
    x = workloads.x_bf16(9, 600 + M, 0, M, K)
    y = nv.gemv(c, s, dev(np.array([g], np.float32)), dev_x(x))
    y_rows = host(y[:, torch.from_numpy(rows).to("cuda")])
    finite = bool(torch.isfinite(y).all())
    del c, s, y
    release()
    y_ref, ad = oracle.gemv(hc, hs, g, x)
    check_tol(y_rows, y_ref, ad, f"large tall gemv M={M}")
    assert finite


@pytest.mark.parametrize("M", [2, 5])
def test_large_segments(big_k256, M):
    """The large matrix as the second segment of one launch."""
    c, s, N, K, rows, hc, hs = big_k256
    say(f"[large] segments M={M}")
    cs, ss = workloads.random_nvfp4(9, 600 + M, 0, 1000, K)
    g0, g1 = np.float32(0.02), np.float32(0.0091)
    x = workloads.x_bf16(9, 600 + M, 1, M, K)
    ys = nv.gemv_segments([(dev(cs), dev(ss), dev(np.array([g0], np.float32))),
                           (c, s, dev(np.array([g1], np.float32)))], dev_x(x))
    y0_ref, ad0 = oracle.gemv(cs, ss, g0, x)
    check_tol(host(ys[0]), y0_ref, ad0, f"segments M={M} small")
    y1 = host(ys[1][:, torch.from_numpy(rows).to("cuda")])
    y1_ref, ad1 = oracle.gemv(hc, hs, g1, x)
    check_tol(y1, y1_ref, ad1, f"segments M={M} large")


@pytest.mark.parametrize("M", [2, 4])
def test_large_w4a4(big_k256, M):
    """M = 2: activations decoded in registers; M = 4: the decoded bf16
    activations through the matrix-core kernel."""
    c, s, N, K, rows, hc, hs = big_k256
    say(f"[large] w4a4 M={M}")
    g = np.float32(0.0091)
    x = workloads.x_bf16(9, 700 + M, 0, M, K)
    gx = np.float32(np.abs(workloads.x_bf16(9, 700 + M, 1, M, K).astype(np.uint32) << 16)
                    .view(np.float32).max() / 2688.0)
    cx, sx = oracle.quantize_act(x, gx)
    y = nv.gemv_w4a4(c, s, dev(np.array([g], np.float32)), dev(cx), dev(sx),
                     dev(np.array([gx], np.float32)))
    y_rows = host(y[:, torch.from_numpy(rows).to("cuda")])
    y_ref, ad = oracle.gemv_w4a4(hc, hs, g, cx, sx, gx)
    check_tol(y_rows, y_ref, ad, f"large w4a4 M={M}")


@pytest.mark.parametrize("M", [1, 3])
def test_large_gemv_other_k(M):
    """K = 16416 (not a multiple of 256): the vector-ALU kernel at M = 1 and
    the chunked matrix-core kernel at M = 3; 17 GB of codes, 2.2 GB of
    scales."""
    N, K = 2_100_000, 16416
    say(f"[large] gemv other-K M={M} N={N} K={K}")
    c, s = device_nvfp4(12 + M, N, K)
    rows = sample_rows(N, K, 6)
    hc, hs = rows_to_host(c, rows), rows_to_host(s, rows)
    g = np.float32(0.0117)
    x = workloads.x_bf16(9, 800 + M, 0, M, K)
    y = nv.gemv(c, s, dev(np.array([g], np.float32)), dev_x(x))
    y_rows = host(y[:, torch.from_numpy(rows).to("cuda")])
    del c, s, y
    release()
    y_ref, ad = oracle.gemv(hc, hs, g, x)
    check_tol(y_rows, y_ref, ad, f"large other-K M={M}")


@pytest.mark.parametrize("M", [1, 3])
def test_large_moe(M):
    """1024 experts (gate|up 3072x4096, down 4096x1536): 6.4 GB of gate|up
    codes and 3.2 GB of down codes; the routed experts include the last ones,
    whose gate|up rows start past 2^32 bytes."""
    E, H, I, topk = 1024, 4096, 1536, 8
    say(f"[large] moe E={E} M={M}")
    c13, s13 = device_nvfp4(21, E * 2 * I, H, 0x30, 0x40)
    c2, s2 = device_nvfp4(22, E * H, I, 0x30, 0x40)
    c13, s13 = c13.view(E, 2 * I, H // 2), s13.view(E, 2 * I, H // 16)
    c2, s2 = c2.view(E, H, I // 2), s2.view(E, H, I // 16)
    rng = np.random.default_rng(30 + M)
    g13 = (0.005 + 0.01 * rng.random(E)).astype(np.float32)
    g2 = (0.005 + 0.01 * rng.random(E)).astype(np.float32)
    ids = np.stack([rng.choice(np.r_[np.arange(8), np.arange(680, E)], topk, replace=False)
                    for _ in range(M)]).astype(np.int32)
    ids[0, :2] = [E - 1, 1000]
    z = rng.standard_normal((M, topk))
    gw = (np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)).astype(np.float32)
    x = workloads.x_bf16(9, 900 + M, 0, M, H)
    y = host(nv.moe_gemv(c13, s13, dev(g13), c2, s2, dev(g2), dev_x(x), dev(ids), dev(gw)))
    used = np.unique(ids)
    sel = torch.from_numpy(used.astype(np.int64)).to("cuda")
    hw = (host(c13[sel]), host(s13[sel]), g13[used], host(c2[sel]), host(s2[sel]), g2[used])
    del c13, s13, c2, s2, sel
    release()
    remap = np.searchsorted(used, ids).astype(np.int32)
    y_ref, bound = oracle.moe(*hw, x, remap, gw)
    check_tol(y, y_ref, bound, f"large moe M={M}")
