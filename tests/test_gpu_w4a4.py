"""GPU W4A4 against the oracle: activation quantization with a static input
scale bit for bit (calibrated and saturating scales), and the W4A4 GEMV within
|y - y_ref| <= 1e-3 sum|w x| + 1e-6 on the pages' W4A4 dense FFN (gate, up,
down 4096x4096 at M=2), on shapes that take every GEMV kernel (vector ALU
for M <= 2, the matrix-core kernels for K % 256 == 0 and otherwise), and
several matrices on the same activations in one call."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say
from refdecode import bf16_value

pytestmark = pytest.mark.gpu


def static_scale(wl, M, K):
    """A static input scale calibrated on another batch of the same
    distribution (rep 1), as an fp32."""
    calib = bf16_value(workloads.x_bf16(wl, 1, 0, M, K))
    return np.float32(np.abs(calib).max() / 2688.0)


@pytest.mark.parametrize("M,K", [(1, 32), (2, 4096), (8, 4096), (3, 12288)])
@pytest.mark.parametrize("under", [1.0, 50.0])
def test_quantize_act_bit_exact(M, K, under):
    """`under` > 1 makes the static scale too small: blocks saturate."""
    x = workloads.x_bf16(6, 0, M * 7 + K, M, K)
    gx = np.float32(static_scale(6, M, K) / under)
    say(f"[w4a4] quantize M={M} K={K} g_x={gx:.3e}")
    cx, sx = nv.quantize_act(dev_x(x), dev(np.array([gx], np.float32)))
    rc, rs = oracle.quantize_act(x, gx)
    assert np.array_equal(host(sx), rs)
    assert np.array_equal(host(cx), rc)
    if under > 1:
        assert np.any(rs == 0x7E)


def run_w4a4(cw, sw, gw, x, gx):
    """GPU: quantize x, then the W4A4 GEMV; the oracle: the same two steps."""
    gxd = dev(np.array([gx], np.float32))
    cx, sx = nv.quantize_act(dev_x(x), gxd)
    y = host(nv.gemv_w4a4(dev(cw), dev(sw), dev(np.array([gw], np.float32)), cx, sx, gxd))
    rcx, rsx = oracle.quantize_act(x, gx)
    assert np.array_equal(host(cx), rcx) and np.array_equal(host(sx), rsx)
    return y, oracle.gemv_w4a4(cw, sw, gw, rcx, rsx, gx)


@pytest.mark.parametrize("i", range(3))
def test_workload_6_w4a4_ffn(i):
    name, N, K = workloads.WORKLOADS[6]["mats"][i]
    M = workloads.WORKLOADS[6]["M"]
    say(f"[w4a4] workload 6 {name} {N}x{K} M={M}")
    W = workloads.dense_weights(6, 0, i, N, K)
    cw, sw, gw = oracle.pack(W)
    c1, s1, g1 = nv.pack(dev(W))
    assert np.array_equal(host(c1), cw) and np.array_equal(host(s1), sw)
    x = workloads.x_bf16(6, 0, 10 + i, M, K)
    y, (y_ref, ad) = run_w4a4(cw, sw, gw, x, static_scale(6, M, K))
    r = check_tol(y, y_ref, ad, f"w4a4 {name}")
    say(f"  max err / tol = {r:.3e}")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(37, 96), (257, 2048), (130, 4096), (64, 12288)])
def test_w4a4_shapes(M, N, K):
    say(f"[w4a4] M={M} N={N} K={K}")
    cw, sw = workloads.random_nvfp4(6, M, N * 5 + K, N, K, 0x20, 0x50)
    gw = np.float32(0.0173)
    x = workloads.x_bf16(6, M, N * 5 + K, M, K)
    y, (y_ref, ad) = run_w4a4(cw, sw, gw, x, static_scale(6, M, K))
    check_tol(y, y_ref, ad, f"w4a4 M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2])
def test_w4a4_four_rows_per_wavefront_with_ragged_tail(M):
    """N >= 32768 takes four rows per wavefront at M <= 2; N = 40003 leaves
    a tail of three rows."""
    N, K = 40003, 64
    say(f"[w4a4] M={M} N={N} K={K}")
    cw, sw = workloads.random_nvfp4(6, M, 77, N, K, 0x20, 0x50)
    gw = np.float32(0.0173)
    x = workloads.x_bf16(6, M, 77, M, K)
    y, (y_ref, ad) = run_w4a4(cw, sw, gw, x, static_scale(6, M, K))
    check_tol(y, y_ref, ad, f"w4a4 M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2])
def test_w4a4_scales_off_16_byte_alignment(M):
    """Activation scales 2-byte but not 16-byte aligned (the least the
    boundary accepts): the oracle's result within tolerance, and the same
    bits as with aligned scales."""
    N, K = 3001, 4096
    say(f"[w4a4] misaligned activation scales M={M} N={N} K={K}")
    cw, sw = workloads.random_nvfp4(6, M, 4242, N, K, 0x20, 0x50)
    gw = np.float32(0.0173)
    x = workloads.x_bf16(6, M, 4242, M, K)
    gx = np.float32(static_scale(6, M, K))
    cx, sx = oracle.quantize_act(x, gx)
    flat = np.zeros(sx.size + 16, np.uint8)
    flat[2:2 + sx.size] = sx.ravel()
    big = dev(flat)
    sx_off = big[2:2 + sx.size].reshape(sx.shape)
    assert sx_off.data_ptr() % 16 == (big.data_ptr() + 2) % 16 != 0
    m = (dev(cw), dev(sw), dev(np.array([gw], np.float32)))
    cxd, gxd = dev(cx), dev(np.array([gx], np.float32))
    y_off = host(nv.gemv_w4a4(*m, cxd, sx_off, gxd))
    y_al = host(nv.gemv_w4a4(*m, cxd, dev(sx), gxd))
    y_ref, ad = oracle.gemv_w4a4(cw, sw, gw, cx, sx, gx)
    check_tol(y_off, y_ref, ad, f"w4a4 misaligned scales M={M}")
    assert np.array_equal(y_off, y_al)


@pytest.mark.parametrize("M,K", [(1, 4096), (2, 4096), (3, 4096), (5, 4096), (8, 4096),
                                 (2, 1056), (5, 1056)])
def test_w4a4_segments(M, K):
    """Several matrices on the same NVFP4 activations in one call (an empty
    one among them): each output is within tolerance of the oracle's W4A4
    GEMV of its matrix and equal, bit for bit, to a separate
    nvfp4_gemv_w4a4 call (K = 1056 takes the other-K kernel at M >= 3)."""
    say(f"[w4a4] segments M={M} K={K}")
    Ns = (1000, 0, 37, 4200)
    x = workloads.x_bf16(6, M, 90 + K, M, K)
    gx = np.float32(static_scale(6, M, K))
    cx, sx = oracle.quantize_act(x, gx)
    cxd, sxd, gxd = dev(cx), dev(sx), dev(np.array([gx], np.float32))
    host_w, mats = [], []
    for i, N in enumerate(Ns):
        cw, sw = workloads.random_nvfp4(6, M, 300 + 10 * i + K, N, K, 0x20, 0x50)
        gw = np.float32(0.0173 * (i + 1))
        host_w.append((cw, sw, gw))
        mats.append((dev(cw), dev(sw), dev(np.array([gw], np.float32))))
    ys = nv.gemv_w4a4_segments(mats, cxd, sxd, gxd)
    for i, ((cw, sw, gw), m, y) in enumerate(zip(host_w, mats, ys)):
        y = host(y)
        assert y.shape == (M, Ns[i])
        if Ns[i] == 0:
            continue
        y_ref, ad = oracle.gemv_w4a4(cw, sw, gw, cx, sx, gx)
        check_tol(y, y_ref, ad, f"segment {i} M={M} K={K}")
        assert np.array_equal(y, host(nv.gemv_w4a4(*m, cxd, sxd, gxd))), f"segment {i}"


def test_w4a4_zero_k_and_empty():
    c = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, device="cuda")
    cx = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    sx = torch.zeros((0, 2), dtype=torch.uint8, device="cuda")
    y = nv.gemv_w4a4(c, s, one, cx, sx, one)
    assert y.shape == (0, 4)
