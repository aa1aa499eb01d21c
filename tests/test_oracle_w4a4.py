"""Pins for the oracle's W4A4 path (CPU only): activation quantization with a
static input scale against a brute-force nearest-value search over the E4M3
and E2M1 grids (fp32 ratios computed with numpy), the W4A4 GEMV against
numpy decode and fp64 matmul, the reduction to the W4A16 GEMV for activations
that lie on the NVFP4 grid, and saturation when the static scale is small."""
import numpy as np
import pytest

import workloads
from refdecode import E2M1, E4M3, bf16_value, decode

E4M3_FINITE = np.arange(0x7F)   # positive finite codes 0x00 .. 0x7E (448)


def _nearest_code(t, values, codes):
    """Code of the value nearest to t among `values` (ascending), ties to the
    even code."""
    d = np.abs(values - t)
    best = d.min()
    cand = codes[d == best]
    even = cand[cand % 2 == 0]
    return int(even[0] if len(even) else cand[0])


def brute_quantize(x_bits, g):
    """Reference quantizer written from the recipe: r = amax / (6 g) and
    t = x / (s g) in fp32, then the nearest grid value (ties to even),
    saturating at 448 and 6; a negative t that rounds to 0 keeps code 0."""
    x = bf16_value(x_bits).astype(np.float32)
    M, K = x.shape
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    g = np.float32(g)
    d6 = np.float32(6.0) * g
    e4 = E4M3[E4M3_FINITE]
    mags = E2M1[:8]
    for m in range(M):
        for b in range(K // 16):
            blk = x[m, 16 * b:16 * b + 16]
            r = np.float32(np.abs(blk).max()) / d6
            sc = 0x7E if r > 448 else _nearest_code(float(r), e4, E4M3_FINITE)
            scales[m, b] = sc
            s = np.float32(E4M3[sc])
            if s == 0:
                continue
            dn = s * g
            for j in range(16):
                t = np.float32(blk[j]) / dn
                a = abs(float(t))
                mag = 7 if a > 6 else _nearest_code(a, mags, np.arange(8))
                code = mag | 8 if (t < 0 and mag != 0) else mag
                k = 16 * b + j
                codes[m, k // 2] |= np.uint8(code << (4 * (k % 2)))
    return codes, scales


@pytest.mark.parametrize("spread", [1.0, 1e3])
def test_quantize_act_brute_force(oracle, spread):
    """bf16 activations whose blocks span several binades (spread) and a
    static scale calibrated on part of them: scales saturate in some blocks
    and reach the E4M3 subnormals in others."""
    g = np.random.default_rng(int(spread))
    x = (g.standard_normal((3, 64)) * spread ** g.uniform(-1, 1, (3, 64))).astype(np.float32)
    x_bits = workloads.bf16_bits_from_f32(x)
    gx = float(np.abs(x[0]).max()) / 2688.0
    codes, scales = oracle.quantize_act(x_bits, gx)
    bc, bs = brute_quantize(x_bits, gx)
    assert np.array_equal(scales, bs)
    assert np.array_equal(codes, bc)


def test_quantize_act_saturates_with_a_small_static_scale(oracle):
    x_bits = workloads.x_bf16(7, 0, 0, 2, 32)
    x = bf16_value(x_bits)
    gx = float(np.abs(x).max()) / 2688.0 / 100.0   # 100x below calibration
    codes, scales = oracle.quantize_act(x_bits, gx)
    nib = np.empty(x.shape, np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
    for m in range(2):
        for b in range(2):
            blk = x[m, 16 * b:16 * b + 16]
            if np.abs(blk).max() / (6 * gx) > 448:
                assert scales[m, b] == 0x7E
                j = int(np.argmax(np.abs(blk)))
                assert nib[m, 16 * b + j] & 7 == 7      # magnitude 6
                assert (nib[m, 16 * b + j] >> 3) == (blk[j] < 0)


def test_gemv_w4a4_numpy(oracle):
    N, K, M = 37, 96, 3
    w = workloads.dense_weights(6, 0, 1, N, K)
    cw, sw, gw = oracle.pack(w)
    x_bits = workloads.x_bf16(7, 0, 2, M, K)
    gx = float(np.float32(np.abs(bf16_value(x_bits)).max() / 2688.0))   # an fp32 scale
    cx, sx = oracle.quantize_act(x_bits, gx)
    y, ad = oracle.gemv_w4a4(cw, sw, gw, cx, sx, gx)
    W = decode(cw, sw)
    X = decode(cx, sx)
    ref = (X @ W.T) * float(gw) * gx
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(ad, np.abs(X) @ np.abs(W).T * abs(float(gw) * gx), rtol=1e-12)
    rows = np.array([0, 5, 36])
    ys, ads = oracle.gemv_w4a4(cw, sw, gw, cx, sx, gx, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(ads, ad[:, rows])


def test_w4a4_reduces_to_w4a16_on_grid_activations(oracle):
    """Activations that are E2M1 values times an E4M3 scale times g_x, with a
    6 in every block, quantize to themselves; the W4A4 GEMV then equals the
    W4A16 GEMV of the same activations."""
    N, K, M = 20, 64, 2
    g = np.random.default_rng(3)
    gx = 0.25
    sc = g.choice([0x30, 0x38, 0x41, 0x4A], size=(M, K // 16))
    mags = g.integers(0, 16, size=(M, K))
    mags[:, ::16] = 7                                # |6| in every block
    x = E2M1[mags] * np.repeat(E4M3[sc], 16, axis=1) * gx
    x_bits = workloads.bf16_bits_from_f32(x.astype(np.float32))
    assert np.array_equal(bf16_value(x_bits), x)     # exact in bf16
    cx, sx = oracle.quantize_act(x_bits, gx)
    assert np.array_equal(sx, sc)
    assert np.array_equal(decode(cx, sx) * gx, x)
    cw, sw, gw = oracle.pack(workloads.dense_weights(6, 1, 0, N, K))
    y4, _ = oracle.gemv_w4a4(cw, sw, gw, cx, sx, gx)
    y16, _ = oracle.gemv(cw, sw, gw, x_bits)
    np.testing.assert_allclose(y4, y16, rtol=1e-13, atol=1e-300)


def test_quantize_act_rejects_bad_input(oracle):
    x = workloads.x_bf16(7, 2, 0, 1, 32)
    with pytest.raises(Exception):
        oracle.quantize_act(x, 0.0)
    with pytest.raises(Exception):
        oracle.quantize_act(x[:, :24], 1.0)
