"""Pins for the oracle's W4A4 MoE path (CPU only): brute force against numpy
with an independent nearest-value quantizer, reduction to the W4A16 MoE and
GEMV oracles when x and h already lie on the NVFP4 grid of power-of-two
static scales, the W4A16 shared expert added unchanged, and the h_in
override that lets a caller take the h rounding decisions on its own h."""
import numpy as np
import pytest

import workloads
from refdecode import E2M1, E4M3, bf16_value, decode
from test_oracle_moe import _bf16_round, _experts, _shared_from_expert
from test_oracle_w4a4 import brute_quantize

E, H, I = 6, 64, 32


@pytest.fixture(scope="module")
def experts():
    return _experts(E, H, I)


def _static_scale(v):
    """max|v| / 2688 as an fp32 number (a calibrated static input scale)."""
    return float(np.float32(np.abs(v).max() / 2688.0))


def _grid_rows(seed, rows, K, g):
    """bf16 rows whose every 16-block is e2m1 * E4M3 * g with a 6 in it, so
    that quantizing them with the static scale g gives them back."""
    r = np.random.default_rng(seed)
    sc = r.choice([0x30, 0x38, 0x41, 0x4A], size=(rows, K // 16))
    mags = r.integers(0, 16, size=(rows, K))
    mags[:, ::16] = 7
    v = E2M1[mags] * np.repeat(E4M3[sc], 16, axis=1) * g
    bits = workloads.bf16_bits_from_f32(v.astype(np.float32))
    assert np.array_equal(bf16_value(bits), v)
    return bits, v


@pytest.mark.parametrize("with_shared", [False, True])
def test_moe_w4a4_brute_force_numpy(oracle, experts, with_shared):
    c13, s13, g13, c2, s2, g2 = experts
    M, topk = 2, 3
    x = workloads.x_bf16(4, 5, 0, M, H)
    ids, gw = workloads.moe_routing(4, 5, M, E, topk)
    ga13 = _static_scale(bf16_value(workloads.x_bf16(4, 6, 0, M, H)))
    _, _, h16 = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw, want_h=True)
    ga2 = _static_scale(bf16_value(h16)) * 0.5     # some h blocks saturate
    shared = _shared_from_expert(experts, 4) if with_shared else None
    y, bound, h, hc, hs = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw,
                                          ga13, ga2, shared=shared)
    xc, xs = brute_quantize(x, ga13)
    xq = decode(xc, xs)
    ref = np.zeros((M, H))
    for m in range(M):
        for j in range(topk):
            e, slot = ids[m, j], m * topk + j
            a = float(g13[e]) * ga13 * (decode(c13[e], s13[e]) @ xq[m])
            G, U = a[:I], a[I:]
            hb = _bf16_round(G / (1 + np.exp(-G)) * U)
            assert np.array_equal(h[slot], hb)
            bc, bs = brute_quantize(hb[None, :], ga2)
            assert np.array_equal(hc[slot], bc[0]) and np.array_equal(hs[slot], bs[0])
            o = float(g2[e]) * ga2 * (decode(c2[e], s2[e]) @ decode(bc, bs)[0])
            ref[m] += float(gw[m, j]) * o
        if with_shared:
            sc13, ss13, sg13, sc2, ss2, sg2 = shared
            a = float(sg13) * (decode(sc13, ss13) @ bf16_value(x[m]))
            Is = sc13.shape[0] // 2
            hsb = bf16_value(_bf16_round(a[:Is] / (1 + np.exp(-a[:Is])) * a[Is:]))
            ref[m] += float(sg2) * (decode(sc2, ss2) @ hsb)
    assert (hs == 0x7E).any()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-10 * np.abs(bound).max())


def test_moe_w4a4_on_grid_reduces_to_w4a16(oracle, experts):
    """x on the grid of g_a13 = 1/4: h equals the W4A16 MoE's h bit for bit.
    h_in on the grid of g_a2 = 1/2: the quantized h decodes to h_in / g_a2 and
    y is the gate-weighted sum of W4A16 GEMVs of h_in, bit for bit (power-of-
    two scales make every rescaling exact in fp64)."""
    c13, s13, g13, c2, s2, g2 = experts
    M, topk = 2, 3
    ids, gw = workloads.moe_routing(4, 7, M, E, topk)
    x, _ = _grid_rows(11, M, H, 0.25)
    h_in, hv = _grid_rows(12, M * topk, I, 0.5)
    y, _, h, hc, hs = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw, 0.25, 0.5,
                                      h_in=h_in)
    _, _, h16 = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw, want_h=True)
    assert np.array_equal(h, h16)
    assert np.array_equal(decode(hc, hs) * 0.5, hv)
    ref = np.zeros((M, H))
    for m in range(M):
        for j in range(topk):
            e, slot = ids[m, j], m * topk + j
            o, _ = oracle.gemv(c2[e], s2[e], g2[e], h_in[slot][None, :])
            ref[m] += float(gw[m, j]) * o[0]
    assert np.array_equal(y, ref)


def test_moe_w4a4_shared_expert_added_unchanged(oracle, experts):
    c13, s13, g13, c2, s2, g2 = experts
    M, topk = 3, 2
    x = workloads.x_bf16(4, 8, 0, M, H)
    ids, gw = workloads.moe_routing(4, 8, M, E, topk)
    shared = _shared_from_expert(experts, 2)
    ga13, ga2 = 0.003, 0.0007
    y0, b0, h0, c0, s0 = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw, ga13, ga2)
    y1, b1, h1, c1, s1 = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw, ga13, ga2,
                                         shared=shared)
    none = np.full_like(ids, -1)
    ys, bs = oracle.moe_shared(c13, s13, g13, c2, s2, g2, x, none, gw, shared)
    assert np.array_equal(y1, y0 + ys) and np.array_equal(b1, b0 + bs)
    assert np.array_equal(h1, h0) and np.array_equal(c1, c0) and np.array_equal(s1, s0)


def test_moe_w4a4_h_in_round_trip_and_invalid_slots(oracle, experts):
    c13, s13, g13, c2, s2, g2 = experts
    M, topk = 2, 4
    x = workloads.x_bf16(4, 9, 0, M, H)
    ids, gw = workloads.moe_routing(4, 9, M, E, topk)
    ids[0, 1], ids[1, 3] = -1, E           # two slots out of range
    ga13, ga2 = 0.002, 0.001
    y, bound, h, hc, hs = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw, ga13, ga2)
    for slot in (1, 7):
        assert not h[slot].any() and not hc[slot].any() and not hs[slot].any()
    # h fed back in gives the same result; junk in skipped slots is ignored
    h_in = h.copy()
    h_in[1] = 0x3F80
    h_in[7] = 0x4000
    y2, b2, _, hc2, hs2 = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw, ga13, ga2,
                                          h_in=h_in)
    assert np.array_equal(y2, y) and np.array_equal(b2, bound)
    assert np.array_equal(hc2, hc) and np.array_equal(hs2, hs)
    # dropping the skipped slots changes nothing
    keep = ids.copy()
    keep[0, 1] = keep[1, 3] = -1
    y3, _, _, _, _ = oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, keep, gw, ga13, ga2)
    assert np.array_equal(y3, y)


def test_moe_w4a4_rejects_bad_scales(oracle, experts):
    c13, s13, g13, c2, s2, g2 = experts
    x = workloads.x_bf16(4, 10, 0, 1, H)
    ids, gw = workloads.moe_routing(4, 10, 1, E, 2)
    for ga13, ga2 in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0)):
        with pytest.raises(Exception):
            oracle.moe_w4a4(c13, s13, g13, c2, s2, g2, x, ids, gw, ga13, ga2)
