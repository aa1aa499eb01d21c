"""Pins for the oracle's MoE expert-slot path (CPU only): reduction to the
GEMV oracle plus SwiGLU, brute force against numpy, and invariants; the
shared expert pinned to the routed path (a shared expert equal to expert e is
an extra slot naming e with gate weight 1) and to plain numpy."""
import numpy as np
import pytest

import workloads
from refdecode import bf16_value, decode


def _experts(E, H, I, rep=0, seed_wl=4):
    c13, s13, g13, c2, s2, g2 = [], [], [], [], [], []
    import oracle
    for e in range(E):
        w13, w2 = workloads.moe_expert_weights(seed_wl, rep, e, H, I)
        a, b, g = oracle.pack(w13)
        c13.append(a); s13.append(b); g13.append(g)
        a, b, g = oracle.pack(w2)
        c2.append(a); s2.append(b); g2.append(g)
    return (np.stack(c13), np.stack(s13), np.array(g13, np.float32),
            np.stack(c2), np.stack(s2), np.array(g2, np.float32))


@pytest.fixture(scope="module")
def small_experts():
    return _experts(6, 64, 32)


def _bf16_round(v):
    import oracle
    return np.array([oracle.bf16_from_double(float(t)) for t in v.ravel()],
                    np.uint16).reshape(v.shape)


def test_moe_topk1_reduces_to_gemv_swiglu_gemv(oracle, small_experts):
    c13, s13, g13, c2, s2, g2 = small_experts
    E, H, I = 6, 64, 32
    x = workloads.x_bf16(4, 0, 0, 1, H)
    for e in range(E):
        ids = np.array([[e]], np.int32)
        gw = np.ones((1, 1), np.float32)
        y, bound, h = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw, want_h=True)
        a, _ = oracle.gemv(c13[e], s13[e], g13[e], x)
        G, U = a[0, :I], a[0, I:]
        hb = _bf16_round(G / (1 + np.exp(-G)) * U)
        assert np.array_equal(h[0], hb)
        o, ad = oracle.gemv(c2[e], s2[e], g2[e], hb[None, :])
        assert np.array_equal(y[0], o[0])
        np.testing.assert_allclose(bound[0], ad[0], rtol=1e-15)


def test_moe_brute_force_numpy(oracle, small_experts):
    c13, s13, g13, c2, s2, g2 = small_experts
    E, H, I = 6, 64, 32
    M, topk = 3, 4
    x = workloads.x_bf16(4, 1, 0, M, H)
    ids, gw = workloads.moe_routing(4, 1, M, E, topk)
    y, bound = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw)
    xv = bf16_value(x)
    ref = np.zeros((M, H))
    for m in range(M):
        for j in range(topk):
            e = ids[m, j]
            a = float(g13[e]) * (decode(c13[e], s13[e]) @ xv[m])
            G, U = a[:I], a[I:]
            h = bf16_value(_bf16_round(G / (1 + np.exp(-G)) * U))
            o = float(g2[e]) * (decode(c2[e], s2[e]) @ h)
            ref[m] += float(gw[m, j]) * o
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-10 * np.abs(bound).max())


def test_moe_slot_permutation_invariant(oracle, small_experts):
    c13, s13, g13, c2, s2, g2 = small_experts
    M, topk = 2, 5
    x = workloads.x_bf16(4, 2, 0, M, 64)
    ids, gw = workloads.moe_routing(4, 2, M, 6, topk)
    y, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw)
    p = np.array([3, 0, 4, 1, 2])
    y2, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids[:, p].copy(), gw[:, p].copy())
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)


def test_moe_rows_independent(oracle, small_experts):
    c13, s13, g13, c2, s2, g2 = small_experts
    M, topk = 4, 3
    x = workloads.x_bf16(4, 3, 0, M, 64)
    ids, gw = workloads.moe_routing(4, 3, M, 6, topk)
    y, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw)
    for m in range(M):
        y1, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x[m:m + 1], ids[m:m + 1], gw[m:m + 1])
        assert np.array_equal(y1[0], y[m])


def test_moe_identical_experts_gates_sum_to_one(oracle, small_experts):
    c13, s13, g13, c2, s2, g2 = small_experts
    # make expert 5 a copy of expert 2
    c13, s13, c2, s2 = c13.copy(), s13.copy(), c2.copy(), s2.copy()
    g13, g2 = g13.copy(), g2.copy()
    for a in (c13, s13, c2, s2, g13, g2):
        a[5] = a[2]
    x = workloads.x_bf16(4, 4, 0, 1, 64)
    y1, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x, np.array([[2]], np.int32),
                       np.ones((1, 1), np.float32))
    y2, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x, np.array([[2, 5]], np.int32),
                       np.array([[0.25, 0.75]], np.float32))
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-14)


def test_moe_out_of_range_ids_contribute_nothing(oracle, small_experts):
    c13, s13, g13, c2, s2, g2 = small_experts
    x = workloads.x_bf16(4, 5, 0, 1, 64)
    ids = np.array([[1, 3]], np.int32)
    gw = np.array([[0.4, 0.6]], np.float32)
    y, _ = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids, gw)
    ids_bad = np.array([[1, -1, 3, 6, 1000]], np.int32)
    gw_bad = np.array([[0.4, 9.0, 0.6, 9.0, 9.0]], np.float32)
    y2, _, h = oracle.moe(c13, s13, g13, c2, s2, g2, x, ids_bad, gw_bad, want_h=True)
    assert np.array_equal(y, y2)
    assert np.all(h[1] == 0) and np.all(h[3] == 0) and np.all(h[4] == 0)


def _shared_from_expert(small_experts, e):
    c13, s13, g13, c2, s2, g2 = small_experts
    return (c13[e], s13[e], g13[e], c2[e], s2[e], g2[e])


def test_moe_shared_equals_extra_slot_with_unit_gate(oracle, small_experts):
    """The blend adds the shared expert after the routed slots with weight 1:
    bit-identical to routing every token to the same expert once more, as its
    last slot, with gate weight 1."""
    E, H, I, M, topk = 6, 64, 32, 3, 2
    x = workloads.x_bf16(4, 2, 0, M, H)
    ids, gw = workloads.moe_routing(4, 2, M, E, topk)
    for e in (0, 5):
        y, bound, h, hs = oracle.moe_shared(*small_experts, x, ids, gw,
                                            _shared_from_expert(small_experts, e),
                                            want_h=True)
        ids2 = np.concatenate([ids, np.full((M, 1), e, np.int32)], axis=1)
        gw2 = np.concatenate([gw, np.ones((M, 1), np.float32)], axis=1)
        y2, bound2, h2 = oracle.moe(*small_experts, x, ids2, gw2, want_h=True)
        assert np.array_equal(y, y2) and np.array_equal(bound, bound2)
        h2 = h2.reshape(M, topk + 1, I)
        assert np.array_equal(h.reshape(M, topk, I), h2[:, :topk])
        assert np.array_equal(hs, h2[:, topk])


def test_moe_shared_zero_expert_adds_nothing(oracle, small_experts):
    E, H, I, Is, M, topk = 6, 64, 32, 48, 2, 3
    x = workloads.x_bf16(4, 3, 0, M, H)
    ids, gw = workloads.moe_routing(4, 3, M, E, topk)
    zero = (np.zeros((2 * Is, H // 2), np.uint8), np.zeros((2 * Is, H // 16), np.uint8),
            np.float32(1.0), np.zeros((H, Is // 2), np.uint8),
            np.zeros((H, Is // 16), np.uint8), np.float32(1.0))
    y, bound = oracle.moe_shared(*small_experts, x, ids, gw, zero)
    y0, bound0 = oracle.moe(*small_experts, x, ids, gw)
    assert np.array_equal(y, y0) and np.array_equal(bound, bound0)


def test_moe_shared_brute_force_numpy(oracle, small_experts):
    """A shared expert of another width (Is = 48) against numpy: decode, fp64
    gate|up, SwiGLU rounded once to bf16, fp64 down."""
    import oracle as o
    E, H, I, Is, M, topk = 6, 64, 32, 48, 2, 3
    x = workloads.x_bf16(4, 4, 0, M, H)
    ids, gw = workloads.moe_routing(4, 4, M, E, topk)
    w13, w2 = workloads.moe_shared_weights(4, 4, H, Is)
    sc13, ss13, sg13 = o.pack(w13)
    sc2, ss2, sg2 = o.pack(w2)
    y, bound, _, hs = oracle.moe_shared(*small_experts, x, ids, gw,
                                        (sc13, ss13, sg13, sc2, ss2, sg2), want_h=True)
    y0, bound0 = oracle.moe(*small_experts, x, ids, gw)
    W13 = decode(sc13, ss13) * np.float64(sg13)
    W2 = decode(sc2, ss2)
    xv = bf16_value(x)
    for m in range(M):
        a = W13 @ xv[m]
        G, U = a[:Is], a[Is:]
        hb = _bf16_round(G / (1 + np.exp(-G)) * U)
        assert np.array_equal(hs[m], hb)
        t = W2 * bf16_value(hb)[None, :]
        sh = np.float64(sg2) * t.sum(axis=1)
        np.testing.assert_allclose(y[m], y0[m] + sh, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(bound[m], bound0[m] + abs(np.float64(sg2)) * np.abs(t).sum(axis=1),
                                   rtol=1e-12)
