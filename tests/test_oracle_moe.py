"""Pins for the oracle's MoE expert-slot path (CPU only): reduction to the
GEMV oracle plus SwiGLU, brute force against numpy, and invariants."""
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
