"""Pins for the oracle's pack and dequant (CPU only): hand-worked examples
from tests/golden/pack_examples.txt and quantisation invariants."""
import numpy as np
import pytest

import workloads
from conftest import pack_cases
from refdecode import E2M1, E4M3, decode


@pytest.mark.parametrize("case", pack_cases(), ids=lambda c: c["name"])
def test_pack_worked_examples(oracle, case):
    codes, scales, g = oracle.pack(case["W"], case["override"])
    assert g == np.float32(case["g"])
    assert np.array_equal(scales, case["exp_scales"]), scales
    assert np.array_equal(codes, case["exp_codes"]), [hex(b) for b in codes.ravel()]
    deq = oracle.dequant(codes, scales, g)
    assert np.array_equal(deq, case["exp_dequant"])


def _check_invariants(W, codes, scales, g):
    N, K = W.shape
    nb = K // 16
    # (v) scale bytes: sign bit clear, never NaN
    assert not np.any(scales & 0x80)
    assert not np.any(scales == 0x7F)
    s = E4M3[scales]                                   # [N, nb]
    q = decode(codes, scales)                          # e2m1 * s
    w = W.astype(np.float64)
    sg = np.repeat(s, 16, axis=1) * float(g)
    nz = sg > 0
    # (i) each element's code is a nearest E2M1 value of w / (s g) (fp32
    # quotient may differ from the fp64 one by an ulp: allow that slack)
    t = np.where(nz, w / np.where(nz, sg, 1.0), 0.0)
    e = np.where(nz, q / np.where(nz, np.repeat(s, 16, axis=1), 1.0), 0.0)
    mags = E2M1[:8]
    dist_best = np.min(np.abs(np.abs(np.minimum(np.abs(t), 6.0))[..., None] - mags), axis=-1)
    dist_got = np.abs(np.minimum(np.abs(t), 6.0) - np.abs(e))
    assert np.all(dist_got[nz] <= dist_best[nz] + 1e-6 * np.maximum(1, np.abs(t[nz])))
    # (ii) signs agree or the value is zero
    assert np.all((np.sign(q) == np.sign(w)) | (q == 0))
    # (iv) zero blocks have scale 0 and zero codes
    wb = np.abs(w).reshape(N, nb, 16).max(axis=2)
    zb = wb == 0
    assert np.all(scales[zb] == 0)
    cb = codes.reshape(N, nb, 8)
    assert np.all(cb[zb] == 0)
    # (iii) the block holding max|W| has scale 448 and a +-6 code there
    A = np.abs(w).max()
    if A > 0:
        n, k = np.unravel_index(np.argmax(np.abs(w)), w.shape)
        assert scales[n, k // 16] == 0x7E
        nib = (codes[n, k // 2] >> (4 * (k % 2))) & 15
        assert nib & 7 == 7
        assert g == np.float32(np.float32(A) / np.float32(2688.0))


@pytest.mark.parametrize("dist", ["normal", "student_t"])
def test_pack_invariants_random(oracle, dist):
    if dist == "normal":
        W = workloads.normal_weights(1, 0, 0, 64, 512)
    else:
        W = workloads.student_t_weights(5, 0, 0, 64, 512)
    codes, scales, g = oracle.pack(W)
    _check_invariants(W, codes, scales, g)
    if dist == "student_t":
        zb = workloads.zero_block_ids(5, 0, 0, 64, 512)
        assert len(zb) == round(0.01 * 64 * 32)
        assert np.all(scales.ravel()[zb] == 0)


def test_pack_invariants_crafted_scales(oracle):
    """Overrides push block scales into the E4M3 subnormal range and past
    448, which the data-driven g never does."""
    W = workloads.normal_weights(1, 1, 0, 32, 256)
    for ov in [1e-3, 0.02, 1.0, 50.0]:
        codes, scales, g = oracle.pack(W, ov)
        assert g == np.float32(ov)
        N, K = W.shape
        _check_invariants_no_max(W, codes, scales, g)
    # with a tiny override, scales saturate at 0x7E
    codes, scales, g = oracle.pack(W, 1e-6)
    assert np.all(scales == 0x7E)
    # with a huge override, every block underflows to scale 0 and codes 0
    codes, scales, g = oracle.pack(W, 1e6)
    assert np.all(scales == 0) and np.all(codes == 0)


def _check_invariants_no_max(W, codes, scales, g):
    assert not np.any(scales & 0x80)
    assert not np.any(scales == 0x7F)
    q = decode(codes, scales)
    w = W.astype(np.float64)
    assert np.all((np.sign(q) == np.sign(w)) | (q == 0))


def test_pack_idempotent_on_normal_scale_blocks(oracle):
    W = workloads.normal_weights(1, 2, 0, 64, 256)
    codes, scales, g = oracle.pack(W)
    Wq = oracle.dequant(codes, scales, g)
    codes2, scales2, g2 = oracle.pack(Wq, float(g))
    normal = scales >= 0x08
    assert normal.mean() > 0.99
    assert np.array_equal(scales2[normal], scales[normal])
    cb, cb2 = codes.reshape(64, 16, 8), codes2.reshape(64, 16, 8)
    assert np.array_equal(cb2[normal], cb[normal])


def test_dequant_is_decode_times_g(oracle):
    W = workloads.normal_weights(1, 3, 0, 16, 128)
    codes, scales, g = oracle.pack(W)
    deq = oracle.dequant(codes, scales, g)
    ref = (decode(codes, scales).astype(np.float32) * np.float32(g))
    assert np.array_equal(deq, ref)
    # reconstruction error bounded by half the largest E2M1 gap (1.0) * s g
    err = np.abs(deq.astype(np.float64) - W)
    bound = np.repeat(E4M3[scales], 16, axis=1) * float(g) * 1.0 + 1e-12
    assert np.all(err <= bound)


def test_pack_rejects_bad_input(oracle):
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((2, 24), np.float32))
    W = np.zeros((2, 32), np.float32)
    W[1, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.pack(W)
    with pytest.raises(ValueError):
        oracle.pack(np.ones((2, 32), np.float32), -1.0)
