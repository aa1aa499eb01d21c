"""Pins for the oracle's element decoders and encoders (CPU only).

Each check compares the oracle against something other than itself: the
hand-enumerated OCP MX tables in tests/golden, torch's independent
float8_e4m3fn conversion, hand-worked ties, and a brute-force argmin over
the decoded table (a different formulation from the oracle's arithmetic
encoder)."""
import math

import numpy as np
import pytest
import torch

from conftest import golden_rows


def _val(s):
    return float("nan") if s == "nan" else float(s)


def test_e2m1_table_matches_hand_enumeration(oracle):
    rows = golden_rows("e2m1_values.txt")
    assert len(rows) == 16
    for code_s, v_s in rows:
        code, want = int(code_s, 16), _val(v_s)
        got = oracle.e2m1_value(code)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e2m1_sign_symmetry_and_monotone(oracle):
    mags = [oracle.e2m1_value(c) for c in range(8)]
    assert all(a < b for a, b in zip(mags, mags[1:]))
    for c in range(8):
        assert oracle.e2m1_value(c | 8) == -mags[c]


def test_e4m3_anchor_values(oracle):
    for byte_s, v_s in golden_rows("e4m3_anchors.txt"):
        b, want = int(byte_s, 16), _val(v_s)
        got = oracle.e4m3_value(b)
        if math.isnan(want):
            assert math.isnan(got), b
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(b), got, want)


def test_e4m3_full_table_matches_torch_float8():
    """All 256 bytes against torch.float8_e4m3fn -> float32 (a library
    routine written independently of the oracle)."""
    import oracle
    raw = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = raw.to(torch.float32).numpy()
    for b in range(256):
        got = oracle.e4m3_value(b)
        if math.isnan(ref[b]):
            assert math.isnan(got), b
        else:
            assert got == float(ref[b]), (hex(b), got, ref[b])


def _argmin_encode(values, codes, v):
    """Brute force: the nearest table value; on a tie the even code."""
    best = None
    for c, tv in zip(codes, values):
        d = abs(v - tv)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


@pytest.fixture(scope="module")
def e4m3_pos(oracle):
    codes = list(range(0x7F))  # 0x00 .. 0x7E, all finite non-negative
    return codes, [oracle.e4m3_value(c) for c in codes]


@pytest.fixture(scope="module")
def e2m1_pos(oracle):
    codes = list(range(8))
    return codes, [oracle.e2m1_value(c) for c in codes]


def test_e4m3_encode_brute_force_sweep(oracle, e4m3_pos):
    codes, vals = e4m3_pos
    rs = np.concatenate([
        np.linspace(0, 2 ** -6, 2001),
        np.geomspace(2 ** -12, 448, 6001),
        # every midpoint between neighbours, and one fp32 ulp either side
        np.array([(a + b) / 2 for a, b in zip(vals, vals[1:])]),
    ]).astype(np.float32)
    mids = np.array([(a + b) / 2 for a, b in zip(vals, vals[1:])], np.float32)
    rs = np.concatenate([rs, np.nextafter(mids, np.float32(np.inf)),
                         np.nextafter(mids, np.float32(0))])
    for r in rs:
        want = _argmin_encode(vals, codes, float(r))
        got = oracle.e4m3_encode(float(r))
        assert got == want, (float(r), hex(got), hex(want))


def test_e4m3_encode_clamps(oracle):
    for r in [448.0, 448.00003, 460.0, 464.0, 1e6, 3e38]:
        assert oracle.e4m3_encode(r) == 0x7E
    for r in [0.0, -0.0, -5.0]:
        assert oracle.e4m3_encode(r) == 0x00


def test_e4m3_encode_matches_torch_in_range(oracle):
    """torch's fp32 -> float8_e4m3fn conversion is round-to-nearest-even; in
    range it must agree with the oracle's encoder byte for byte."""
    g = np.random.default_rng(7)
    r = np.concatenate([g.uniform(0, 448, 20000), np.exp(g.uniform(-12, 6, 20000))])
    r = r[r <= 448].astype(np.float32)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in r], np.uint8)
    assert np.array_equal(got, ref)


def test_e2m1_encode_brute_force_sweep(oracle, e2m1_pos):
    codes, vals = e2m1_pos
    ts = np.concatenate([np.linspace(-7, 7, 14001),
                         np.array([(a + b) / 2 for a, b in zip(vals, vals[1:])]),
                         -np.array([(a + b) / 2 for a, b in zip(vals, vals[1:])])]).astype(np.float32)
    for t in ts:
        mag = _argmin_encode(vals, codes, min(abs(float(t)), 6.0))
        want = (mag | 8) if (t < 0 and mag != 0) else mag
        got = oracle.e2m1_encode(float(t))
        assert got == want, (float(t), got, want)


def test_encoder_tie_table(oracle):
    rows = golden_rows("encode_ties.txt")
    assert len(rows) > 20
    for fmt, v_s, code_s in rows:
        v, want = float(v_s), int(code_s, 16)
        got = oracle.e2m1_encode(v) if fmt == "e2m1" else oracle.e4m3_encode(v)
        assert got == want, (fmt, v_s, hex(got), hex(want))


def test_bf16_from_double(oracle):
    """Against hand cases and torch's fp32 -> bf16 RNE for fp32 inputs (for an
    input that is exactly an fp32 number one rounding is the same)."""
    assert oracle.bf16_from_double(1.0) == 0x3F80
    assert oracle.bf16_from_double(-2.0) == 0xC000
    assert oracle.bf16_from_double(1.0 + 2 ** -8) == 0x3F80      # tie -> even
    assert oracle.bf16_from_double(1.0 + 3 * 2 ** -8) == 0x3F82  # tie -> even (up)
    assert oracle.bf16_from_double(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.bf16_from_double(0.0) == 0
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert oracle.bf16_from_double(1e39) == 0x7F80
    g = np.random.default_rng(3)
    f = (g.standard_normal(5000) * np.exp(g.uniform(-30, 30, 5000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, ref)
