"""GPU pack and dequant against the oracle: bit-exact (codes, scales, tensor
scale and dequantised fp32) on every workload's weights and on crafted
cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from conftest import pack_cases
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def gpu_pack(W, override=None):
    ov = None if override is None else dev(np.array([override], np.float32))
    c, s, g = nv.pack(dev(W), ov)
    return host(c), host(s), np.float32(host(g)[0])


def assert_pack_equal(W, override=None, what="", with_dequant=True):
    say(f"[pack] {what} shape={W.shape} override={override}")
    c0, s0, g0 = oracle.pack(W, override)
    c1, s1, g1 = gpu_pack(W, override)
    assert np.float32(g1).view(np.uint32) == np.float32(g0).view(np.uint32), (what, g1, g0)
    assert np.array_equal(s1, s0), (what, int((s1 != s0).sum()))
    nbad = int((c1 != c0).sum())
    assert nbad == 0, (what, nbad)
    if with_dequant and W.shape[1] % 32 == 0 and W.size:
        d0 = oracle.dequant(c0, s0, g0)
        d1 = host(nv.dequant(dev(c1), dev(s1), dev(np.array([g1], np.float32))))
        assert np.array_equal(d1.view(np.uint32), d0.view(np.uint32)), what
    return c0, s0, g0


@pytest.mark.parametrize("case", pack_cases(), ids=lambda c: c["name"])
def test_pack_worked_examples_on_gpu(case):
    c, s, g = gpu_pack(case["W"], case["override"])
    assert g == np.float32(case["g"])
    assert np.array_equal(s, case["exp_scales"])
    assert np.array_equal(c, case["exp_codes"])
    if case["K"] % 32 == 0:
        d = host(nv.dequant(dev(c), dev(s), dev(np.array([g], np.float32))))
        assert np.array_equal(d, case["exp_dequant"])


DENSE = [(1, 0, 1024, 4096)] + [(2, i, n, k) for i, (_, n, k) in
                                 enumerate(workloads.DECODE_LAYER)] + \
        [(5, 0, 12288, 4096), (5, 1, 4096, 12288)]


@pytest.mark.parametrize("wl,stream,N,K", DENSE)
def test_pack_bitexact_workload_weights(wl, stream, N, K):
    W = workloads.dense_weights(wl, 0, stream, N, K)
    assert_pack_equal(W, None, f"workload {wl} matrix {stream}")


def test_pack_bitexact_lm_head_full_size():
    W = workloads.dense_weights(3, 0, 0, 151936, 4096)
    assert_pack_equal(W, None, "lm head 151936x4096")


@pytest.mark.parametrize("override", [1e-7, 1e-5, 1e-3, 0.02, 1.0, 50.0, 1e6])
def test_pack_bitexact_crafted_scales(override):
    """Overrides push block scales into the E4M3 subnormal range, to zero and
    past 448 (saturation)."""
    W = workloads.student_t_weights(5, 3, 0, 96, 512)
    assert_pack_equal(W, override, f"override {override}")


def test_pack_edge_values():
    rng = np.random.default_rng(11)
    cases = {
        "all_zero": np.zeros((4, 64), np.float32),
        "negative_zero": -np.zeros((2, 32), np.float32),
        "single_block": rng.standard_normal((1, 16)).astype(np.float32),
        "huge": (rng.standard_normal((8, 64)) * 1e30).astype(np.float32),
        "tiny_normal": (rng.standard_normal((8, 64)) * 1e-30).astype(np.float32),
        "fp32_subnormal": (rng.standard_normal((4, 64)) * 1e-40).astype(np.float32),
        "ties": np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2,
                                 np.float32), (3, 2)),
        "ragged_rows": rng.standard_normal((3, 48)).astype(np.float32),
    }
    for name, W in cases.items():
        assert_pack_equal(W, None, name)


def test_pack_empty():
    c, s, g = nv.pack(torch.empty((0, 64), dtype=torch.float32, device="cuda"))
    assert host(g)[0] == 1.0 and c.shape == (0, 32) and s.shape == (0, 4)
