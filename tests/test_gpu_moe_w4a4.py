"""GPU W4A4 MoE (nvfp4_moe_w4a4_gemv) against the oracle: the 288-expert
workload at M = 1 and M = 8 with and without the W4A16 shared expert, a
small model with duplicate and invalid ids, the single-token path (both
quantizations inside gate|up) and its edges, and grid activations.

What is compared, and how:
  - x on the NVFP4 grid of its static scale (the workspace's xq): bit for bit
    against the oracle's quantizer, decoded;
  - h (bf16 SwiGLU output): the kernel rounds an fp32 gate|up sum, the oracle
    an fp64 one, so every value is within one ulp and at least 99% are equal;
  - h on the grid of its static scale (hq): the oracle quantizes the kernel's
    own h (its h_in argument), so both take the rounding decisions on the
    same input, and the decoded values must agree bit for bit;
  - y: against the oracle fed the kernel's h, within the GEMV tolerance
    1e-3 * sum |terms| + 1e-6 (the down product and the combine differ only in
    fp32 summation order);
  - y end to end: against the oracle run from x alone (its own fp64 h). Where
    a one-ulp flip of h moves a value across a rounding decision of h's
    quantization, the two sides multiply different NVFP4 activations; every
    output outside the tolerance must then be covered by the effect of those
    flips, which the oracle measures as the difference between its runs on
    its own h and on the kernel's h. The flips are counted and reported."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say
from refdecode import bf16_value, decode
from test_gpu_moe import build_experts
from test_gpu_moe_shared import build_shared, check_hs

pytestmark = pytest.mark.gpu


def _bits(ws, off, rows, cols):
    t = ws[off:off + rows * cols * 2].view(torch.int16)
    return host(t).view(np.uint16).reshape(rows, cols)


def run_w4a4_moe(hw, dw, x, ids, gw, H, I, ga13, ga2_under, shared=None, what=""):
    """One kernel call and its checks; returns the largest error / tolerance.
    ga2 = max|h| / 2688 / ga2_under, from the oracle's h (so ga2_under > 1
    saturates the largest blocks of h)."""
    hsw, dsw = shared if shared is not None else (None, None)
    M, topk = ids.shape
    E = hw[0].shape[0]
    Is = hsw[0].shape[0] // 2 if hsw is not None else 0
    _, _, h_ref, _, _ = oracle.moe_w4a4(*hw, x, ids, gw, ga13, 1.0, shared=hsw)
    valid = ((ids >= 0) & (ids < E)).ravel()
    hmax = np.abs(bf16_value(h_ref[valid])).max() if valid.any() else 1.0
    ga2 = np.float32(max(hmax, 1e-30) / 2688.0 / ga2_under)
    lay = nv.moe_w4a4_workspace_layout(M, H, I, topk, Is)
    ws = torch.empty(nv.moe_w4a4_workspace_bytes(M, H, I, topk, Is), dtype=torch.uint8,
                     device="cuda")
    say(f"[moe w4a4] {what} M={M} topk={topk} E={E} H={H} I={I} Is={Is} "
        f"g_x={float(ga13):.4g} g_h={float(ga2):.4g}")
    y = host(nv.moe_w4a4_gemv(*dw, dev_x(x), dev(np.array([ga13], np.float32)),
                              dev(np.array([ga2], np.float32)), dev(ids), dev(gw),
                              shared=dsw, workspace=ws))
    xq = _bits(ws, lay["xq"], M, H)
    cx, sx = oracle.quantize_act(x, ga13)
    assert np.array_equal(bf16_value(xq), decode(cx, sx)), "x on the grid"
    h = _bits(ws, lay["h"], M * topk, I)
    hq = _bits(ws, lay["hq"], M * topk, I)
    if valid.any():
        check_hs(h[valid], h_ref[valid])
    h_in = np.where(valid[:, None], h, 0).astype(np.uint16)
    y_ref, bound, _, hc, hs = oracle.moe_w4a4(*hw, x, ids, gw, ga13, ga2, shared=hsw,
                                              h_in=h_in)
    assert np.array_equal(bf16_value(hq[valid]), decode(hc, hs)[valid]), "h on the grid"
    r = check_tol(y, y_ref, bound, what)
    # end to end: the oracle from x alone
    y_x, bound_x, _, hc_x, hs_x = oracle.moe_w4a4(*hw, x, ids, gw, ga13, ga2, shared=hsw)
    flips_h = int(np.count_nonzero(h[valid] != h_ref[valid])) if valid.any() else 0
    flips_q = (int(np.count_nonzero(hc[valid] != hc_x[valid])) +
               int(np.count_nonzero(hs[valid] != hs_x[valid]))) if valid.any() else 0
    tol = np.maximum(1e-3 * bound, 1e-3 * bound_x) + 1e-6
    err = np.abs(y.astype(np.float64) - y_x)
    flip_effect = np.abs(y_x - y_ref)          # the oracle's own measure of the flips
    outside = err > tol
    assert np.all(err <= tol + flip_effect * (1 + 1e-6) + 1e-9), \
        f"{what}: end-to-end error not covered by the h flips"
    assert not outside.any() or flips_q > 0, f"{what}: outputs outside tolerance without flips"
    sat = float(np.mean(hs[valid] == 0x7E)) if valid.any() else 0.0
    eq = float(np.mean(h[valid] == h_ref[valid])) if valid.any() else 1.0
    say(f"  max err / tol = {r:.3e}; h bit-equal {eq:.6f}; saturated h blocks {sat:.4f}")
    say(f"  end to end from x: {int(outside.sum())} of {y.size} outputs outside the tolerance, "
        f"covered by {flips_h} h flips ({flips_q} quantized codes/scales changed)")
    return y


@pytest.mark.parametrize("M,with_shared", [(1, True), (8, True), (8, False)])
def test_moe_w4a4_workload_4(M, with_shared):
    E, H, I, topk, Is = 288, 4096, 1536, 8, 768
    ids, gw = workloads.moe_routing(4, 0, M, E, topk)
    hw, dw = build_experts(4, 0, E, H, I, ids.ravel())
    shared = build_shared(4, 0, H, Is) if with_shared else None
    x = workloads.x_bf16(4, 0, 0, M, H)
    calib = bf16_value(workloads.x_bf16(4, 1, 0, M, H))
    ga13 = np.float32(np.abs(calib).max() / 2688.0)
    run_w4a4_moe(hw, dw, x, ids, gw, H, I, ga13, 2.0, shared, f"workload 4 M={M}")


@pytest.mark.parametrize("Is", [0, 96])
def test_moe_w4a4_duplicates_invalid_ids_and_saturation(Is):
    E, H, I = 6, 512, 256
    hw, dw = build_experts(45, 0, E, H, I, range(E))
    shared = build_shared(45, 1, H, Is) if Is else None
    cases = {
        "m1": np.array([[3, 1]], np.int32),
        "dup_invalid": np.array([[2, 2, -1], [7, 0, 0], [5, 4, 3]], np.int32),
        "all_invalid": np.array([[-1, 6], [99, -3]], np.int32),
        "m8": np.random.default_rng(Is + 1).integers(0, E, size=(8, 4)).astype(np.int32),
    }
    for name, ids in cases.items():
        M, topk = ids.shape
        gw = np.random.default_rng(M * 5 + topk).random((M, topk)).astype(np.float32)
        x = workloads.x_bf16(45, M, Is, M, H)
        # x's static scale 20x below calibration: many x blocks saturate
        ga13 = np.float32(np.abs(bf16_value(x)).max() / 2688.0 / 20.0)
        y = run_w4a4_moe(hw, dw, x, ids, gw, H, I, ga13, 8.0, shared, f"Is={Is} {name}")
        if name == "all_invalid" and not Is:
            assert not y.any()


@pytest.mark.parametrize("case", ["dup_invalid", "all_invalid_shared", "shared_wider_than_i",
                                  "topk16", "h16384", "h16416"])
def test_moe_w4a4_single_token(case):
    """M = 1 takes three launches: x onto its grid, then a gate|up launch that
    also puts each 16-row block of h onto its grid, then down and combine.
    Covers invalid and duplicate ids, ids that are all invalid (the shared
    expert alone contributes), a shared expert wider than I, topk = 16, and
    long rows (H = 16384 and 16416)."""
    E, H, I, Is = 6, 512, 256, 0
    ids = np.array([[2, -1, 2, 9]], np.int32)
    if case == "all_invalid_shared":
        ids, Is = np.array([[-1, 6]], np.int32), 96
    elif case == "shared_wider_than_i":
        E, H, I, Is = 5, 256, 64, 160
        ids = np.array([[1, 4, 0]], np.int32)
    elif case == "topk16":
        E, H, I = 20, 128, 32
        ids = np.random.default_rng(16).choice(E, 16, replace=False).astype(np.int32)[None]
    elif case in ("h16384", "h16416"):
        E, I, Is = 3, 64, 32
        H = int(case[1:])
        ids = np.array([[0, 2]], np.int32)
    hw, dw = build_experts(47, 0, E, H, I, range(E))
    shared = build_shared(47, 1, H, Is) if Is else None
    topk = ids.shape[1]
    gw = np.random.default_rng(topk).random((1, topk)).astype(np.float32)
    x = workloads.x_bf16(47, 1, H, 1, H)
    ga13 = np.float32(np.abs(bf16_value(x)).max() / 2688.0 / 4.0)
    y = run_w4a4_moe(hw, dw, x, ids, gw, H, I, ga13, 2.0, shared, f"M=1 {case}")
    if case == "all_invalid_shared":
        assert y.any()


def test_moe_w4a4_grid_activations_match_w4a16_h_and_repeat():
    """x on the NVFP4 grid of a power-of-two static scale: the W4A4 gate|up
    sees x / g_x exactly and multiplies by g_x exactly, so its h equals the
    W4A16 MoE kernel's h bit for bit. Two calls agree bit for bit."""
    E, H, I, M, topk = 6, 256, 128, 3, 2
    hw, dw = build_experts(46, 0, E, H, I, range(E))
    ids, gw = workloads.moe_routing(46, 0, M, E, topk)
    r = np.random.default_rng(46)
    sc = r.choice([0x30, 0x38, 0x41, 0x4A], size=(M, H // 16))
    mags = r.integers(0, 16, size=(M, H))
    mags[:, ::16] = 7
    from refdecode import E2M1, E4M3
    xv = E2M1[mags] * np.repeat(E4M3[sc], 16, axis=1) * 0.25
    x = workloads.bf16_bits_from_f32(xv.astype(np.float32))
    assert np.array_equal(bf16_value(x), xv)
    xd, idd, gwd = dev_x(x), dev(ids), dev(gw)
    g13, g2 = dev(np.array([0.25], np.float32)), dev(np.array([0.01], np.float32))
    ws = torch.empty(nv.moe_w4a4_workspace_bytes(M, H, I, topk), dtype=torch.uint8,
                     device="cuda")
    say(f"[moe w4a4] grid activations M={M} topk={topk} H={H} I={I}")
    a = host(nv.moe_w4a4_gemv(*dw, xd, g13, g2, idd, gwd, workspace=ws))
    h4 = _bits(ws, 0, M * topk, I).copy()
    b = host(nv.moe_w4a4_gemv(*dw, xd, g13, g2, idd, gwd, workspace=ws))
    assert np.array_equal(a, b)
    ws16 = torch.empty(nv.moe_workspace_bytes(M, H, I, topk), dtype=torch.uint8,
                       device="cuda")
    nv.moe_gemv_into(*dw, xd, idd, gwd, torch.empty((M, H), device="cuda"), ws16)
    assert np.array_equal(h4, _bits(ws16, 0, M * topk, I))
