"""GPU MoE with a shared expert (nvfp4_moe_shared_gemv) against the oracle:
the 288-expert workload with the pages' shared expert (gate|up 768 + 768 by
4096, down 4096 by 768) at M = 1 and M = 8, shared widths below and above the
routed one, duplicate and invalid ids (a token with no valid slot gets the
shared expert alone), and the shared activations hs checked bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say
from test_gpu_moe import build_experts

pytestmark = pytest.mark.gpu


def build_shared(wl, rep, H, Is):
    """Oracle-packed (host) and GPU-packed (device) shared expert; the packs
    must agree byte for byte."""
    w13, w2 = workloads.moe_shared_weights(wl, rep, H, Is)
    h13 = oracle.pack(w13)
    h2 = oracle.pack(w2)
    d13 = nv.pack(dev(w13))
    d2 = nv.pack(dev(w2))
    for a, b in zip(h13 + h2, d13 + d2):
        assert np.array_equal(host(b), np.asarray(a).reshape(host(b).shape))
    return (h13[0], h13[1], h13[2], h2[0], h2[1], h2[2]), (*d13, *d2)


def check_hs(hs, hs_ref):
    """The bf16 shared activations: the kernel rounds an fp32 gate|up sum,
    the oracle an fp64 one, so a value near a rounding boundary can land one
    ulp apart; every value is within one ulp (same sign) and at least 99% are
    bit-equal."""
    diff = np.abs(hs.astype(np.int32) - hs_ref.astype(np.int32))
    assert diff.max() <= 1, diff.max()
    assert np.mean(diff == 0) >= 0.99


def run_shared(hw, dw, hsw, dsw, x, ids, gw, H, I):
    M, topk = ids.shape
    Is = hsw[0].shape[0] // 2
    ws = torch.empty(nv.moe_shared_workspace_bytes(M, H, I, topk, Is), dtype=torch.uint8,
                     device="cuda")
    y = host(nv.moe_shared_gemv(*dw, dev_x(x), dev(ids), dev(gw), dsw, workspace=ws))
    y_ref, bound, h_ref, hs_ref = oracle.moe_shared(*hw, x, ids, gw, hsw, want_h=True)
    lay = nv.moe_shared_workspace_layout(M, H, I, topk, Is)
    hs = host(ws[lay["hs"]:lay["hs"] + M * Is * 2].view(torch.int16)).view(np.uint16)
    return y, y_ref, bound, hs.reshape(M, Is), hs_ref


@pytest.mark.parametrize("M", [1, 8])
def test_moe_shared_workload_4(M):
    E, H, I, topk, Is = 288, 4096, 1536, 8, 768
    ids, gw = workloads.moe_routing(4, 0, M, E, topk)
    say(f"[moe shared] M={M} distinct experts={len(set(ids.ravel()))} Is={Is}")
    hw, dw = build_experts(4, 0, E, H, I, ids.ravel())
    hsw, dsw = build_shared(4, 0, H, Is)
    x = workloads.x_bf16(4, 0, 0, M, H)
    y, y_ref, bound, hs, hs_ref = run_shared(hw, dw, hsw, dsw, x, ids, gw, H, I)
    r = check_tol(y, y_ref, bound, f"moe shared M={M}")
    same = np.mean(hs == hs_ref)
    say(f"  max err / tol = {r:.3e}; hs bit-equal fraction {same:.6f}")
    check_hs(hs, hs_ref)


def test_moe_shared_one_token_staged():
    """One token with a shared expert at H = 2048 (gate|up without x staged
    in LDS) and the down pass over 136 pairs (8 slots of I = 512, then the
    shared expert's 8 chunks), 3 per lane run as 4."""
    E, H, I, topk, Is = 12, 2048, 512, 8, 256
    rng = np.random.default_rng(5)
    ids = rng.choice(E, size=(1, topk), replace=False).astype(np.int32)
    gw = rng.random((1, topk)).astype(np.float32)
    say(f"[moe shared] one token H={H} I={I} Is={Is} ids={ids[0].tolist()}")
    hw, dw = build_experts(50, 0, E, H, I, ids.ravel())
    hsw, dsw = build_shared(50, 0, H, Is)
    x = workloads.x_bf16(50, 1, topk, 1, H)
    y, y_ref, bound, hs, hs_ref = run_shared(hw, dw, hsw, dsw, x, ids, gw, H, I)
    check_tol(y, y_ref, bound, "moe shared one token H=2048")
    check_hs(hs, hs_ref)


@pytest.mark.parametrize("M,Is", [(3, 512), (2, 64)])
def test_moe_shared_h4096_widths(M, Is):
    """H = 4096 at M >= 2 (the gate|up kernel that loads a wavefront's
    weights once for all passes): a shared expert wider than the routed one
    (routed wavefronts past I idle through the passes) and a narrower one,
    with a repeated expert across tokens and an invalid id."""
    E, H, I, topk = 8, 4096, 256, 4
    rng = np.random.default_rng(M * 7 + Is)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
    ids[:, 0] = 5
    for m in range(M):
        row = ids[m]
        dup = np.flatnonzero(row[1:] == 5) + 1
        row[dup] = [e for e in range(E) if e not in row][:len(dup)]
    ids[M - 1, topk - 1] = -1
    gw = rng.random((M, topk)).astype(np.float32)
    say(f"[moe shared] H=4096 M={M} I={I} Is={Is} ids={ids.tolist()}")
    valid = ids[(ids >= 0) & (ids < E)]
    hw, dw = build_experts(52, 0, E, H, I, valid)
    hsw, dsw = build_shared(52, Is, H, Is)
    x = workloads.x_bf16(52, M, Is, M, H)
    y, y_ref, bound, hs, hs_ref = run_shared(hw, dw, hsw, dsw, x, ids, gw, H, I)
    check_tol(y, y_ref, bound, f"moe shared H=4096 M={M} Is={Is}")
    check_hs(hs, hs_ref)


@pytest.mark.parametrize("Is", [32, 96, 512])
def test_moe_shared_widths_duplicates_and_invalid_ids(Is):
    E, H, I = 6, 512, 256
    hw, dw = build_experts(43, 0, E, H, I, range(E))
    hsw, dsw = build_shared(43, Is, H, Is)
    cases = {
        "m1": np.array([[3, 1]], np.int32),
        "dup_invalid": np.array([[2, 2, -1], [7, 0, 0], [5, 4, 3]], np.int32),
        "all_invalid": np.array([[-1, 6], [99, -3]], np.int32),
        "m8": np.random.default_rng(Is).integers(0, E, size=(8, 4)).astype(np.int32),
    }
    for name, ids in cases.items():
        M, topk = ids.shape
        say(f"[moe shared] Is={Is} {name} ids={ids.tolist()}")
        gw = np.random.default_rng(M * 7 + topk).random((M, topk)).astype(np.float32)
        x = workloads.x_bf16(43, M, Is, M, H)
        y, y_ref, bound, hs, hs_ref = run_shared(hw, dw, hsw, dsw, x, ids, gw, H, I)
        check_tol(y, y_ref, bound, f"Is={Is} {name}")
        check_hs(hs, hs_ref)
        if name == "all_invalid":
            # no routed slot: y is the shared expert alone
            zero_ids = np.full_like(ids, -1)
            y_sh, _ = oracle.moe_shared(*hw, x, zero_ids, gw, hsw)
            assert np.array_equal(y_ref, y_sh)


def test_moe_shared_is_deterministic_and_matches_routed_part():
    """Two calls agree bit for bit; with a zero shared expert the result is
    the routed-only call's, bit for bit (the shared chunks add exact zeros)."""
    E, H, I, Is, M, topk = 6, 256, 128, 64, 3, 2
    hw, dw = build_experts(44, 0, E, H, I, range(E))
    hsw, dsw = build_shared(44, 0, H, Is)
    ids, gw = workloads.moe_routing(44, 0, M, E, topk)
    x = workloads.x_bf16(44, 0, 0, M, H)
    xd, idd, gwd = dev_x(x), dev(ids), dev(gw)
    a = host(nv.moe_shared_gemv(*dw, xd, idd, gwd, dsw))
    b = host(nv.moe_shared_gemv(*dw, xd, idd, gwd, dsw))
    assert np.array_equal(a, b)
    zero = (torch.zeros((2 * Is, H // 2), dtype=torch.uint8, device="cuda"),
            torch.zeros((2 * Is, H // 16), dtype=torch.uint8, device="cuda"),
            torch.ones(1, device="cuda"),
            torch.zeros((H, Is // 2), dtype=torch.uint8, device="cuda"),
            torch.zeros((H, Is // 16), dtype=torch.uint8, device="cuda"),
            torch.ones(1, device="cuda"))
    c = host(nv.moe_shared_gemv(*dw, xd, idd, gwd, zero))
    d = host(nv.moe_gemv(*dw, xd, idd, gwd))
    assert np.array_equal(c, d)
