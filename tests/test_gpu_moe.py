"""GPU MoE expert slots against the oracle: the 288-expert workload at full
per-expert size (M = 1 and M = 8; only routed experts are generated, the
rest stay zero), union sharing, duplicates, invalid ids and topk limits."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


def build_experts(wl, rep, E, H, I, used):
    """Oracle-packed (host) and GPU-packed (device) stacks; experts outside
    `used` are all-zero storage with g = 1. The two packs must agree."""
    hc13 = np.zeros((E, 2 * I, H // 2), np.uint8)
    hs13 = np.zeros((E, 2 * I, H // 16), np.uint8)
    hg13 = np.ones(E, np.float32)
    hc2 = np.zeros((E, H, I // 2), np.uint8)
    hs2 = np.zeros((E, H, I // 16), np.uint8)
    hg2 = np.ones(E, np.float32)
    dc13, ds13, dg13 = dev(hc13), dev(hs13), dev(hg13)
    dc2, ds2, dg2 = dev(hc2), dev(hs2), dev(hg2)
    for e in sorted(set(int(v) for v in used)):
        w13, w2 = workloads.moe_expert_weights(wl, rep, e, H, I)
        hc13[e], hs13[e], hg13[e] = oracle.pack(w13)
        hc2[e], hs2[e], hg2[e] = oracle.pack(w2)
        nv.pack_into(dev(w13), dc13[e], ds13[e], dg13[e:e + 1])
        nv.pack_into(dev(w2), dc2[e], ds2[e], dg2[e:e + 1])
    for a, b in [(hc13, dc13), (hs13, ds13), (hg13, dg13), (hc2, dc2), (hs2, ds2), (hg2, dg2)]:
        assert np.array_equal(host(b), a)
    return (hc13, hs13, hg13, hc2, hs2, hg2), (dc13, ds13, dg13, dc2, ds2, dg2)


def run_both(hw, dw, x, ids, gw, H, I, want_h=False):
    ws = torch.empty(nv.moe_workspace_bytes(ids.shape[0], H, I, ids.shape[1]),
                     dtype=torch.uint8, device="cuda")
    y = host(nv.moe_gemv(*dw, dev_x(x), dev(ids), dev(gw), workspace=ws))
    res = oracle.moe(*hw, x, ids, gw, want_h=want_h)
    return y, res, ws


@pytest.mark.parametrize("M", [1, 8])
def test_moe_workload_4_full_size(M):
    E, H, I, topk = 288, 4096, 1536, 8
    ids, gw = workloads.moe_routing(4, 0, M, E, topk)
    say(f"[moe] M={M} distinct experts={len(set(ids.ravel()))}")
    hw, dw = build_experts(4, 0, E, H, I, ids.ravel())
    x = workloads.x_bf16(4, 0, 0, M, H)
    y, (y_ref, bound, h_ref), ws = run_both(hw, dw, x, ids, gw, H, I, want_h=True)
    r = check_tol(y, y_ref, bound, f"moe M={M}")
    say(f"  max err / tol = {r:.3e}")
    # stage 1: the bf16 SwiGLU activations agree except for rare one-ulp
    # rounding flips (fp32 vs fp64 gate/up sums)
    lay = nv.moe_workspace_layout(M, H, I, topk)
    h = host(ws[lay["h"]:lay["h"] + M * topk * I * 2].view(torch.int16)).view(np.uint16)
    h = h.reshape(M * topk, I)
    same = np.mean(h == h_ref)
    ulp = np.abs(h.astype(np.int32) - h_ref.astype(np.int32))
    say(f"  h bit-equal fraction {same:.6f}, max ulp diff {ulp.max()}")
    assert same > 0.999


@pytest.mark.parametrize("H, I, topk", [(2048, 1024, 16), (2048, 768, 8), (6144, 256, 8)])
def test_moe_one_token_shapes(H, I, topk):
    """One token across the launch variants of its two passes: gate|up at
    H other than 4096 (the kernel without x staged in LDS), the down pass
    with all of a lane's (slot, chunk) pairs in flight at once: 512 pairs
    (8 per lane: 16 slots of I = 1024), 192 (3 per lane, run as 4) and 64.
    The slot ids hold a repeat and two invalid ids; y and the valid slots'
    h against the oracle."""
    E = 20
    rng = np.random.default_rng(H + I + topk)
    row = rng.choice(E, size=topk, replace=False).astype(np.int32)
    row[1] = row[0]
    row[2] = -1
    row[topk - 1] = E + 3
    ids = row.reshape(1, topk)
    gw = rng.random((1, topk)).astype(np.float32)
    say(f"[moe] one token H={H} I={I} topk={topk} ids={row.tolist()}")
    valid = (row >= 0) & (row < E)
    hw, dw = build_experts(49, 0, E, H, I, row[valid])
    x = workloads.x_bf16(49, 1, topk, 1, H)
    y, (y_ref, bound, h_ref), ws = run_both(hw, dw, x, ids, gw, H, I, want_h=True)
    check_tol(y, y_ref, bound, f"moe one token H={H} I={I} topk={topk}")
    lay = nv.moe_workspace_layout(1, H, I, topk)
    h = host(ws[lay["h"]:lay["h"] + topk * I * 2].view(torch.int16)).view(np.uint16)
    h = h.reshape(topk, I)[valid]
    hr = np.asarray(h_ref).reshape(topk, I)[valid]
    ulp = np.abs(h.astype(np.int32) - hr.astype(np.int32))
    say(f"  h bit-equal fraction {np.mean(ulp == 0):.6f}, max ulp diff {ulp.max()}")
    assert ulp.max() <= 1 and np.mean(ulp == 0) > 0.99


@pytest.mark.parametrize("case", ["same_8_experts", "one_expert_all_tokens", "odd_tokens"])
def test_moe_gate_up_passes_at_h4096(case):
    """H = 4096 at M >= 2 loads a wavefront's gate|up weights once for all
    its passes of two slots and stages each pass's activation rows in LDS:
    experts named by 8 slots (four passes), one expert named by every token,
    and 5 tokens on the same experts (a last pass with a lone slot); y and
    every valid h against the oracle."""
    E, H, I, topk = 16, 4096, 256, 8
    rng = np.random.default_rng(len(case))
    if case == "same_8_experts":
        M = 8
        ids = np.tile(rng.choice(E, size=topk, replace=False).astype(np.int32), (M, 1))
    elif case == "one_expert_all_tokens":
        M = 8
        ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
        ids[:, 0] = 3
        for m in range(M):   # keep a token's experts distinct
            row = ids[m]
            dup = np.flatnonzero(row[1:] == 3) + 1
            row[dup] = [e for e in range(E) if e not in row][:len(dup)]
    else:
        M = 5
        ids = np.tile(np.arange(topk, dtype=np.int32), (M, 1))
    gw = rng.random((M, topk)).astype(np.float32)
    say(f"[moe] gate|up passes at H=4096: {case} M={M} ids[0]={ids[0].tolist()}")
    hw, dw = build_experts(51, 0, E, H, I, ids.ravel())
    x = workloads.x_bf16(51, M, len(case), M, H)
    y, (y_ref, bound, h_ref), ws = run_both(hw, dw, x, ids, gw, H, I, want_h=True)
    check_tol(y, y_ref, bound, f"moe {case}")
    lay = nv.moe_workspace_layout(M, H, I, topk)
    h = host(ws[lay["h"]:lay["h"] + M * topk * I * 2].view(torch.int16)).view(np.uint16)
    ulp = np.abs(h.reshape(M * topk, I).astype(np.int32) - h_ref.astype(np.int32))
    say(f"  h bit-equal fraction {np.mean(ulp == 0):.6f}, max ulp diff {ulp.max()}")
    assert ulp.max() <= 1 and np.mean(ulp == 0) > 0.99


def test_moe_shared_experts_union():
    """All 8 rows route to the same 8 experts (each expert streamed once for
    8 slots), in different slot orders."""
    E, H, I, topk, M = 16, 512, 256, 8, 8
    base = np.array([3, 9, 0, 15, 7, 1, 12, 4], np.int32)
    g = np.random.default_rng(1)
    ids = np.stack([g.permutation(base) for _ in range(M)]).astype(np.int32)
    gw = g.dirichlet(np.ones(topk), size=M).astype(np.float32)
    hw, dw = build_experts(40, 0, E, H, I, base)
    x = workloads.x_bf16(40, 0, 0, M, H)
    y, (y_ref, bound), _ = run_both(hw, dw, x, ids, gw, H, I)
    check_tol(y, y_ref, bound, "shared union")


def test_moe_duplicates_invalid_ids_and_limits():
    E, H, I = 6, 256, 128
    hw, dw = build_experts(41, 0, E, H, I, range(E))
    cases = {
        "dup_in_row": np.array([[2, 2, 5], [1, 1, 1]], np.int32),
        "invalid": np.array([[-1, 3, 6], [1000, -7, 0]], np.int32),
        "all_invalid": np.array([[-1, 6, 99]], np.int32),
        "topk1": np.array([[4], [0], [5]], np.int32),
        "topk16": np.tile(np.arange(16, dtype=np.int32) % E, (2, 1)),
        "m8": np.random.default_rng(2).integers(0, E, size=(8, 4)).astype(np.int32),
    }
    for name, ids in cases.items():
        say(f"[moe] {name} ids={ids.tolist()}")
        M, topk = ids.shape
        gw = np.random.default_rng(M * 31 + topk).random((M, topk)).astype(np.float32)
        x = workloads.x_bf16(41, M, topk, M, H)
        y, (y_ref, bound), _ = run_both(hw, dw, x, ids, gw, H, I)
        check_tol(y, y_ref, bound, name)
        if name == "all_invalid":
            assert np.all(y == 0)


@pytest.mark.parametrize("M", range(1, 9))
def test_moe_every_m(M):
    """Every token count (M = 1 takes the one-slot-per-pass gate|up and the
    per-wavefront down pass; M >= 2 the slot union and the split down pass),
    with a repeated id in the first token and 128 slots at M = 8."""
    E, H, I = 6, 256, 128
    hw, dw = build_experts(47, 0, E, H, I, range(E))
    topk = 16 if M == 8 else 4
    ids = np.random.default_rng(M).integers(0, E, size=(M, topk)).astype(np.int32)
    ids[0, 1] = ids[0, 0]
    gw = np.random.default_rng(M + 100).random((M, topk)).astype(np.float32)
    say(f"[moe] every M: M={M} topk={topk} ids[0]={ids[0].tolist()}")
    x = workloads.x_bf16(47, M, topk, M, H)
    y, (y_ref, bound), _ = run_both(hw, dw, x, ids, gw, H, I)
    check_tol(y, y_ref, bound, f"M={M}")


@pytest.mark.parametrize("M", [1, 2, 3])
def test_moe_minimum_sizes(M):
    """One expert and H = I = 32: one 32-element chunk per slot, so the down
    pass's (slot, chunk) decode divides by 1, and every slot names expert 0."""
    E, H, I, topk = 1, 32, 32, 2
    hw, dw = build_experts(48, M, E, H, I, [0])
    ids = np.zeros((M, topk), np.int32)
    gw = np.random.default_rng(M).random((M, topk)).astype(np.float32)
    x = workloads.x_bf16(48, M, 0, M, H)
    say(f"[moe] minimum sizes M={M}")
    y, (y_ref, bound), _ = run_both(hw, dw, x, ids, gw, H, I)
    check_tol(y, y_ref, bound, f"minimum M={M}")


def test_moe_empty_batch():
    E, H, I = 2, 64, 32
    hw, dw = build_experts(42, 0, E, H, I, [])
    y = nv.moe_gemv(*dw, torch.zeros((0, H), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                    torch.zeros((0, 2), dtype=torch.float32, device="cuda"))
    assert y.shape == (0, H)


@pytest.mark.parametrize("case", ["one_expert_all_tokens", "same_experts_all_tokens"])
def test_moe_skewed_routing(case):
    """Skewed routing at M = 8, full per-expert size: one expert named by all
    eight tokens (slot 0 of every token; the other slots distinct), or all
    tokens naming the same eight experts (in permuted slot order, different
    gate weights). The gate|up pass streams a shared expert's rows for all
    its slots and the down pass reads them per token (the L2 serves the
    repeats); the result is checked against the oracle."""
    E, H, I, topk, M = 288, 4096, 1536, 8, 8
    rng = np.random.default_rng(77)
    if case == "one_expert_all_tokens":
        ids, gw = workloads.moe_routing(4, 3, M, E, topk)
        ids = ids.copy()
        for m in range(M):
            row = [e for e in ids[m] if e != 7][:topk - 1]
            while len(row) < topk - 1:
                row.append(int(rng.integers(8, E)))
            ids[m] = [7] + row
    else:
        ids = np.stack([rng.permutation(np.arange(40, 48)) for _ in range(M)]).astype(np.int32)
        gw = rng.random((M, topk)).astype(np.float32)
    ids = ids.astype(np.int32)
    say(f"[moe] skewed routing {case}: distinct experts={len(set(ids.ravel()))}")
    hw, dw = build_experts(4, 3, E, H, I, ids.ravel())
    x = workloads.x_bf16(4, 3, 1, M, H)
    y, (y_ref, bound), _ = run_both(hw, dw, x, ids, gw, H, I)
    r = check_tol(y, y_ref, bound, f"moe {case}")
    say(f"  max err / tol = {r:.3e}")
