"""Every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: each replay, with eager launches and synchronisations between the
replays and the graph's outputs poisoned before each one, must reproduce the
eager result bit for bit. Covers the vector-ALU, split-K and other-K MFMA
GEMV paths, the segmented GEMV, the MoE with and without a shared expert,
the W4A4 MoE (at M = 3 and on the single-token path), and the W4A4
quantizer and GEMV (direct and decoded paths, one matrix or several).
Nothing here clears memory with hipMemsetAsync, so nothing of the kind is
recorded into a graph."""
import numpy as np
import pytest
import torch

import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import dev, dev_x, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def check_graph(name, run, outs, disturb):
    """run(): launches into outs (a list of tensors); disturb(): eager work
    with other inputs and outputs."""
    say(f"[graph] {name}")
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in outs:
            if o.is_floating_point():
                o.fill_(float("nan"))
            else:
                o.fill_(0x7F)
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} replay {rep}"
        disturb()
    del g


def _gemv_case(M, N, K, seed):
    c, s = workloads.random_nvfp4(1, seed, 0, N, K, 0x30, 0x48)
    c, s = dev(c), dev(s)
    g = dev(np.array([0.0123], np.float32))
    x = dev_x(workloads.x_bf16(1, seed, 1, M, K))
    return c, s, g, x


@pytest.mark.parametrize("M,N,K", [(1, 5000, 4096), (2, 40003, 64), (5, 3000, 4096),
                                   (8, 700, 12288), (3, 300, 4128)])
def test_graph_gemv(M, N, K):
    c, s, g, x = _gemv_case(M, N, K, M * 7 + N)
    y = torch.empty((M, N), device="cuda")
    c2, s2, g2, x2 = _gemv_case(M, N, K, M * 7 + N + 1)
    y2 = torch.empty((M, N), device="cuda")
    check_graph(f"gemv M={M} N={N} K={K}", lambda: nv.gemv_into(c, s, g, x, y), [y],
                lambda: nv.gemv_into(c2, s2, g2, x2, y2))


@pytest.mark.parametrize("M", [2, 5])
def test_graph_segments(M):
    K = 4096
    mats = [_gemv_case(M, N, K, 100 + i)[:3] for i, N in enumerate((1024, 256, 256))]
    x = dev_x(workloads.x_bf16(1, 100, 9, M, K))
    ys = [torch.empty((M, m[0].shape[0]), device="cuda") for m in mats]
    x2 = dev_x(workloads.x_bf16(1, 101, 9, M, K))
    ys2 = [torch.empty_like(y) for y in ys]
    check_graph(f"segments M={M}", lambda: nv.gemv_segments_into(mats, x, ys), ys,
                lambda: nv.gemv_segments_into(mats, x2, ys2))


def _experts(E, H, I, seed):
    w = []
    for name, N, K in (("13", 2 * I, H), ("2", H, I)):
        cs, ss = zip(*[workloads.random_nvfp4(2, seed, e + (0 if name == "13" else 100), N, K,
                                              0x30, 0x40) for e in range(E)])
        w += [dev(np.stack(cs)), dev(np.stack(ss)),
              dev(np.full(E, 0.01 if name == "13" else 0.02, np.float32))]
    return w


def _shared(H, Is, seed):
    c13, s13 = workloads.random_nvfp4(2, seed, 200, 2 * Is, H, 0x30, 0x40)
    c2, s2 = workloads.random_nvfp4(2, seed, 201, H, Is, 0x30, 0x40)
    return (dev(c13), dev(s13), dev(np.array([0.01], np.float32)),
            dev(c2), dev(s2), dev(np.array([0.02], np.float32)))


@pytest.mark.parametrize("kind", ["routed", "shared", "w4a4", "w4a4_shared", "w4a4_m1",
                                  "w4a4_shared_m1"])
def test_graph_moe(kind):
    """M = 3, and M = 1 for W4A4 (the two-launch single-token path)."""
    E, H, I, topk = 6, 512, 256, 4
    M = 1 if kind.endswith("_m1") else 3
    w = _experts(E, H, I, 5)
    sh = _shared(H, 96, 5) if "shared" in kind else None
    Is = 96 if sh is not None else 0
    ids, gw = workloads.moe_routing(2, 5, M, E, topk)
    ids[M - 1, 2] = -1                               # an invalid slot too
    ids, gw = dev(ids), dev(gw)
    x = dev_x(workloads.x_bf16(2, 5, 0, M, H))
    x2 = dev_x(workloads.x_bf16(2, 6, 0, M, H))
    y, y2 = torch.empty((M, H), device="cuda"), torch.empty((M, H), device="cuda")
    gx = dev(np.array([np.abs(workloads.x_bf16(2, 7, 0, M, H).astype(np.uint32) << 16)
                       .view(np.float32).max() / 2688.0], np.float32))
    gh = dev(np.array([0.0005], np.float32))
    if kind.startswith("w4a4"):
        nb = nv.moe_w4a4_workspace_bytes(M, H, I, topk, Is)
    elif sh is not None:
        nb = nv.moe_shared_workspace_bytes(M, H, I, topk, Is)
    else:
        nb = nv.moe_workspace_bytes(M, H, I, topk)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def call(xx, yy, wsx):
        if kind.startswith("w4a4"):
            nv.moe_w4a4_gemv_into(*w, xx, gx, gh, ids, gw, yy, wsx, shared=sh)
        elif sh is not None:
            nv.moe_shared_gemv_into(*w, xx, ids, gw, sh, yy, wsx)
        else:
            nv.moe_gemv_into(*w, xx, ids, gw, yy, wsx)

    check_graph(f"moe {kind}", lambda: call(x, y, ws), [y], lambda: call(x2, y2, ws2))


@pytest.mark.parametrize("M", [2, 4])
def test_graph_w4a4(M):
    N, K = 1000, 4096
    c, s, g, x = _gemv_case(M, N, K, 300 + M)
    gx = dev(np.array([0.002], np.float32))
    cx = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), device="cuda")
    ws = torch.empty(nv.gemv_w4a4_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    x2 = dev_x(workloads.x_bf16(1, 301, 1, M, K))
    cx2, sx2, y2 = torch.empty_like(cx), torch.empty_like(sx), torch.empty_like(y)
    ws2 = torch.empty_like(ws)

    def run():
        nv.quantize_act_into(x, gx, cx, sx)
        nv.gemv_w4a4_into(c, s, g, cx, sx, gx, y, ws)

    def disturb():
        nv.quantize_act_into(x2, gx, cx2, sx2)
        nv.gemv_w4a4_into(c, s, g, cx2, sx2, gx, y2, ws2)

    check_graph(f"w4a4 M={M}", run, [cx, sx, y], disturb)


@pytest.mark.parametrize("M", [2, 4])
def test_graph_w4a4_segments(M):
    K = 4096
    mats = [_gemv_case(M, N, K, 400 + i)[:3] for i, N in enumerate((1024, 300))]
    x = dev_x(workloads.x_bf16(1, 400, 9, M, K))
    gx = dev(np.array([0.002], np.float32))
    cx, sx = nv.quantize_act(x, gx)
    ys = [torch.empty((M, m[0].shape[0]), device="cuda") for m in mats]
    ws = torch.empty(nv.gemv_w4a4_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    cx2, sx2 = nv.quantize_act(dev_x(workloads.x_bf16(1, 401, 9, M, K)), gx)
    ys2 = [torch.empty_like(y) for y in ys]
    ws2 = torch.empty_like(ws)
    check_graph(f"w4a4 segments M={M}",
                lambda: nv.gemv_w4a4_segments_into(mats, cx, sx, gx, ys, ws), ys,
                lambda: nv.gemv_w4a4_segments_into(mats, cx2, sx2, gx, ys2, ws2))
