"""nvfp4_moe_gemv_noalloc through the C ABI against nvfp4_moe_gemv (the same
kernels with a caller workspace): two calls in a row, the second smaller, so
the library's device array is reused with a different layout; both outputs
must equal the workspace entry point's bit for bit and be within the oracle's
tolerance. A call too large for the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


def experts(wl, E, H, I):
    hw = [[], [], [], [], [], []]
    for e in range(E):
        w13, w2 = workloads.moe_expert_weights(wl, 0, e, H, I)
        for k, v in enumerate((*oracle.pack(w13), *oracle.pack(w2))):
            hw[k].append(v)
    return [np.stack(a) if a[0].ndim else np.array(a, np.float32) for a in hw]


def call_c(fn, dw, x, ids, gw, y, ws=None):
    """One C-ABI call (ctypes, no binding logic): nvfp4_moe_gemv with `ws`,
    or nvfp4_moe_gemv_noalloc without it."""
    L = nv.lib()
    E, twoI, Hh = dw[0].shape
    M, topk = ids.shape
    args = [t.data_ptr() for t in dw] + [x.data_ptr(), ids.data_ptr(), gw.data_ptr(),
                                         M, E, Hh * 2, twoI // 2, topk, y.data_ptr()]
    stream = torch.cuda.current_stream().cuda_stream
    if ws is None:
        st = getattr(L, fn)(*args, stream)
    else:
        st = getattr(L, fn)(*args, ws.data_ptr(), ws.numel(), stream)
    assert st == 0, (fn, st, L.nvfp4_last_error())


def test_noalloc_matches_workspace_entry_point():
    cases = [
        # (workload stream, E, H, I, M, topk): the first call fills more of the
        # array than the second
        (61, 12, 512, 256, 8, 8),
        (62, 5, 256, 128, 3, 4),
    ]
    for wl, E, H, I, M, topk in cases:
        say(f"[noalloc] E={E} H={H} I={I} M={M} topk={topk}")
        hw = experts(wl, E, H, I)
        dw = [dev(a) for a in hw]
        ids = np.random.default_rng(wl).integers(0, E, size=(M, topk)).astype(np.int32)
        ids[0, -1] = -1                       # an invalid slot adds nothing
        gw = np.random.default_rng(wl + 1).random((M, topk)).astype(np.float32)
        xb = workloads.x_bf16(wl, 0, 0, M, H)
        x, dids, dgw = dev_x(xb), dev(ids), dev(gw)
        y_na = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
        y_ws = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(nv.moe_workspace_bytes(M, H, I, topk), dtype=torch.uint8,
                         device="cuda")
        call_c("nvfp4_moe_gemv_noalloc", dw, x, dids, dgw, y_na)
        call_c("nvfp4_moe_gemv", dw, x, dids, dgw, y_ws, ws)
        a, b = host(y_na), host(y_ws)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        y_ref, bound = oracle.moe(*hw, xb, ids, gw)
        r = check_tol(a, y_ref, bound, f"noalloc M={M}")
        say(f"  bit-equal to nvfp4_moe_gemv; max err / tol = {r:.3e}")


def test_noalloc_refuses_a_call_larger_than_its_array():
    L = nv.lib()
    y = torch.empty((8, 4096), dtype=torch.float32, device="cuda")
    # M * topk * I * 2 = 8 * 16 * 32768 * 2 = 8 MiB > 4 MiB
    st = L.nvfp4_moe_gemv_noalloc(*([y.data_ptr()] * 9), 8, 4, 4096, 32768, 16,
                                  y.data_ptr(), None)
    assert st == 4   # NVFP4_ERR_UNSUPPORTED
    assert b"scratch" in L.nvfp4_last_error()
