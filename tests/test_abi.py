"""The C ABI boundary on the CPU: the library loads, exports every entry point
include/nvfp4_gemv.h declares, and rejects bad arguments on the host before
any HIP call (only argument checks run here; nothing is launched)."""
import ctypes
import re

import pytest

import nvfp4_block_scaled_gemv_amd as nv

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIAS = range(8)

# Fake, never-dereferenced device addresses: every call below fails its host
# checks before it could touch them.
A = 0x7F0000000000
B = 0x7F0100000000


@pytest.fixture(scope="module")
def L():
    return nv.lib()


def declared_functions():
    text = open(nv.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"nvfp4_pack", "nvfp4_dequant", "nvfp4_gemv", "nvfp4_gemv_segments", "nvfp4_moe_gemv",
            "nvfp4_moe_workspace_bytes", "nvfp4_moe_shared_gemv",
            "nvfp4_moe_shared_workspace_bytes", "nvfp4_quantize_act", "nvfp4_gemv_w4a4",
            "nvfp4_gemv_w4a4_workspace_bytes", "nvfp4_gemv_w4a4_segments", "nvfp4_moe_w4a4_gemv",
            "nvfp4_moe_w4a4_workspace_bytes", "nvfp4_abi_version", "nvfp4_status_string",
            "nvfp4_last_error", "nvfp4_stream_read", "nvfp4_moe_gemv_noalloc",
            "nvfp4_check_device_faults", "nvfp4_debug_set_wait_limit"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.nvfp4_abi_version() == 9
    for s in range(8):
        assert L.nvfp4_status_string(s)
    assert L.nvfp4_status_string(99) == b"unknown status"


def test_binding_limits_match_the_header():
    text = open(nv.HEADER_PATH).read()
    defs = dict(re.findall(r"#define (NVFP4_[A-Z_]+) \(?([0-9LU]+(?: << [0-9]+)?)\)?", text))

    def value(name):
        v = defs[name].replace("LL", "").replace("U", "")
        if "<<" in v:
            a, b = v.split("<<")
            return int(a) << int(b)
        return int(v)

    assert value("NVFP4_MAX_M") == nv.MAX_M
    assert value("NVFP4_MOE_MAX_M") == nv.MOE_MAX_M
    assert value("NVFP4_MAX_TOPK") == nv.MAX_TOPK
    assert value("NVFP4_MAX_N") == nv.MAX_N
    assert value("NVFP4_MAX_K") == nv.MAX_K
    assert value("NVFP4_MOE_MAX_I") == nv.MOE_MAX_I
    assert value("NVFP4_MOE_MAX_H") == nv.MOE_MAX_H
    assert value("NVFP4_MAX_SEGMENTS") == nv.MAX_SEGMENTS
    assert value("NVFP4_NOALLOC_SCRATCH_BYTES") == nv.NOALLOC_SCRATCH_BYTES


def _err(L):
    return L.nvfp4_last_error().decode()


def test_gemv_rejects_k_past_its_limit(L):
    """K above NVFP4_MAX_K is refused on the host by every GEMV entry point."""
    K = nv.MAX_K + 32
    assert L.nvfp4_gemv(A, A, A, A, 9, 16, K, B, None) == ERR_UNSUPPORTED
    assert "K=" in _err(L)
    assert L.nvfp4_gemv_w4a4(A, A, A, A, A, A, 1, 16, K, B, A, 1 << 30, None) == ERR_UNSUPPORTED


def test_gemv_rejects_bad_shapes(L):
    assert L.nvfp4_gemv(A, A, A, A, 1, 16, 48, B, None) == ERR_SHAPE       # K % 32
    assert "K % 32" in _err(L)
    assert L.nvfp4_gemv(A, A, A, A, -1, 16, 64, B, None) == ERR_SHAPE
    assert L.nvfp4_gemv(A, A, A, A, 129, 16, 64, B, None) == ERR_UNSUPPORTED
    assert L.nvfp4_gemv(A, A, A, A, 1, (1 << 30) + 1, 64, B, None) == ERR_UNSUPPORTED   # N
    assert "N=" in _err(L)
    assert L.nvfp4_gemv(A, A, A, A, 0, 16, 64, B, None) == OK              # nothing to do
    assert L.nvfp4_gemv(A, A, A, A, 2, 0, 64, B, None) == OK


def test_gemv_rejects_null_and_misaligned(L):
    assert L.nvfp4_gemv(None, A, A, A, 1, 16, 64, B, None) == ERR_NULL
    assert L.nvfp4_gemv(A, A, A, A, 1, 16, 64, None, None) == ERR_NULL
    assert L.nvfp4_gemv(A + 8, A, A, A, 1, 16, 64, B, None) == ERR_ALIGN   # codes 16B
    assert L.nvfp4_gemv(A, A + 1, A, A, 1, 16, 64, B, None) == ERR_ALIGN   # scales 2B
    assert L.nvfp4_gemv(A, A, A, A + 4, 1, 16, 64, B, None) == ERR_ALIGN   # x 16B
    assert L.nvfp4_gemv(A, A, A, A, 1, 16, 64, B + 2, None) == ERR_ALIGN   # y 4B


def test_gemv_rejects_aliasing(L):
    # y overlapping x
    codes, scales, g, x = A, A + 0x10000, A + 0x20000, A + 0x30000
    assert L.nvfp4_gemv(codes, scales, g, x, 1, 16, 64, x + 16, None) == ERR_ALIAS
    assert L.nvfp4_gemv(codes, scales, g, x, 1, 16, 64, codes, None) == ERR_ALIAS


def test_pack_and_dequant_checks(L):
    assert L.nvfp4_pack(A, 4, 24, A, A, A, None, None) == ERR_SHAPE
    assert L.nvfp4_pack(A, 4, 32, A, A, None, None, None) == ERR_NULL
    assert L.nvfp4_pack(A + 4, 4, 32, B, B + 0x1000, B + 0x2000, None, None) == ERR_ALIGN
    assert L.nvfp4_pack(A, 4, 32, A + 64, B, B + 0x1000, None, None) == ERR_ALIAS
    assert L.nvfp4_dequant(A, A, A, 4, 16, B, None) == ERR_SHAPE             # K % 32
    assert L.nvfp4_dequant(A, A, A, 0, 32, B, None) == OK
    assert L.nvfp4_dequant(A, A, A, 4, 32, A + 8, None) == ERR_ALIGN
    assert L.nvfp4_dequant(A, A + 0x1000, A + 0x2000, 4, 32, A, None) == ERR_ALIAS


def test_moe_checks(L):
    ws = nv.moe_workspace_bytes(8, 4096, 1536, 8)
    assert ws == nv.moe_workspace_layout(8, 4096, 1536, 8)["total"]
    assert ws == 64 * 1536 * 2   # bf16 h[M*topk, I], already a multiple of 256
    assert nv.moe_workspace_bytes(1, 64, 32, 3) == 256
    args = [A + i * 0x10000000 for i in range(9)]
    f = L.nvfp4_moe_gemv
    assert f(*args, 1, 4, 64, 48, 2, B, B + 0x1000000, ws, None) == ERR_SHAPE   # I % 32
    assert f(*args, 9, 4, 64, 64, 2, B, B + 0x1000000, ws, None) == ERR_UNSUPPORTED
    assert f(*args, 1, 4, 64, 64, 17, B, B + 0x1000000, ws, None) == ERR_UNSUPPORTED
    assert f(*args, 1, 0, 64, 64, 2, B, B + 0x1000000, ws, None) == ERR_SHAPE
    big_i = (1 << 24) + 32
    assert f(*args, 1, 4, 64, big_i, 2, B, B + 0x1000000, 1 << 40, None) == ERR_UNSUPPORTED
    big_h = (1 << 24) + 32
    assert f(*args, 1, 4, big_h, 64, 2, B, B + 0x1000000, 1 << 40, None) == ERR_UNSUPPORTED
    need = nv.moe_workspace_bytes(1, 64, 64, 2)
    assert f(*args, 1, 4, 64, 64, 2, B, B + 0x1000000, need - 1, None) == ERR_WORKSPACE
    assert f(*args, 1, 4, 64, 64, 2, B, None, need, None) == ERR_WORKSPACE
    assert f(*args, 1, 4, 64, 64, 2, B, B + 0x1000000 + 64, need, None) == ERR_ALIGN
    assert f(*args, 1, 4, 64, 64, 2, args[6], B + 0x1000000, need, None) == ERR_ALIAS
    assert f(*args, 0, 4, 64, 64, 2, B, B + 0x1000000, need, None) == OK


def test_moe_shared_checks(L):
    """Host-side validation of the MoE call with a shared expert (no launch)."""
    Sh = nv.MoeShared
    ws = nv.moe_shared_workspace_bytes(8, 4096, 1536, 8, 768)
    assert ws == nv.moe_shared_workspace_layout(8, 4096, 1536, 8, 768)["total"]
    assert ws == 64 * 1536 * 2 + 8 * 768 * 2
    assert nv.moe_shared_workspace_bytes(1, 64, 32, 3, 32) == 512
    assert nv.moe_shared_workspace_bytes(1, 64, 32, 3, -32) == 0
    args = [A + i * 0x10000000 for i in range(9)]
    sh_base = [A + 0x90000000 + i * 0x1000000 for i in range(6)]
    f = L.nvfp4_moe_shared_gemv
    Y, WS = B, B + 0x1000000
    need = nv.moe_shared_workspace_bytes(1, 64, 64, 2, 96)
    good = Sh(*sh_base, 96)
    assert f(*args, 1, 4, 64, 64, 2, None, Y, WS, need, None) == ERR_NULL
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(Sh(*sh_base, 80)), Y, WS, need,
             None) == ERR_SHAPE                                              # Is % 32
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(Sh(*sh_base, 0)), Y, WS, need,
             None) == ERR_SHAPE
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(Sh(*sh_base, (1 << 24) + 32)), Y, WS,
             1 << 40, None) == ERR_UNSUPPORTED
    nul = Sh(*sh_base, 96)
    nul.w2_scales = None
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(nul), Y, WS, need, None) == ERR_NULL
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(good), Y, WS, need - 1, None) == ERR_WORKSPACE
    # the routed-only size is too small once a shared expert needs hs
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(good), Y, WS,
             nv.moe_workspace_bytes(1, 64, 64, 2), None) == ERR_WORKSPACE
    mis = Sh(*sh_base, 96)
    mis.w2_codes = sh_base[3] + 8
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(mis), Y, WS, need, None) == ERR_ALIGN
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(good), sh_base[0], WS, need,
             None) == ERR_ALIAS                                              # y on WS13
    assert f(*args, 1, 4, 64, 64, 2, ctypes.byref(good), Y, sh_base[4], need,
             None) == ERR_ALIAS                                              # workspace on WS2 scales
    assert f(*args, 0, 4, 64, 64, 2, ctypes.byref(good), Y, WS, need, None) == OK


def test_moe_w4a4_checks(L):
    """Host-side validation of the W4A4 MoE call (no launch)."""
    Sh = nv.MoeShared
    lay = nv.moe_w4a4_workspace_layout(8, 4096, 1536, 8, 768)
    assert nv.moe_w4a4_workspace_bytes(8, 4096, 1536, 8, 768) == lay["total"]
    assert lay["hq"] == nv.moe_shared_workspace_bytes(8, 4096, 1536, 8, 768)
    assert lay["total"] == lay["hq"] + 64 * 1536 * 2 + 8 * 4096 * 2
    assert nv.moe_w4a4_workspace_bytes(1, 64, 32, 3, 0) == 256 + 256 + 256
    assert nv.moe_w4a4_workspace_bytes(1, 64, 32, -3, 0) == 0
    w = [A + i * 0x10000000 for i in range(7)]          # w13 x3, w2 x3, x
    gx, gh = A + 0x70000000, A + 0x70000100
    ids, gw = A + 0x80000000, A + 0x80001000
    sh_base = [A + 0x90000000 + i * 0x1000000 for i in range(6)]
    f = L.nvfp4_moe_w4a4_gemv
    Y, WS = B, B + 0x1000000
    need = nv.moe_w4a4_workspace_bytes(1, 64, 64, 2, 0)
    assert f(*w, None, gh, ids, gw, 1, 4, 64, 64, 2, None, Y, WS, need, None) == ERR_NULL
    assert f(*w, gx, None, ids, gw, 1, 4, 64, 64, 2, None, Y, WS, need, None) == ERR_NULL
    assert f(*w, gx + 2, gh, ids, gw, 1, 4, 64, 64, 2, None, Y, WS, need, None) == ERR_ALIGN
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 48, 2, None, Y, WS, need, None) == ERR_SHAPE
    assert f(*w, gx, gh, ids, gw, 9, 4, 64, 64, 2, None, Y, WS, 1 << 40,
             None) == ERR_UNSUPPORTED
    # the W4A16 size lacks the quantized h and x
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 64, 2, None, Y, WS,
             nv.moe_workspace_bytes(1, 64, 64, 2), None) == ERR_WORKSPACE
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 64, 2, None, Y, WS, need - 1,
             None) == ERR_WORKSPACE
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 64, 2, None, gx, WS, need,
             None) == ERR_ALIAS                                              # y on g_x
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 64, 2, None, Y, gh - 256, need,
             None) == ERR_ALIAS                                              # workspace on g_h
    good = Sh(*sh_base, 96)
    need_s = nv.moe_w4a4_workspace_bytes(1, 64, 64, 2, 96)
    assert need_s > need
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 64, 2, ctypes.byref(good), Y, WS, need,
             None) == ERR_WORKSPACE
    nul = Sh(*sh_base, 96)
    nul.w13_gscale = None
    assert f(*w, gx, gh, ids, gw, 1, 4, 64, 64, 2, ctypes.byref(nul), Y, WS, need_s,
             None) == ERR_NULL
    assert f(*w, gx, gh, ids, gw, 0, 4, 64, 64, 2, ctypes.byref(good), Y, WS, need_s,
             None) == OK


def test_w4a4_checks(L):
    """Host-side validation of the W4A4 calls (no launch)."""
    q = L.nvfp4_quantize_act
    X, G, C, S = A, A + 0x1000000, A + 0x2000000, A + 0x3000000
    assert q(X, 2, 48, G, C, S, None) == ERR_SHAPE                # K % 32
    assert q(X, -1, 64, G, C, S, None) == ERR_SHAPE
    assert q(X, 0, 64, G, C, S, None) == OK
    assert q(X, 2, 64, None, C, S, None) == ERR_NULL
    assert q(X + 8, 2, 64, G, C, S, None) == ERR_ALIGN
    assert q(X, 2, 64, G, X, S, None) == ERR_ALIAS                # codes over x
    assert q(X, 2, 64, G, C, C + 16, None) == ERR_ALIAS           # scales over codes
    f = L.nvfp4_gemv_w4a4
    assert nv.gemv_w4a4_workspace_bytes(8, 4096) == 8 * 4096 * 2 + 256
    assert nv.gemv_w4a4_workspace_bytes(1, 32) == 256 + 256
    w = [A + i * 0x1000000 for i in range(6)]
    Y, WS = B, B + 0x1000000
    need = nv.gemv_w4a4_workspace_bytes(2, 64)
    assert f(*w, 2, 16, 48, Y, WS, need, None) == ERR_SHAPE
    assert f(*w, 129, 16, 64, Y, WS, need, None) == ERR_UNSUPPORTED
    assert f(*w, 2, (1 << 30) + 1, 64, Y, WS, need, None) == ERR_UNSUPPORTED
    assert f(*w, 0, 16, 64, Y, WS, need, None) == OK
    assert f(*w, 2, 16, 64, Y, WS, need - 1, None) == ERR_WORKSPACE
    assert f(*w, 2, 16, 64, Y, None, need, None) == ERR_WORKSPACE
    assert f(*w[:5], None, 2, 16, 64, Y, WS, need, None) == ERR_NULL
    assert f(*w, 2, 16, 64, Y, WS + 64, need, None) == ERR_ALIGN
    assert f(*w, 2, 16, 64, w[3], WS, need, None) == ERR_ALIAS    # y over codes_x
    assert f(*w, 2, 16, 64, Y, w[0], need, None) == ERR_ALIAS     # workspace over codes_w


def test_binding_raises_without_device_tensors():
    import torch
    with pytest.raises(ValueError):
        nv.gemv(torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(4, 2, dtype=torch.uint8),
                torch.ones(1), torch.zeros(1, 32, dtype=torch.bfloat16))


def test_gemv_segments_checks(L):
    """Host-side validation of the fused multi-projection call (no launch)."""
    Seg = nv.GemvSegment
    arr = (Seg * 9)()
    for i in range(9):
        arr[i] = Seg(A + i * 0x100000, A + 0x10000000 + i * 0x10000, A + 0x20000000 + 16 * i,
                     B + i * 0x100000, 64)
    f = L.nvfp4_gemv_segments
    X = A + 0x30000000
    assert f(arr, 9, X, 1, 64, None) == ERR_UNSUPPORTED          # > 8 segments
    assert f(arr, 2, X, 129, 64, None) == ERR_UNSUPPORTED        # M > 128
    assert f(arr, 2, X, 1, 48, None) == ERR_SHAPE                # K % 32
    assert f(arr, -1, X, 1, 64, None) == ERR_SHAPE
    assert f(None, 2, X, 1, 64, None) == ERR_NULL
    assert f(arr, 0, X, 1, 64, None) == OK                       # nothing to do
    assert f(arr, 2, X, 0, 64, None) == OK                       # M == 0
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].N = -1
    assert f(bad, 2, X, 1, 64, None) == ERR_SHAPE
    bad = (Seg * 2)(arr[0], arr[1])
    bad[0].N = bad[1].N = (1 << 29) + 1                         # together above 2^30 rows
    assert f(bad, 2, X, 1, 64, None) == ERR_UNSUPPORTED
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].y = None
    assert f(bad, 2, X, 1, 64, None) == ERR_NULL
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].codes = A + 8
    assert f(bad, 2, X, 1, 64, None) == ERR_ALIGN
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].y = bad[0].y + 16                                    # outputs overlap
    assert f(bad, 2, X, 1, 64, None) == ERR_ALIAS
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].y = bad[0].codes                                     # output on an input
    assert f(bad, 2, X, 1, 64, None) == ERR_ALIAS
    bad = (Seg * 2)(arr[0], arr[1])
    bad[0].y = X                                                # output on x
    assert f(bad, 2, X, 1, 64, None) == ERR_ALIAS
    assert "segment" in L.nvfp4_last_error().decode()


def test_last_error_is_per_thread(L):
    """nvfp4_last_error describes the calling thread's last failure: two
    threads fail different calls, meet at a barrier, then each reads its own
    text."""
    import threading
    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, call):
        for _ in range(200):
            assert call() != OK
            barrier.wait()
            seen.setdefault(name, set()).add(_err(L))
            barrier.wait()

    t1 = threading.Thread(target=worker, args=(
        "shape", lambda: L.nvfp4_gemv(A, A, A, A, 1, 16, 48, B, None)))
    t2 = threading.Thread(target=worker, args=(
        "unsupported", lambda: L.nvfp4_gemv(A, A, A, A, 129, 16, 64, B, None)))
    t1.start(), t2.start()
    t1.join(), t2.join()
    assert len(seen["shape"]) == 1 and "K % 32" in next(iter(seen["shape"]))
    assert len(seen["unsupported"]) == 1 and "M=129" in next(iter(seen["unsupported"]))


def test_gemv_w4a4_segments_checks(L):
    """Host-side validation of the W4A4 multi-projection call (no launch)."""
    Seg = nv.GemvSegment
    arr = (Seg * 9)()
    for i in range(9):
        arr[i] = Seg(A + i * 0x100000, A + 0x10000000 + i * 0x10000, A + 0x20000000 + 16 * i,
                     B + i * 0x100000, 64)
    f = L.nvfp4_gemv_w4a4_segments
    CX, SX, GX, WS = A + 0x30000000, A + 0x31000000, A + 0x32000000, B + 0x10000000
    need = nv.gemv_w4a4_workspace_bytes(2, 64)
    assert f(arr, 9, CX, SX, GX, 2, 64, WS, need, None) == ERR_UNSUPPORTED     # > 8 segments
    assert f(arr, 2, CX, SX, GX, 129, 64, WS, need, None) == ERR_UNSUPPORTED   # M > 128
    assert f(arr, 2, CX, SX, GX, 2, 48, WS, need, None) == ERR_SHAPE           # K % 32
    assert f(arr, 0, CX, SX, GX, 2, 64, WS, need, None) == OK
    assert f(arr, 2, CX, SX, GX, 0, 64, WS, need, None) == OK
    assert f(None, 2, CX, SX, GX, 2, 64, WS, need, None) == ERR_NULL
    assert f(arr, 2, None, SX, GX, 2, 64, WS, need, None) == ERR_NULL
    assert f(arr, 2, CX + 8, SX, GX, 2, 64, WS, need, None) == ERR_ALIGN
    assert f(arr, 2, CX, SX, GX, 2, 64, WS, need - 1, None) == ERR_WORKSPACE
    assert f(arr, 2, CX, SX, GX, 2, 64, None, need, None) == ERR_WORKSPACE
    assert f(arr, 2, CX, SX, GX, 2, 64, WS + 64, need, None) == ERR_ALIGN
    bad = (Seg * 2)(arr[0], arr[1])
    bad[0].N = bad[1].N = (1 << 29) + 1
    assert f(bad, 2, CX, SX, GX, 2, 64, WS, need, None) == ERR_UNSUPPORTED
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].y = bad[0].y + 16                                    # outputs overlap
    assert f(bad, 2, CX, SX, GX, 2, 64, WS, need, None) == ERR_ALIAS
    bad = (Seg * 2)(arr[0], arr[1])
    bad[1].y = CX                                               # output on codes_x
    assert f(bad, 2, CX, SX, GX, 2, 64, WS, need, None) == ERR_ALIAS
    assert f(arr, 2, CX, SX, GX, 2, 64, arr[0].codes, need, None) == ERR_ALIAS  # workspace on W
    assert f(arr, 2, CX, SX, GX, 2, 64, arr[1].y, need, None) == ERR_ALIAS      # workspace on y


def test_stream_read_checks(L):
    """Host-side validation of the read-bandwidth measurement aid (no launch)."""
    f = L.nvfp4_stream_read
    assert f(A, 24, B, None) == ERR_SHAPE                       # bytes % 16
    assert f(A, 0, B, None) == OK                               # nothing to read
    assert f(None, 64, B, None) == ERR_NULL
    assert f(A, 64, None, None) == ERR_NULL
    assert f(A + 8, 64, B, None) == ERR_ALIGN
    assert f(A, 64, B + 2, None) == ERR_ALIGN
    assert f(A, 64, A + 32, None) == ERR_ALIAS                  # sink inside buf


def test_moe_noalloc_refuses_calls_larger_than_its_array(L):
    """nvfp4_moe_gemv_noalloc checks its size limit before touching a device:
    M * topk * I * 2 bytes of activations must fit NVFP4_NOALLOC_SCRATCH_BYTES."""
    assert nv.NOALLOC_SCRATCH_BYTES == 4 << 20
    args = [A + i * 0x10000000 for i in range(9)]
    f = L.nvfp4_moe_gemv_noalloc
    # 8 * 16 * 16416 * 2 bytes: just over 4 MiB
    assert f(*args, 8, 4, 64, 16416, 16, B, None) == ERR_UNSUPPORTED
    assert "scratch" in _err(L)
    assert f(*args, 0, 4, 64, 64, 2, B, None) == OK              # nothing to do
    assert f(*args, 1, 4, 64, 48, 2, B, None) == ERR_SHAPE       # I % 32, before any device
    assert f(*args, 9, 4, 64, 64, 2, B, None) == ERR_UNSUPPORTED
