"""NVFP4 g16 W4A16 small-M GEMV for MI355X (gfx950): a thin Python binding.

Every function here marshals torch tensors into the C ABI declared in
``include/nvfp4_gemv.h`` and calls ``libnvfp4_gemv.so``; all computation runs
in the library's HIP kernels on the tensors' device, on the current torch
stream. PyTorch only provides device memory and streams. There is no CPU
fallback: if the library is not built, every call raises.

Functions (same names as the C entry points, without the prefix):
  pack(W[, gscale_override])             -> codes, scales, gscale
  dequant(codes, scales, gscale)         -> W_hat (fp32)
  gemv(codes, scales, gscale, x)         -> y (fp32 [M, N])
  gemv_segments([(codes, scales, gscale), ...], x) -> [y_s] (one launch)
  quantize_act(x, gscale_x)              -> codes_x, scales_x (static input scale)
  gemv_w4a4(codes, scales, gscale, codes_x, scales_x, gscale_x) -> y (fp32)
  moe_workspace_bytes(M, H, I, topk)     -> int
  moe_gemv(w13..., w2..., x, ids, gate_w[, workspace]) -> y (fp32 [M, H])
  moe_shared_workspace_bytes(M, H, I, topk, I_shared) -> int
  moe_shared_gemv(w13..., w2..., x, ids, gate_w, shared[, workspace]) -> y
  moe_gemv_noalloc_into(w13..., w2..., x, ids, gate_w, y)  (no workspace)
  stream_read(buf, sink)                 (measurement aid: one pure read of buf)
The ``*_into`` variants write into caller-provided outputs.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import traffic  # noqa: F401  (algorithmic byte model, pure Python)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_gemv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "nvfp4_gemv.h")

# The size limits of include/nvfp4_gemv.h (NVFP4_MAX_M, NVFP4_MOE_MAX_M,
# NVFP4_MAX_TOPK, NVFP4_MAX_N, NVFP4_MAX_K, NVFP4_MOE_MAX_I, NVFP4_MOE_MAX_H).
MAX_M = 128
MOE_MAX_M = 8
MAX_TOPK = 16
MAX_N = 1 << 30
MAX_K = 1 << 20
MOE_MAX_I = 1 << 24
MOE_MAX_H = 1 << 24
# NVFP4_NOALLOC_SCRATCH_BYTES: the device array of nvfp4_moe_gemv_noalloc.
NOALLOC_SCRATCH_BYTES = 4 << 20

_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status


class GemvSegment(ctypes.Structure):
    """nvfp4_gemv_segment: one matrix of a fused multi-projection GEMV."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64)]


MAX_SEGMENTS = 8


class MoeShared(ctypes.Structure):
    """nvfp4_moe_shared: the shared expert of a MoE call."""
    _fields_ = [("w13_codes", ctypes.c_void_p), ("w13_scales", ctypes.c_void_p),
                ("w13_gscale", ctypes.c_void_p), ("w2_codes", ctypes.c_void_p),
                ("w2_scales", ctypes.c_void_p), ("w2_gscale", ctypes.c_void_p),
                ("I", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run "
                "`python -m nvfp4_block_scaled_gemv_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        L.nvfp4_abi_version.restype = ctypes.c_int
        L.nvfp4_abi_version.argtypes = []
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_status_string.argtypes = [ctypes.c_int]
        L.nvfp4_last_error.restype = ctypes.c_char_p
        L.nvfp4_last_error.argtypes = []
        L.nvfp4_pack.restype = ctypes.c_int
        L.nvfp4_pack.argtypes = [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP]
        L.nvfp4_dequant.restype = ctypes.c_int
        L.nvfp4_dequant.argtypes = [_VP, _VP, _VP, _I64, _I64, _VP, _VP]
        L.nvfp4_gemv.restype = ctypes.c_int
        L.nvfp4_gemv.argtypes = [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _VP, _VP]
        L.nvfp4_gemv_segments.restype = ctypes.c_int
        L.nvfp4_gemv_segments.argtypes = [ctypes.POINTER(GemvSegment), _I64, _VP, _I64, _I64,
                                          _VP]
        L.nvfp4_quantize_act.restype = ctypes.c_int
        L.nvfp4_quantize_act.argtypes = [_VP, _I64, _I64, _VP, _VP, _VP, _VP]
        L.nvfp4_gemv_w4a4_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_gemv_w4a4_workspace_bytes.argtypes = [_I64, _I64]
        L.nvfp4_gemv_w4a4.restype = ctypes.c_int
        L.nvfp4_gemv_w4a4.argtypes = [_VP] * 6 + [_I64] * 3 + [_VP, _VP, ctypes.c_size_t, _VP]
        L.nvfp4_gemv_w4a4_segments.restype = ctypes.c_int
        L.nvfp4_gemv_w4a4_segments.argtypes = [ctypes.POINTER(GemvSegment), _I64, _VP, _VP, _VP,
                                               _I64, _I64, _VP, ctypes.c_size_t, _VP]
        L.nvfp4_moe_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_moe_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64]
        L.nvfp4_moe_gemv.restype = ctypes.c_int
        L.nvfp4_moe_gemv.argtypes = [_VP] * 9 + [_I64] * 5 + [_VP, _VP, ctypes.c_size_t, _VP]
        L.nvfp4_moe_shared_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_moe_shared_workspace_bytes.argtypes = [_I64] * 5
        L.nvfp4_moe_shared_gemv.restype = ctypes.c_int
        L.nvfp4_moe_shared_gemv.argtypes = ([_VP] * 9 + [_I64] * 5 +
                                            [ctypes.POINTER(MoeShared), _VP, _VP,
                                             ctypes.c_size_t, _VP])
        L.nvfp4_moe_w4a4_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_moe_w4a4_workspace_bytes.argtypes = [_I64] * 5
        L.nvfp4_moe_w4a4_gemv.restype = ctypes.c_int
        L.nvfp4_moe_w4a4_gemv.argtypes = ([_VP] * 11 + [_I64] * 5 +
                                          [ctypes.POINTER(MoeShared), _VP, _VP,
                                           ctypes.c_size_t, _VP])
        L.nvfp4_moe_gemv_noalloc.restype = ctypes.c_int
        L.nvfp4_moe_gemv_noalloc.argtypes = [_VP] * 9 + [_I64] * 5 + [_VP, _VP]
        L.nvfp4_stream_read.restype = ctypes.c_int
        L.nvfp4_stream_read.argtypes = [_VP, ctypes.c_size_t, _VP, _VP]
        L.nvfp4_check_device_faults.restype = ctypes.c_int
        L.nvfp4_check_device_faults.argtypes = [_VP]
        L.nvfp4_debug_set_wait_limit.restype = None
        L.nvfp4_debug_set_wait_limit.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = lib()
        detail = (L.nvfp4_last_error() or b"").decode() or \
            L.nvfp4_status_string(status).decode()
        raise Nvfp4Error(fn, status, detail)


# The current stream's raw handle for a device index: torch's own accessor
# when it has one (about 0.06 us a call, against about 1.8 us for building a
# Stream object through torch.cuda.current_stream).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _p(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(*ts):
    d = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if d is None:
            d = t.device
        elif t.device != d:
            raise ValueError("tensors must be on one device")
    return d


def _dtype(t, *dts, name="tensor"):
    if t.dtype not in dts:
        raise TypeError(f"{name} must be one of {dts}, got {t.dtype}")


# ------------------------------------------------------------------ pack

def pack_into(W, codes, scales, gscale, gscale_override=None) -> None:
    _dev(W, codes, scales, gscale, gscale_override)
    _dtype(W, torch.float32, name="W")
    N, K = W.shape
    _check("nvfp4_pack", lib().nvfp4_pack(_p(W), N, K, _p(codes), _p(scales), _p(gscale),
                                          _p(gscale_override), _stream(W)))


def pack(W: torch.Tensor, gscale_override: torch.Tensor | None = None):
    """fp32 W[N, K] -> (codes u8[N, K/2], scales u8[N, K/16], gscale f32[1])."""
    N, K = W.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=W.device)
    gscale = torch.empty((1,), dtype=torch.float32, device=W.device)
    pack_into(W, codes, scales, gscale, gscale_override)
    return codes, scales, gscale


# --------------------------------------------------------------- dequant

def dequant_into(codes, scales, gscale, out) -> None:
    _dev(codes, scales, gscale, out)
    N, K = codes.shape[0], codes.shape[1] * 2
    _check("nvfp4_dequant", lib().nvfp4_dequant(_p(codes), _p(scales), _p(gscale), N, K,
                                                _p(out), _stream(codes)))


def dequant(codes, scales, gscale) -> torch.Tensor:
    N, K = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((N, K), dtype=torch.float32, device=codes.device)
    dequant_into(codes, scales, gscale, out)
    return out


# ----------------------------------------------------------- measurement

def stream_read(buf: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None) -> None:
    """Read the first `nbytes` (default: all) bytes of `buf` once on the
    device (the read-bandwidth ceiling of the benchmark); `sink` is a
    uint32/int32 [1] device tensor that keeps the loads alive."""
    _dev(buf, sink)
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _check("nvfp4_stream_read", lib().nvfp4_stream_read(_p(buf), n, _p(sink), _stream(buf)))


# ------------------------------------------------------------ diagnostics

def check_device_faults(stream=None) -> None:
    """Wait for `stream` (default: torch's current stream) and raise if a
    kernel gave up a bounded internal wait since the last check (the fault
    word is cleared by the read)."""
    s = torch.cuda.current_stream() if stream is None else stream
    _check("nvfp4_check_device_faults", lib().nvfp4_check_device_faults(s.cuda_stream))


def debug_set_wait_limit(polls: int) -> None:
    """Test hook: polls before the split-K slot wait gives up (0: default,
    negative: give up at once)."""
    lib().nvfp4_debug_set_wait_limit(int(polls))


# ------------------------------------------------------------------ gemv

def gemv_into(codes, scales, gscale, x, y) -> None:
    """y[M, N] (fp32) = g * decode(W) . x^T for bf16 x[M, K]."""
    _dev(codes, scales, gscale, x, y)
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    _dtype(y, torch.float32, name="y")
    N, K = codes.shape[0], codes.shape[1] * 2
    M = x.shape[0]
    if x.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: codes {tuple(codes.shape)}, x {tuple(x.shape)}, "
                         f"y {tuple(y.shape)}")
    _check("nvfp4_gemv", lib().nvfp4_gemv(_p(codes), _p(scales), _p(gscale), _p(x), M, N, K,
                                          _p(y), _stream(codes)))


def gemv(codes, scales, gscale, x) -> torch.Tensor:
    y = torch.empty((x.shape[0], codes.shape[0]), dtype=torch.float32, device=codes.device)
    gemv_into(codes, scales, gscale, x, y)
    return y


def gemv_segments_into(mats, x, ys) -> None:
    """One launch for several matrices reading the same x[M, K]:
    ys[s] = g_s * decode(W_s) . x^T, mats[s] = (codes, scales, gscale)."""
    if len(mats) != len(ys):
        raise ValueError("one output per matrix")
    if len(mats) > MAX_SEGMENTS:
        raise ValueError(f"at most {MAX_SEGMENTS} matrices per launch")
    _dev(x, *ys, *[t for m in mats for t in m])
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    M, K = x.shape
    segs = (GemvSegment * max(1, len(mats)))()
    for i, ((c, sc, g), y) in enumerate(zip(mats, ys)):
        _dtype(y, torch.float32, name="y")
        N = c.shape[0]
        if c.shape[1] * 2 != K or tuple(y.shape) != (M, N):
            raise ValueError(f"segment {i}: codes {tuple(c.shape)}, x {tuple(x.shape)}, "
                             f"y {tuple(y.shape)}")
        segs[i] = GemvSegment(_p(c), _p(sc), _p(g), _p(y), N)
    _check("nvfp4_gemv_segments",
           lib().nvfp4_gemv_segments(segs, len(mats), _p(x), M, K, _stream(x)))


def gemv_segments(mats, x):
    """[y_s] for mats = [(codes, scales, gscale), ...] sharing x (one launch)."""
    ys = [torch.empty((x.shape[0], c.shape[0]), dtype=torch.float32, device=x.device)
          for c, _, _ in mats]
    gemv_segments_into(mats, x, ys)
    return ys


# ------------------------------------------------------------------ w4a4

def quantize_act_into(x, gscale_x, codes_x, scales_x) -> None:
    """bf16 x[M, K] -> NVFP4 codes_x u8[M, K/2], scales_x u8[M, K/16] with the
    static input scale gscale_x (fp32 [1])."""
    _dev(x, gscale_x, codes_x, scales_x)
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    M, K = x.shape
    if tuple(codes_x.shape) != (M, K // 2) or tuple(scales_x.shape) != (M, K // 16):
        raise ValueError("codes_x / scales_x have the wrong shape")
    _check("nvfp4_quantize_act", lib().nvfp4_quantize_act(
        _p(x), M, K, _p(gscale_x), _p(codes_x), _p(scales_x), _stream(x)))


def quantize_act(x, gscale_x):
    M, K = x.shape
    codes_x = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales_x = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    quantize_act_into(x, gscale_x, codes_x, scales_x)
    return codes_x, scales_x


def gemv_w4a4_workspace_bytes(M: int, K: int) -> int:
    return int(lib().nvfp4_gemv_w4a4_workspace_bytes(M, K))


def gemv_w4a4_into(codes, scales, gscale, codes_x, scales_x, gscale_x, y, workspace) -> None:
    """y[M, N] (fp32) = g_w g_x decode(W) . decode(x)^T, both NVFP4 g16."""
    _dev(codes, scales, gscale, codes_x, scales_x, gscale_x, y, workspace)
    _dtype(y, torch.float32, name="y")
    N, K = codes.shape[0], codes.shape[1] * 2
    M = codes_x.shape[0]
    if codes_x.shape[1] * 2 != K or tuple(scales_x.shape) != (M, K // 16) \
            or tuple(y.shape) != (M, N):
        raise ValueError(f"shape mismatch: codes {tuple(codes.shape)}, codes_x "
                         f"{tuple(codes_x.shape)}, y {tuple(y.shape)}")
    _check("nvfp4_gemv_w4a4", lib().nvfp4_gemv_w4a4(
        _p(codes), _p(scales), _p(gscale), _p(codes_x), _p(scales_x), _p(gscale_x), M, N, K,
        _p(y), _p(workspace), workspace.numel() * workspace.element_size(), _stream(codes)))


def gemv_w4a4(codes, scales, gscale, codes_x, scales_x, gscale_x,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    M, K = codes_x.shape[0], codes_x.shape[1] * 2
    if workspace is None:
        workspace = torch.empty(max(gemv_w4a4_workspace_bytes(M, K), 256), dtype=torch.uint8,
                                device=codes.device)
    y = torch.empty((M, codes.shape[0]), dtype=torch.float32, device=codes.device)
    gemv_w4a4_into(codes, scales, gscale, codes_x, scales_x, gscale_x, y, workspace)
    return y


def gemv_w4a4_segments_into(mats, codes_x, scales_x, gscale_x, ys, workspace) -> None:
    """One launch (two at M >= 3) for several weight matrices on the same
    NVFP4 activations: ys[s] = g_s g_x decode(W_s) . decode(x)^T,
    mats[s] = (codes, scales, gscale)."""
    if len(mats) != len(ys):
        raise ValueError("one output per matrix")
    if len(mats) > MAX_SEGMENTS:
        raise ValueError(f"at most {MAX_SEGMENTS} matrices per launch")
    _dev(codes_x, scales_x, gscale_x, workspace, *ys, *[t for m in mats for t in m])
    M, K = codes_x.shape[0], codes_x.shape[1] * 2
    segs = (GemvSegment * max(1, len(mats)))()
    for i, ((c, sc, g), y) in enumerate(zip(mats, ys)):
        _dtype(y, torch.float32, name="y")
        N = c.shape[0]
        if c.shape[1] * 2 != K or tuple(y.shape) != (M, N):
            raise ValueError(f"segment {i}: codes {tuple(c.shape)}, codes_x "
                             f"{tuple(codes_x.shape)}, y {tuple(y.shape)}")
        segs[i] = GemvSegment(_p(c), _p(sc), _p(g), _p(y), N)
    _check("nvfp4_gemv_w4a4_segments", lib().nvfp4_gemv_w4a4_segments(
        segs, len(mats), _p(codes_x), _p(scales_x), _p(gscale_x), M, K, _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(codes_x)))


def gemv_w4a4_segments(mats, codes_x, scales_x, gscale_x, workspace=None):
    """[y_s] for mats = [(codes, scales, gscale), ...] on the same NVFP4 x."""
    M, K = codes_x.shape[0], codes_x.shape[1] * 2
    if workspace is None:
        workspace = torch.empty(max(gemv_w4a4_workspace_bytes(M, K), 256), dtype=torch.uint8,
                                device=codes_x.device)
    ys = [torch.empty((M, c.shape[0]), dtype=torch.float32, device=codes_x.device)
          for c, _, _ in mats]
    gemv_w4a4_segments_into(mats, codes_x, scales_x, gscale_x, ys, workspace)
    return ys


# ------------------------------------------------------------------- moe

def moe_workspace_bytes(M: int, H: int, I: int, topk: int) -> int:
    return int(lib().nvfp4_moe_workspace_bytes(M, H, I, topk))


def moe_gemv_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale,
                  x, expert_ids, gate_w, y, workspace) -> None:
    _dev(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
         expert_ids, gate_w, y, workspace)
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    _dtype(expert_ids, torch.int32, name="expert_ids")
    _dtype(gate_w, torch.float32, name="gate_w")
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    if tuple(w2_codes.shape) != (E, H, I // 2) or tuple(x.shape) != (M, H) \
            or tuple(gate_w.shape) != (M, topk) or tuple(y.shape) != (M, H):
        raise ValueError("inconsistent MoE shapes")
    _check("nvfp4_moe_gemv", lib().nvfp4_moe_gemv(
        _p(w13_codes), _p(w13_scales), _p(w13_gscale), _p(w2_codes), _p(w2_scales),
        _p(w2_gscale), _p(x), _p(expert_ids), _p(gate_w), M, E, H, I, topk, _p(y),
        _p(workspace), workspace.numel() * workspace.element_size(), _stream(x)))


def moe_gemv(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
             expert_ids, gate_w, workspace: torch.Tensor | None = None) -> torch.Tensor:
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    if workspace is None:
        workspace = torch.empty(max(moe_workspace_bytes(M, H, I, topk), 256),
                                dtype=torch.uint8, device=x.device)
    y = torch.empty((M, H), dtype=torch.float32, device=x.device)
    moe_gemv_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
                  expert_ids, gate_w, y, workspace)
    return y


def moe_gemv_noalloc_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale,
                          x, expert_ids, gate_w, y) -> None:
    """moe_gemv_into without a workspace: the library's own device array
    holds the SwiGLU activations (calls on one device must not overlap)."""
    _dev(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
         expert_ids, gate_w, y)
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    _dtype(expert_ids, torch.int32, name="expert_ids")
    _dtype(gate_w, torch.float32, name="gate_w")
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    if tuple(w2_codes.shape) != (E, H, I // 2) or tuple(x.shape) != (M, H) \
            or tuple(gate_w.shape) != (M, topk) or tuple(y.shape) != (M, H):
        raise ValueError("inconsistent MoE shapes")
    _check("nvfp4_moe_gemv_noalloc", lib().nvfp4_moe_gemv_noalloc(
        _p(w13_codes), _p(w13_scales), _p(w13_gscale), _p(w2_codes), _p(w2_scales),
        _p(w2_gscale), _p(x), _p(expert_ids), _p(gate_w), M, E, H, I, topk, _p(y),
        _stream(x)))


def moe_workspace_layout(M: int, H: int, I: int, topk: int) -> dict:
    """Byte offsets inside the MoE workspace (for inspecting the bf16 SwiGLU
    activations h[M*topk, I] after a call)."""
    S = M * topk
    return {"h": 0, "total": (S * I * 2 + 255) & ~255}


def moe_shared_workspace_bytes(M: int, H: int, I: int, topk: int, I_shared: int) -> int:
    return int(lib().nvfp4_moe_shared_workspace_bytes(M, H, I, topk, I_shared))


def moe_shared_gemv_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale,
                         x, expert_ids, gate_w, shared, y, workspace) -> None:
    """`shared` = (codes13 [2Is, H/2], scales13 [2Is, H/16], gscale13 [1],
    codes2 [H, Is/2], scales2 [H, Is/16], gscale2 [1]) device tensors."""
    sc13, ss13, sg13, sc2, ss2, sg2 = shared
    _dev(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
         expert_ids, gate_w, y, workspace, sc13, ss13, sg13, sc2, ss2, sg2)
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    _dtype(expert_ids, torch.int32, name="expert_ids")
    _dtype(gate_w, torch.float32, name="gate_w")
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    Is = sc13.shape[0] // 2
    if tuple(w2_codes.shape) != (E, H, I // 2) or tuple(x.shape) != (M, H) \
            or tuple(gate_w.shape) != (M, topk) or tuple(y.shape) != (M, H) \
            or tuple(sc13.shape) != (2 * Is, H // 2) or tuple(sc2.shape) != (H, Is // 2):
        raise ValueError("inconsistent MoE shapes")
    sh = MoeShared(_p(sc13), _p(ss13), _p(sg13), _p(sc2), _p(ss2), _p(sg2), Is)
    _check("nvfp4_moe_shared_gemv", lib().nvfp4_moe_shared_gemv(
        _p(w13_codes), _p(w13_scales), _p(w13_gscale), _p(w2_codes), _p(w2_scales),
        _p(w2_gscale), _p(x), _p(expert_ids), _p(gate_w), M, E, H, I, topk, ctypes.byref(sh),
        _p(y), _p(workspace), workspace.numel() * workspace.element_size(), _stream(x)))


def moe_shared_gemv(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
                    expert_ids, gate_w, shared,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    Is = shared[0].shape[0] // 2
    if workspace is None:
        workspace = torch.empty(max(moe_shared_workspace_bytes(M, H, I, topk, Is), 256),
                                dtype=torch.uint8, device=x.device)
    y = torch.empty((M, H), dtype=torch.float32, device=x.device)
    moe_shared_gemv_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
                         expert_ids, gate_w, shared, y, workspace)
    return y


def moe_shared_workspace_layout(M: int, H: int, I: int, topk: int, I_shared: int) -> dict:
    """Byte offsets inside the workspace of nvfp4_moe_shared_gemv: the routed
    h[M*topk, I] and the shared hs[M, I_shared] bf16 activations."""
    hs = (M * topk * I * 2 + 255) & ~255
    return {"h": 0, "hs": hs, "total": (hs + M * I_shared * 2 + 255) & ~255}


def moe_w4a4_workspace_bytes(M: int, H: int, I: int, topk: int, I_shared: int = 0) -> int:
    return int(lib().nvfp4_moe_w4a4_workspace_bytes(M, H, I, topk, I_shared))


def moe_w4a4_gemv_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale,
                       x, gscale_x, gscale_h, expert_ids, gate_w, y, workspace,
                       shared=None) -> None:
    """W4A4 routed experts (static input scales gscale_x for x and gscale_h
    for h, fp32 [1] device tensors) and an optional W4A16 shared expert
    (the tuple of moe_shared_gemv_into)."""
    extra = list(shared) if shared is not None else []
    _dev(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x, gscale_x,
         gscale_h, expert_ids, gate_w, y, workspace, *extra)
    _dtype(x, torch.bfloat16, torch.int16, torch.uint16, name="x")
    _dtype(expert_ids, torch.int32, name="expert_ids")
    _dtype(gate_w, torch.float32, name="gate_w")
    _dtype(gscale_x, torch.float32, name="gscale_x")
    _dtype(gscale_h, torch.float32, name="gscale_h")
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    if tuple(w2_codes.shape) != (E, H, I // 2) or tuple(x.shape) != (M, H) \
            or tuple(gate_w.shape) != (M, topk) or tuple(y.shape) != (M, H):
        raise ValueError("inconsistent MoE shapes")
    sh = None
    if shared is not None:
        sc13, ss13, sg13, sc2, ss2, sg2 = shared
        Is = sc13.shape[0] // 2
        if tuple(sc13.shape) != (2 * Is, H // 2) or tuple(sc2.shape) != (H, Is // 2):
            raise ValueError("inconsistent shared expert shapes")
        sh = MoeShared(_p(sc13), _p(ss13), _p(sg13), _p(sc2), _p(ss2), _p(sg2), Is)
    _check("nvfp4_moe_w4a4_gemv", lib().nvfp4_moe_w4a4_gemv(
        _p(w13_codes), _p(w13_scales), _p(w13_gscale), _p(w2_codes), _p(w2_scales),
        _p(w2_gscale), _p(x), _p(gscale_x), _p(gscale_h), _p(expert_ids), _p(gate_w),
        M, E, H, I, topk, ctypes.byref(sh) if sh is not None else None,
        _p(y), _p(workspace), workspace.numel() * workspace.element_size(), _stream(x)))


def moe_w4a4_gemv(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
                  gscale_x, gscale_h, expert_ids, gate_w, shared=None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    E, twoI, Hh = w13_codes.shape
    H, I = Hh * 2, twoI // 2
    M, topk = expert_ids.shape
    Is = shared[0].shape[0] // 2 if shared is not None else 0
    if workspace is None:
        workspace = torch.empty(max(moe_w4a4_workspace_bytes(M, H, I, topk, Is), 256),
                                dtype=torch.uint8, device=x.device)
    y = torch.empty((M, H), dtype=torch.float32, device=x.device)
    moe_w4a4_gemv_into(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
                       gscale_x, gscale_h, expert_ids, gate_w, y, workspace, shared=shared)
    return y


def moe_w4a4_workspace_layout(M: int, H: int, I: int, topk: int, I_shared: int = 0) -> dict:
    """Byte offsets inside the workspace of nvfp4_moe_w4a4_gemv: h[M*topk, I]
    (bf16 SwiGLU output), hs[M, I_shared], and h and x on the NVFP4 grid
    (bf16 e2m1 * s): hq[M*topk, I], xq[M, H]."""
    def a(v):
        return (v + 255) & ~255
    hs = a(M * topk * I * 2)
    hq = a(hs + M * I_shared * 2)
    xq = a(hq + M * topk * I * 2)
    return {"h": 0, "hs": hs, "hq": hq, "xq": xq, "total": a(xq + M * H * 2)}
