"""CPU oracle for NVFP4 (g16) W4A16 GEMV and the MoE expert-slot variant.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's ``cpu_baseline`` leg may import this package. It shares no
code with the GPU library and never imports it.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, fp32 quantisation
decisions, fp64 dot products); this module only marshals numpy arrays.
Definitions and their sources are documented in ``nvfp4_oracle.h``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib():
    """Load the oracle library, building it first if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint]
        L.oracle_e4m3_encode.restype = ctypes.c_uint
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode.restype = ctypes.c_uint
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_pack.restype = ctypes.c_int
        L.oracle_pack.argtypes = [_f32p, _i64, _i64, _u8p, _u8p, _f32p, _f32p]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_dequant.argtypes = [_u8p, _u8p, ctypes.c_float, _i64, _i64, _f32p]
        L.oracle_gemv.restype = ctypes.c_int
        L.oracle_gemv.argtypes = [_u8p, _u8p, ctypes.c_float, _u16p, _i64, _i64,
                                  _i64, _i64p, _i64, _f64p, _f64p]
        L.oracle_moe.restype = ctypes.c_int
        L.oracle_moe.argtypes = [_u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _u16p,
                                 _i32p, _f32p, _i64, _i64, _i64, _i64, _i64,
                                 _f64p, _f64p, _u16p]
        L.oracle_moe_shared.restype = ctypes.c_int
        L.oracle_moe_shared.argtypes = [_u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _u16p,
                                        _i32p, _f32p, _i64, _i64, _i64, _i64, _i64,
                                        _u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _i64,
                                        _f64p, _f64p, _u16p, _u16p]
        L.oracle_quantize_act.restype = ctypes.c_int
        L.oracle_quantize_act.argtypes = [_u16p, _i64, _i64, ctypes.c_float, _u8p, _u8p]
        L.oracle_gemv_w4a4.restype = ctypes.c_int
        L.oracle_gemv_w4a4.argtypes = [_u8p, _u8p, ctypes.c_float, _u8p, _u8p, ctypes.c_float,
                                       _i64, _i64, _i64, _i64p, _i64, _f64p, _f64p]
        L.oracle_moe_w4a4.restype = ctypes.c_int
        L.oracle_moe_w4a4.argtypes = [_u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _u16p,
                                      _i32p, _f32p, _i64, _i64, _i64, _i64, _i64,
                                      ctypes.c_float, ctypes.c_float,
                                      _u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _i64,
                                      _u16p, _f64p, _f64p, _u16p, _u8p, _u8p]
        _lib = L
    return _lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


# ---------------------------------------------------------------- elements

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().oracle_e4m3_value(byte)


def e4m3_encode(r: float) -> int:
    return lib().oracle_e4m3_encode(float(np.float32(r)))


def e2m1_encode(t: float) -> int:
    return lib().oracle_e2m1_encode(float(np.float32(t)))


def bf16_from_double(v: float) -> int:
    return lib().oracle_bf16_from_double(float(v))


# ------------------------------------------------------------------- pack

def pack(W, gscale_override=None):
    """fp32 W[N,K] -> (codes u8[N,K/2], scales u8[N,K/16], g float32)."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 16), np.uint8)
    g = np.zeros(1, np.float32)
    ov = None
    if gscale_override is not None:
        ov = np.array([gscale_override], np.float32)
    rc = lib().oracle_pack(_ptr(W, _f32p), N, K, _ptr(codes, _u8p),
                           _ptr(scales, _u8p), _ptr(g, _f32p),
                           _ptr(ov, _f32p) if ov is not None else None)
    _check(rc, "pack")
    return codes, scales, np.float32(g[0])


def dequant(codes, scales, g):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((N, K), np.float32)
    rc = lib().oracle_dequant(_ptr(codes, _u8p), _ptr(scales, _u8p),
                              float(np.float32(g)), N, K, _ptr(out, _f32p))
    _check(rc, "dequant")
    return out


# ------------------------------------------------------------------- gemv

def gemv(codes, scales, g, x_bits, rows=None):
    """y, absdot (fp64, [M, N] or [M, len(rows)]) for bf16 x given as uint16."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x_bits = _c(x_bits, np.uint16)
    N, K = codes.shape[0], codes.shape[1] * 2
    M = x_bits.shape[0]
    if x_bits.shape[1] != K:
        raise ValueError("x has the wrong K")
    if rows is not None:
        rows = _c(np.asarray(rows, np.int64), np.int64)
        cnt = rows.shape[0]
    else:
        cnt = N
    y = np.empty((M, cnt), np.float64)
    ad = np.empty((M, cnt), np.float64)
    rc = lib().oracle_gemv(_ptr(codes, _u8p), _ptr(scales, _u8p),
                           float(np.float32(g)), _ptr(x_bits, _u16p), M, N, K,
                           _ptr(rows, _i64p) if rows is not None else None,
                           cnt, _ptr(y, _f64p), _ptr(ad, _f64p))
    _check(rc, "gemv")
    return y, ad


# -------------------------------------------------------------------- moe

def moe(w13_codes, w13_scales, w13_g, w2_codes, w2_scales, w2_g, x_bits,
        ids, gate_w, want_h=False):
    """y, bound (fp64 [M, H]) and optionally h bits (uint16 [M*topk, I])."""
    w13_codes = _c(w13_codes, np.uint8)
    w13_scales = _c(w13_scales, np.uint8)
    w2_codes = _c(w2_codes, np.uint8)
    w2_scales = _c(w2_scales, np.uint8)
    w13_g = _c(w13_g, np.float32)
    w2_g = _c(w2_g, np.float32)
    x_bits = _c(x_bits, np.uint16)
    ids = _c(ids, np.int32)
    gate_w = _c(gate_w, np.float32)
    E, twoI, Hh = w13_codes.shape
    H = Hh * 2
    I = twoI // 2
    M, topk = ids.shape
    if w2_codes.shape != (E, H, I // 2) or x_bits.shape != (M, H):
        raise ValueError("inconsistent MoE shapes")
    y = np.empty((M, H), np.float64)
    bound = np.empty((M, H), np.float64)
    h = np.empty((M * topk, I), np.uint16) if want_h else None
    rc = lib().oracle_moe(_ptr(w13_codes, _u8p), _ptr(w13_scales, _u8p),
                          _ptr(w13_g, _f32p), _ptr(w2_codes, _u8p),
                          _ptr(w2_scales, _u8p), _ptr(w2_g, _f32p),
                          _ptr(x_bits, _u16p), _ptr(ids, _i32p),
                          _ptr(gate_w, _f32p), M, E, H, I, topk,
                          _ptr(y, _f64p), _ptr(bound, _f64p),
                          _ptr(h, _u16p) if h is not None else None)
    _check(rc, "moe")
    return (y, bound, h) if want_h else (y, bound)


def moe_shared(w13_codes, w13_scales, w13_g, w2_codes, w2_scales, w2_g, x_bits,
               ids, gate_w, shared, want_h=False):
    """MoE with a shared expert: y, bound (fp64 [M, H]) and optionally the h
    bits (uint16 [M*topk, I]) and hs bits (uint16 [M, Is]). `shared` is
    (codes13 [2Is, H/2], scales13 [2Is, H/16], g13, codes2 [H, Is/2],
    scales2 [H, Is/16], g2) with g13, g2 scalars."""
    w13_codes = _c(w13_codes, np.uint8)
    w13_scales = _c(w13_scales, np.uint8)
    w2_codes = _c(w2_codes, np.uint8)
    w2_scales = _c(w2_scales, np.uint8)
    w13_g = _c(w13_g, np.float32)
    w2_g = _c(w2_g, np.float32)
    x_bits = _c(x_bits, np.uint16)
    ids = _c(ids, np.int32)
    gate_w = _c(gate_w, np.float32)
    sc13, ss13, sg13, sc2, ss2, sg2 = shared
    sc13 = _c(sc13, np.uint8)
    ss13 = _c(ss13, np.uint8)
    sc2 = _c(sc2, np.uint8)
    ss2 = _c(ss2, np.uint8)
    sg13 = _c(np.asarray(sg13, np.float32).reshape(1), np.float32)
    sg2 = _c(np.asarray(sg2, np.float32).reshape(1), np.float32)
    E, twoI, Hh = w13_codes.shape
    H = Hh * 2
    I = twoI // 2
    M, topk = ids.shape
    Is = sc13.shape[0] // 2
    if (w2_codes.shape != (E, H, I // 2) or x_bits.shape != (M, H)
            or sc13.shape != (2 * Is, H // 2) or sc2.shape != (H, Is // 2)):
        raise ValueError("inconsistent MoE shapes")
    y = np.empty((M, H), np.float64)
    bound = np.empty((M, H), np.float64)
    h = np.empty((M * topk, I), np.uint16) if want_h else None
    hs = np.empty((M, Is), np.uint16) if want_h else None
    rc = lib().oracle_moe_shared(_ptr(w13_codes, _u8p), _ptr(w13_scales, _u8p),
                                 _ptr(w13_g, _f32p), _ptr(w2_codes, _u8p),
                                 _ptr(w2_scales, _u8p), _ptr(w2_g, _f32p),
                                 _ptr(x_bits, _u16p), _ptr(ids, _i32p),
                                 _ptr(gate_w, _f32p), M, E, H, I, topk,
                                 _ptr(sc13, _u8p), _ptr(ss13, _u8p), _ptr(sg13, _f32p),
                                 _ptr(sc2, _u8p), _ptr(ss2, _u8p), _ptr(sg2, _f32p), Is,
                                 _ptr(y, _f64p), _ptr(bound, _f64p),
                                 _ptr(h, _u16p) if h is not None else None,
                                 _ptr(hs, _u16p) if hs is not None else None)
    _check(rc, "moe_shared")
    return (y, bound, h, hs) if want_h else (y, bound)


# ------------------------------------------------------------------- w4a4

def quantize_act(x_bits, g_x):
    """bf16 x [M, K] (uint16 bits) -> (codes u8[M, K/2], scales u8[M, K/16])
    with the static input scale g_x."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    rc = lib().oracle_quantize_act(_ptr(x_bits, _u16p), M, K, float(g_x),
                                   _ptr(codes, _u8p), _ptr(scales, _u8p))
    _check(rc, "quantize_act")
    return codes, scales


def gemv_w4a4(codes_w, scales_w, g_w, codes_x, scales_x, g_x, rows=None):
    """y, absdot (fp64, [M, N] or [M, len(rows)]) of the W4A4 product."""
    codes_w = _c(codes_w, np.uint8)
    scales_w = _c(scales_w, np.uint8)
    codes_x = _c(codes_x, np.uint8)
    scales_x = _c(scales_x, np.uint8)
    N, K = codes_w.shape[0], codes_w.shape[1] * 2
    M = codes_x.shape[0]
    if codes_x.shape[1] * 2 != K:
        raise ValueError("x has the wrong K")
    if rows is not None:
        rows = _c(np.asarray(rows, np.int64), np.int64)
        cnt = rows.shape[0]
    else:
        cnt = N
    y = np.empty((M, cnt), np.float64)
    ad = np.empty((M, cnt), np.float64)
    rc = lib().oracle_gemv_w4a4(_ptr(codes_w, _u8p), _ptr(scales_w, _u8p), float(g_w),
                                _ptr(codes_x, _u8p), _ptr(scales_x, _u8p), float(g_x),
                                M, N, K, _ptr(rows, _i64p) if rows is not None else None,
                                cnt, _ptr(y, _f64p), _ptr(ad, _f64p))
    _check(rc, "gemv_w4a4")
    return y, ad


def moe_w4a4(w13_codes, w13_scales, w13_g, w2_codes, w2_scales, w2_g, x_bits,
             ids, gate_w, g_a13, g_a2, shared=None, h_in=None):
    """W4A4 routed experts with static input scales g_a13 (x) and g_a2 (h),
    and an optional W4A16 shared expert (the tuple of moe_shared).
    Returns y, bound (fp64 [M, H]), h bits (uint16 [M*topk, I], computed
    here), and the quantized h: codes (uint8 [M*topk, I/2]) and scales
    (uint8 [M*topk, I/16]) of h_in if given, else of h."""
    w13_codes = _c(w13_codes, np.uint8)
    w13_scales = _c(w13_scales, np.uint8)
    w2_codes = _c(w2_codes, np.uint8)
    w2_scales = _c(w2_scales, np.uint8)
    w13_g = _c(w13_g, np.float32)
    w2_g = _c(w2_g, np.float32)
    x_bits = _c(x_bits, np.uint16)
    ids = _c(ids, np.int32)
    gate_w = _c(gate_w, np.float32)
    E, twoI, Hh = w13_codes.shape
    H = Hh * 2
    I = twoI // 2
    M, topk = ids.shape
    if w2_codes.shape != (E, H, I // 2) or x_bits.shape != (M, H):
        raise ValueError("inconsistent MoE shapes")
    sp = [None] * 6
    Is = 0
    if shared is not None:
        sc13, ss13, sg13, sc2, ss2, sg2 = shared
        sp = [_c(sc13, np.uint8), _c(ss13, np.uint8),
              _c(np.asarray(sg13, np.float32).reshape(1), np.float32),
              _c(sc2, np.uint8), _c(ss2, np.uint8),
              _c(np.asarray(sg2, np.float32).reshape(1), np.float32)]
        Is = sp[0].shape[0] // 2
        if sp[0].shape != (2 * Is, H // 2) or sp[3].shape != (H, Is // 2):
            raise ValueError("inconsistent shared expert shapes")
    if h_in is not None:
        h_in = _c(h_in, np.uint16)
        if h_in.shape != (M * topk, I):
            raise ValueError("h_in must be [M*topk, I]")
    y = np.empty((M, H), np.float64)
    bound = np.empty((M, H), np.float64)
    h = np.empty((M * topk, I), np.uint16)
    hc = np.empty((M * topk, I // 2), np.uint8)
    hs = np.empty((M * topk, I // 16), np.uint8)
    types = [_u8p, _u8p, _f32p, _u8p, _u8p, _f32p]
    rc = lib().oracle_moe_w4a4(_ptr(w13_codes, _u8p), _ptr(w13_scales, _u8p),
                               _ptr(w13_g, _f32p), _ptr(w2_codes, _u8p),
                               _ptr(w2_scales, _u8p), _ptr(w2_g, _f32p),
                               _ptr(x_bits, _u16p), _ptr(ids, _i32p),
                               _ptr(gate_w, _f32p), M, E, H, I, topk,
                               float(g_a13), float(g_a2),
                               *[_ptr(a, t) if a is not None else None
                                 for a, t in zip(sp, types)], Is,
                               _ptr(h_in, _u16p) if h_in is not None else None,
                               _ptr(y, _f64p), _ptr(bound, _f64p), _ptr(h, _u16p),
                               _ptr(hc, _u8p), _ptr(hs, _u8p))
    _check(rc, "moe_w4a4")
    return y, bound, h, hc, hs
