"""Algorithmic HBM bytes of one call: what the method must move, used for the
achieved-bandwidth and roofline figures.

The blueprint's card.json prices every W4A16 GEMV row at
  N*K*bits/8 + M*K*2 + M*N*2  bytes (floor_us = bytes / 249 GB/s),
with 4.5 bits per weight (a 4-bit code plus one 8-bit scale per 16 weights);
``pages_floor_us`` reproduces the printed floors. This library returns fp32
y, so its own per-call count is
  gemv_bytes = N*K/2 (codes) + N*K/16 (scales) + 4 (g) + M*K*2 (x) + M*N*4 (y).
"""
from __future__ import annotations


def gemv_bytes(M: int, N: int, K: int) -> int:
    return N * K // 2 + N * K // 16 + 4 + M * K * 2 + M * N * 4


def weight_bytes(N: int, K: int) -> int:
    return N * K // 2 + N * K // 16


def quantize_act_bytes(M: int, K: int) -> int:
    """Activation quantization: read bf16 x, write its codes and scales (the
    static scale is 4 bytes)."""
    return M * K * 2 + 4 + M * K // 2 + M * K // 16


def gemv_w4a4_bytes(M: int, N: int, K: int) -> int:
    """One W4A4 GEMV: the weight (codes, scales, g) and the NVFP4 activation
    (codes, scales, g) read once, fp32 y written."""
    return weight_bytes(N, K) + 4 + M * K // 2 + M * K // 16 + 4 + M * N * 4


def moe_bytes(M: int, H: int, I: int, topk: int, distinct: int) -> int:
    """One MoE call: every distinct expert's gate|up [2I, H] and down [H, I]
    weights plus its two tensor scales, x, ids and gate weights, the bf16
    SwiGLU activations h[M*topk, I] (written once, read once) and y."""
    S = M * topk
    per_expert = weight_bytes(2 * I, H) + weight_bytes(H, I) + 8
    return distinct * per_expert + M * H * 2 + S * 8 + 2 * S * I * 2 + M * H * 4


def moe_shared_bytes(M: int, H: int, I: int, topk: int, distinct: int, Is: int) -> int:
    """moe_bytes plus the shared expert: its gate|up [2Is, H] and down [H, Is]
    weights and two tensor scales, and its bf16 activations hs[M, Is]
    (written once, read once)."""
    shared = weight_bytes(2 * Is, H) + weight_bytes(H, Is) + 8 + 2 * M * Is * 2
    return moe_bytes(M, H, I, topk, distinct) + shared


def moe_w4a4_bytes(M: int, H: int, I: int, topk: int, distinct: int, Is: int = 0) -> int:
    """One W4A4 MoE call: moe_bytes (moe_shared_bytes with a shared expert)
    plus the two quantizations, each writing the values on the NVFP4 grid
    that the next pass reads, and the two static scales. x[M, H] is read,
    written and read again by its own pass. h[M*topk, I] is too at M >= 2; at
    M = 1 gate|up puts h on the grid as it produces it, so h is only written
    once more."""
    base = (moe_shared_bytes(M, H, I, topk, distinct, Is) if Is
            else moe_bytes(M, H, I, topk, distinct))
    h_extra = (1 if M == 1 else 2) * M * topk * I * 2
    return base + 2 * M * H * 2 + h_extra + 8


def pages_floor_us(M: float, N: int, K: int, experts: float, bits: float,
                   act_bytes_per_elem: float, out_elems: int,
                   bw_bytes_per_s: float = 249e9) -> float:
    """The blueprint's floor for one kernel row, in microseconds."""
    b = experts * N * K * bits / 8 + M * K * act_bytes_per_elem + out_elems * 2
    return b / bw_bytes_per_s * 1e6
