"""Seeded synthetic inputs for the NVFP4 W4A16 GEMV and MoE workloads.

This module is shared by the tests, the benchmark and the oracle checks. It
holds no arithmetic of the method itself: it only draws fp32 weights, bf16
activations, expert ids and gate weights from seeded numpy streams. The
quantisation (pack), the GEMV and the MoE combine live elsewhere.

Stream layout: every array comes from ``np.random.SeedSequence([workload,
rep, stream, chunk])``. Large weight matrices are filled in chunks of
``ROWS_PER_CHUNK`` rows, one stream per chunk, so that any chunk can be
regenerated on its own and the result does not depend on the thread count.

Workload shapes (N x K = output rows x input columns, the ggml ``{K, N}``
convention of the llama.cpp trace page):

1. single GEMV, M=1, 1024 x 4096, W ~ N(0, 0.02);
2. dense decode layer at M=5: q, o 4096 x 4096; k, v 1024 x 4096;
   gate, up 12288 x 4096; down 4096 x 12288 (the MUL_MAT rows of the
   llama.cpp trace page at 5 tokens), W ~ N(0, 0.02);
3. LM-head GEMV, M=1, 151936 x 4096 (the trace page's output.weight);
4. MoE expert slots: 288 experts, hidden 4096, gate|up 3072 x 4096 and
   down 4096 x 1536 per expert, top-8 ids per token drawn uniformly without
   replacement, gate weights = softmax of N(0,1) logits over the 8 chosen
   slots; M = 1 and M = 8;
5. stress GEMV at M=8 on 12288 x 4096 and 4096 x 12288 with W = 0.02 * t_3
   (Student-t, nu = 3) and exactly round(1% of all 16-element blocks)
   zeroed, chosen uniformly without replacement.
x is bf16 N(0, 1): a float32 N(0,1) draw rounded to bf16 by torch's
round-to-nearest-even conversion.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROWS_PER_CHUNK = 1024
_STREAM_X = 1 << 20          # stream ids at or above this are activations
_STREAM_ROUTING = 1 << 21    # expert ids and gate weights
_STREAM_ZERO_BLOCKS = 1 << 22


def rng(workload: int, rep: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([workload, rep, stream, chunk])))


def _threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    try:
        n = int(n) if n else (os.cpu_count() or 1)
    except ValueError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _fill_chunks(N: int, K: int, fill, threads: int | None = None) -> np.ndarray:
    out = np.empty((N, K), np.float32)
    chunks = [(c, c * ROWS_PER_CHUNK, min(N, (c + 1) * ROWS_PER_CHUNK))
              for c in range((N + ROWS_PER_CHUNK - 1) // ROWS_PER_CHUNK)]

    def run(item):
        c, r0, r1 = item
        fill(c, out[r0:r1])

    t = threads or _threads()
    if t <= 1 or len(chunks) <= 1:
        for item in chunks:
            run(item)
    else:
        with ThreadPoolExecutor(max_workers=t) as ex:
            list(ex.map(run, chunks))
    return out


def normal_weights(workload: int, rep: int, stream: int, N: int, K: int,
                   std: float = 0.02, threads: int | None = None) -> np.ndarray:
    """fp32 W[N, K] ~ N(0, std^2), chunked streams."""
    def fill(c, view):
        g = rng(workload, rep, stream, c)
        g.standard_normal(out=view, dtype=np.float32)
        view *= np.float32(std)
    return _fill_chunks(N, K, fill, threads)


def student_t_weights(workload: int, rep: int, stream: int, N: int, K: int,
                      nu: float = 3.0, scale: float = 0.02,
                      zero_block_frac: float = 0.01,
                      threads: int | None = None) -> np.ndarray:
    """fp32 W[N, K] = scale * t_nu, with round(zero_block_frac * N*K/16)
    16-element blocks (along K) set to zero, chosen without replacement."""
    def fill(c, view):
        g = rng(workload, rep, stream, c)
        view[...] = (scale * g.standard_t(nu, size=view.shape)).astype(np.float32)
    W = _fill_chunks(N, K, fill, threads)
    nblocks = N * (K // 16)
    nzero = int(round(zero_block_frac * nblocks))
    if nzero:
        g = rng(workload, rep, _STREAM_ZERO_BLOCKS + stream)
        pick = g.choice(nblocks, size=nzero, replace=False)
        Wb = W.reshape(nblocks, 16)
        Wb[pick] = 0.0
    return W


def zero_block_ids(workload: int, rep: int, stream: int, N: int, K: int,
                   zero_block_frac: float = 0.01) -> np.ndarray:
    """The block indices (row-major over [N, K/16]) that student_t_weights zeroes."""
    nblocks = N * (K // 16)
    nzero = int(round(zero_block_frac * nblocks))
    g = rng(workload, rep, _STREAM_ZERO_BLOCKS + stream)
    return np.sort(g.choice(nblocks, size=nzero, replace=False))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (torch's round-to-nearest-even) and return the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def x_bf16(workload: int, rep: int, stream: int, M: int, K: int) -> np.ndarray:
    """bf16 x[M, K] ~ N(0, 1) as uint16 bit patterns."""
    g = rng(workload, rep, _STREAM_X + stream)
    return bf16_bits_from_f32(g.standard_normal((M, K), dtype=np.float32))


def moe_routing(workload: int, rep: int, M: int, E: int, topk: int):
    """ids int32[M, topk] (distinct per token, uniform) and gate_w f32[M, topk]
    (softmax of N(0,1) logits over the chosen slots)."""
    g = rng(workload, rep, _STREAM_ROUTING)
    ids = np.stack([g.choice(E, size=topk, replace=False) for _ in range(M)])
    z = g.standard_normal((M, topk))
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), p.astype(np.float32)


# ------------------------------------------------------------- workloads

# The dense decode layer's seven linears at 5 tokens: (name, N, K).
DECODE_LAYER = [
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 12288, 4096),
    ("up", 12288, 4096),
    ("down", 4096, 12288),
]

WORKLOADS = {
    1: dict(name="gemv_m1_1024x4096", M=1, mats=[("w", 1024, 4096)], dist="normal"),
    2: dict(name="decode_layer_m5", M=5, mats=DECODE_LAYER, dist="normal"),
    3: dict(name="lm_head_m1_151936x4096", M=1, mats=[("head", 151936, 4096)],
            dist="normal"),
    4: dict(name="moe_288x(3072x4096,4096x1536)_top8", E=288, H=4096, I=1536,
            topk=8, Ms=(1, 8), dist="normal"),
    5: dict(name="stress_m8_t3", M=8, mats=[("a", 12288, 4096), ("b", 4096, 12288)],
            dist="student_t"),
    # the pages' W4A4 dense FFN (card.json performance[20], [24]: "dense FFN
    # gate/up/down M=2 N=4096 K=4096", NVFP4 x NVFP4 with a static input scale)
    6: dict(name="w4a4_ffn_m2", M=2,
            mats=[("gate", 4096, 4096), ("up", 4096, 4096), ("down", 4096, 4096)],
            dist="normal"),
}


def dense_weights(workload: int, rep: int, stream: int, N: int, K: int,
                  threads: int | None = None) -> np.ndarray:
    """The fp32 weight matrix `stream` of a dense workload."""
    if WORKLOADS[workload]["dist"] == "student_t":
        return student_t_weights(workload, rep, stream, N, K, threads=threads)
    return normal_weights(workload, rep, stream, N, K, threads=threads)


def moe_expert_weights(workload: int, rep: int, e: int, H: int, I: int,
                       threads: int | None = None):
    """fp32 (W13[2I, H], W2[H, I]) of expert e, each from its own stream."""
    w13 = normal_weights(workload, rep, 2 * e, 2 * I, H, threads=threads)
    w2 = normal_weights(workload, rep, 2 * e + 1, H, I, threads=threads)
    return w13, w2


def moe_shared_weights(workload: int, rep: int, H: int, Is: int,
                       threads: int | None = None):
    """fp32 (WS13[2 Is, H], WS2[H, Is]) of the shared expert, N(0, 0.02), each
    from its own stream (apart from every routed expert's)."""
    w13 = normal_weights(workload, rep, 1 << 22, 2 * Is, H, threads=threads)
    w2 = normal_weights(workload, rep, (1 << 22) + 1, H, Is, threads=threads)
    return w13, w2


def random_nvfp4(workload: int, rep: int, stream: int, N: int, K: int,
                 scale_lo: int = 0x00, scale_hi: int = 0x7E):
    """Arbitrary NVFP4 storage (not produced by a pack): uniform code bytes
    (every nibble 0..15) and uniform scale bytes in [scale_lo, scale_hi]."""
    g = rng(workload, rep, (1 << 23) + stream)
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = g.integers(scale_lo, scale_hi + 1, size=(N, K // 16), dtype=np.uint8)
    return codes, scales
