"""GPU GEMV against the oracle within |y - y_ref| <= 1e-3 sum|w x| + 1e-6:
every workload at full size (the LM head on sampled rows), ragged and edge
shapes, arbitrary codes and scales, determinism and stream use."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import nvfp4_block_scaled_gemv_amd as nv
from gpu_util import check_tol, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


def run_gpu(codes, scales, g, x_bits):
    return host(nv.gemv(dev(codes), dev(scales), dev(np.array([g], np.float32)), dev_x(x_bits)))


def packed_pair(W):
    """Oracle pack (for the oracle) and GPU pack (for the GPU), which must be
    identical byte for byte."""
    c0, s0, g0 = oracle.pack(W)
    c1, s1, g1 = nv.pack(dev(W))
    assert np.array_equal(host(c1), c0) and np.array_equal(host(s1), s0)
    assert np.float32(host(g1)[0]) == g0
    return (c0, s0, g0), (c1, s1, g1)


def test_closed_form_all_ones():
    for K in (32, 4096, 12288):
        N, M = 77, 3
        codes = np.full((N, K // 2), 0x22, np.uint8)
        scales = np.full((N, K // 16), 0x38, np.uint8)
        x = np.full((M, K), 0x3F80, np.uint16)
        y = run_gpu(codes, scales, 1.0, x)
        assert np.all(y == K), (K, y.min(), y.max())


@pytest.mark.parametrize("M", list(range(1, 9)))
@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (37, 96), (257, 2048), (1001, 2080),
                                 (130, 4096), (64, 12288)])
def test_random_storage_shapes(M, N, K):
    say(f"[gemv] random storage M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(9, M, N * 7 + K, N, K)
    x = workloads.x_bf16(9, M, N * 7 + K, M, K)
    g = np.float32(0.0123)
    y = run_gpu(codes, scales, g, x)
    y_ref, ad = oracle.gemv(codes, scales, g, x)
    check_tol(y, y_ref, ad, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N", [(1, 4097), (1, 32767), (2, 4095), (1, 1), (2, 130),
                                 (3, 1024), (4, 1), (5, 1024), (5, 1025)])
def test_staged_vector_alu_shapes(M, N):
    """K = 4096 below 32768 rows: one row group per wavefront with x staged in
    LDS, two rows per wavefront from 4096 rows and one below (M = 2 stays on
    the vector ALUs below 4096 rows, 3 <= M <= 5 up to 1024 rows; 1025 rows
    at M = 5 is the matrix cores' again); ragged last groups, the largest row
    counts and a one-row matrix, every output compared."""
    K = 4096
    say(f"[gemv] staged vector-ALU shape M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(9, M, 3 * N + 1, N, K)
    x = workloads.x_bf16(9, M, 3 * N + 1, M, K)
    g = np.float32(0.0211)
    y = run_gpu(codes, scales, g, x)
    y_ref, ad = oracle.gemv(codes, scales, g, x)
    check_tol(y, y_ref, ad, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2])
def test_four_rows_per_wavefront_with_ragged_tail(M):
    """N >= 32768 takes four rows per wavefront on the vector ALUs; N = 40003
    leaves a tail of three rows."""
    N, K = 40003, 64
    say(f"[gemv] M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(9, M, 41, N, K)
    x = workloads.x_bf16(9, M, 41, M, K)
    y = run_gpu(codes, scales, np.float32(0.02), x)
    y_ref, ad = oracle.gemv(codes, scales, np.float32(0.02), x)
    check_tol(y, y_ref, ad, f"M={M} N={N}")


@pytest.mark.parametrize("N,K", [(4095, 4096), (4096, 4096), (6001, 512), (12288, 4096),
                                 (4096, 12288), (8000, 2304)])
def test_two_tokens_on_the_matrix_cores(N, K):
    """M = 2 from 4096 rows with K % 256 == 0 runs on the matrix-core kernels
    (below that, and for other K, on the vector ALUs): both sides of the
    switch, a ragged last tile (6001 rows), tall K, and K = 2304 (9 slices)."""
    M = 2
    say(f"[gemv] two tokens N={N} K={K}")
    codes, scales = workloads.random_nvfp4(9, M, N + K, N, K)
    x = workloads.x_bf16(9, M, N + K, M, K)
    g = np.float32(0.017)
    y = run_gpu(codes, scales, g, x)
    y_ref, ad = oracle.gemv(codes, scales, g, x)
    check_tol(y, y_ref, ad, f"M=2 N={N} K={K}")


@pytest.mark.parametrize("M", [3, 6, 8])
@pytest.mark.parametrize("N,K", [(33, 256), (77, 512), (100, 768), (300, 3840), (50, 4352),
                                 (4800, 8192), (40, 30720), (21, 65536)])
def test_split_k_shapes(M, N, K):
    """The matrix-core kernel's K splits: one wavefront holding one x slice
    (K = 256) or two (K = 512), three and fifteen wavefronts holding one (odd
    slice counts), one wavefront streaming x over 17 slices (a prime slice
    count), eight wavefronts streaming four slices each with several tiles
    per workgroup (4800 rows), eight streaming fifteen (K = 30720) and
    thirty-two (K = 65536); the largest N compares a sample of rows, first
    and last included."""
    say(f"[gemv] split-K M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(9, M, N * 3 + K, N, K)
    x = workloads.x_bf16(9, M, N * 3 + K, M, K)
    g = np.float32(0.031)
    y = run_gpu(codes, scales, g, x)
    rows = None
    if N > 1000:
        rows = np.unique(np.concatenate([[0, 15, 16, N - 1],
                                         np.random.default_rng(N).choice(N, 600, replace=False)]))
    y_ref, ad = oracle.gemv(codes, scales, g, x, rows=rows)
    check_tol(y if rows is None else y[:, rows], y_ref, ad, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [3, 5, 8])
@pytest.mark.parametrize("N,K", [(49157, 2048), (12291, 4096), (6150, 2048), (100, 1024),
                                 (33, 3840), (70, 8192), (300, 12288), (50, 16384)])
def test_matrix_core_launch_shapes(M, N, K):
    """Every launch shape of the eight-token matrix-core kernel, each with a
    ragged last tile: two tiles per workgroup from 3073 tiles up, three from
    769 and two from 385 tiles (one slice per wavefront), one tile with one
    slice (4 and 15 wavefronts), two (K = 8192), three (K = 12288) and four
    (K = 16384) slices per wavefront. Large N compares a sample of rows, the
    last included."""
    say(f"[gemv] matrix-core shape M={M} N={N} K={K}")
    codes, scales = workloads.random_nvfp4(16, M, N + K, N, K)
    x = workloads.x_bf16(16, M, N + K, M, K)
    g = np.float32(0.027)
    y = run_gpu(codes, scales, g, x)
    rows = None
    if N > 2000:
        rows = np.unique(np.concatenate([[0, 15, 16, 47, 48, N - 17, N - 16, N - 1],
                                         np.random.default_rng(N).choice(N, 800, replace=False)]))
    y_ref, ad = oracle.gemv(codes, scales, g, x, rows=rows)
    check_tol(y if rows is None else y[:, rows], y_ref, ad, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_subnormal_and_max_scales(M):
    N, K = 200, 1024
    for lo, hi in [(0x00, 0x07), (0x70, 0x7E), (0x78, 0x7E)]:
        codes, scales = workloads.random_nvfp4(9, 100 + M, lo, N, K, lo, hi)
        x = workloads.x_bf16(9, 100 + M, lo, M, K)
        y = run_gpu(codes, scales, 1.0, x)
        y_ref, ad = oracle.gemv(codes, scales, 1.0, x)
        check_tol(y, y_ref, ad, f"scales {lo:#x}-{hi:#x}")


def test_workload_1_single_gemv():
    W = workloads.dense_weights(1, 0, 0, 1024, 4096)
    (c0, s0, g0), (c1, s1, g1) = packed_pair(W)
    x = workloads.x_bf16(1, 0, 0, 1, 4096)
    y = host(nv.gemv(c1, s1, g1, dev_x(x)))
    y_ref, ad = oracle.gemv(c0, s0, g0, x)
    r = check_tol(y, y_ref, ad, "workload 1")
    say(f"  max err / tol = {r:.3e}")


@pytest.mark.parametrize("i", range(len(workloads.DECODE_LAYER)))
def test_workload_2_decode_layer(i):
    name, N, K = workloads.DECODE_LAYER[i]
    say(f"[gemv] decode layer {name} {N}x{K} M=5")
    W = workloads.dense_weights(2, 0, i, N, K)
    (c0, s0, g0), (c1, s1, g1) = packed_pair(W)
    x = workloads.x_bf16(2, 0, i, 5, K)
    y = host(nv.gemv(c1, s1, g1, dev_x(x)))
    y_ref, ad = oracle.gemv(c0, s0, g0, x)
    check_tol(y, y_ref, ad, name)


@pytest.mark.parametrize("i,N,K", [(0, 12288, 4096), (1, 4096, 12288)])
def test_workload_5_stress_m8(i, N, K):
    say(f"[gemv] stress t3 {N}x{K} M=8")
    W = workloads.dense_weights(5, 0, i, N, K)
    (c0, s0, g0), (c1, s1, g1) = packed_pair(W)
    zb = workloads.zero_block_ids(5, 0, i, N, K)
    assert np.all(s0.ravel()[zb] == 0)
    x = workloads.x_bf16(5, 0, i, 8, K)
    y = host(nv.gemv(c1, s1, g1, dev_x(x)))
    y_ref, ad = oracle.gemv(c0, s0, g0, x)
    check_tol(y, y_ref, ad, f"stress {N}x{K}")


def test_workload_3_lm_head_all_rows():
    """Full 151936 x 4096 at M=1, in the launch the benchmark times, every
    output against the oracle."""
    N, K = 151936, 4096
    W = workloads.dense_weights(3, 0, 0, N, K)
    (c0, s0, g0), (c1, s1, g1) = packed_pair(W)
    del W
    x = workloads.x_bf16(3, 0, 0, 1, K)
    y = host(nv.gemv(c1, s1, g1, dev_x(x)))
    y_ref, ad = oracle.gemv(c0, s0, g0, x)
    check_tol(y, y_ref, ad, "lm head")
    assert np.all(np.isfinite(y))


def test_empty_and_zero_k():
    c = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    y = torch.full((0, 4), 7.0, device="cuda")
    nv.gemv_into(c, s, g, torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda"), y)
    # K == 0: y becomes zero
    c0 = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    s0 = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    y = torch.full((2, 5), 7.0, device="cuda")
    nv.gemv_into(c0, s0, g, torch.zeros((2, 0), dtype=torch.bfloat16, device="cuda"), y)
    assert torch.all(y == 0)
    # N == 0: nothing launched
    y = torch.empty((3, 0), device="cuda")
    nv.gemv_into(torch.zeros((0, 16), dtype=torch.uint8, device="cuda"),
                 torch.zeros((0, 2), dtype=torch.uint8, device="cuda"), g,
                 torch.zeros((3, 32), dtype=torch.bfloat16, device="cuda"), y)


def test_rejects_m129():
    c = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.gemv(c, s, torch.ones(1, device="cuda"),
                torch.zeros((129, 32), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 4


def test_deterministic_and_on_side_stream():
    N, K, M = 3000, 4096, 4
    codes, scales = workloads.random_nvfp4(9, 1, 1, N, K)
    x = workloads.x_bf16(9, 1, 1, M, K)
    cd, sd, gd, xd = dev(codes), dev(scales), dev(np.array([0.5], np.float32)), dev_x(x)
    y1 = nv.gemv(cd, sd, gd, xd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y2 = nv.gemv(cd, sd, gd, xd)
    torch.cuda.current_stream().wait_stream(side)
    assert np.array_equal(host(y1), host(y2))
    y_ref, ad = oracle.gemv(codes, scales, 0.5, x)
    check_tol(host(y2), y_ref, ad, "side stream")


def test_splitk_fault_path_is_reported_and_cleared():
    """The split-K kernel's bounded slot wait, forced to give up from the host
    (a negative wait bound: every tile gives up at once, no wait at all): the
    kernel still ends normally, its outputs are NaN, the fault is reported by
    nvfp4_check_device_faults and cleared by the read; with the default bound
    the same call is correct again and reports nothing. K = 17 slices of 256
    takes the split-K kernel (the 16-wavefront kernel cannot split 17)."""
    M, N, K = 5, 256, 256 * 17
    codes, scales = workloads.random_nvfp4(40, M, 1, N, K)
    x = workloads.x_bf16(40, M, 1, M, K)
    g = np.float32(0.02)
    args = (dev(codes), dev(scales), dev(np.array([g], np.float32)), dev_x(x))
    say("[fault] forced give-up of the split-K slot wait")
    try:
        nv.debug_set_wait_limit(-1)
        y_bad = host(nv.gemv(*args))
        with pytest.raises(nv.Nvfp4Error) as err:
            nv.check_device_faults()
        assert "slot wait" in str(err.value)
        assert np.isnan(y_bad).all()
        nv.check_device_faults()   # cleared by the first read
    finally:
        nv.debug_set_wait_limit(0)
    y = host(nv.gemv(*args))
    nv.check_device_faults()
    y_ref, ad = oracle.gemv(codes, scales, g, x)
    check_tol(y, y_ref, ad, "after the fault path")
