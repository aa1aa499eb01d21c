"""The algorithmic byte model against the floors the blueprint prints
(card.json performance[i].floor_us), and the per-workload totals."""
import pytest

from conftest import golden_rows
from nvfp4_block_scaled_gemv_amd import traffic


def test_pages_floors_reproduce():
    rows = golden_rows("roofline_floors.txt")
    assert len(rows) == 6
    for idx, M, N, K, experts, bits, act, out, floor in rows:
        got = traffic.pages_floor_us(float(M), int(N), int(K), float(experts), float(bits),
                                     float(act), int(out))
        assert abs(got - float(floor)) < 0.0015, (idx, got, floor)


def test_gemv_bytes_workloads():
    assert traffic.gemv_bytes(1, 1024, 4096) == 2_371_588
    assert traffic.gemv_bytes(1, 151936, 4096) == 350_676_484
    layer = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (12288, 4096),
             (12288, 4096), (4096, 12288)]
    assert sum(traffic.gemv_bytes(5, n, k) for n, k in layer) == 109_674_524
    assert traffic.gemv_bytes(8, 12288, 4096) == 28_770_308
    assert traffic.gemv_bytes(8, 4096, 12288) == 28_639_236


def test_weight_bytes_are_4p5_bits():
    assert traffic.weight_bytes(3072, 4096) * 8 == 3072 * 4096 * 4.5


def test_moe_bytes_counts_distinct_experts():
    one = traffic.moe_bytes(1, 4096, 1536, 8, 8)
    assert one > 8 * (traffic.weight_bytes(3072, 4096) + traffic.weight_bytes(4096, 1536))
    assert traffic.moe_bytes(8, 4096, 1536, 8, 58) < traffic.moe_bytes(8, 4096, 1536, 8, 64)


def test_moe_shared_bytes_add_the_shared_expert_once():
    # the pages' shared expert: gate|up 768 + 768 by 4096, down 4096 by 768
    routed = traffic.moe_bytes(8, 4096, 1536, 8, 58)
    shared = traffic.moe_shared_bytes(8, 4096, 1536, 8, 58, 768)
    w = 1536 * 4096 * 9 // 16 + 4096 * 768 * 9 // 16   # 4.5 bits per weight
    assert shared - routed == w + 8 + 2 * 8 * 768 * 2
    assert traffic.moe_shared_bytes(1, 64, 32, 2, 1, 0) == traffic.moe_bytes(1, 64, 32, 2, 1) + 8


def test_w4a4_bytes():
    # the pages' W4A4 dense FFN matrix: 4096 x 4096 at M=2
    assert traffic.gemv_w4a4_bytes(2, 4096, 4096) == (4096 * 4096 * 9 // 16 + 4
                                                      + 2 * 4096 * 9 // 16 + 4 + 2 * 4096 * 4)
    assert traffic.quantize_act_bytes(2, 4096) == 2 * 4096 * 2 + 4 + 2 * 4096 * 9 // 16


def test_moe_w4a4_bytes_add_the_two_quantization_passes():
    # the pages' W4A4 MoE sweeps: 288 experts of [3072, 4096] and [4096, 1536]
    routed = traffic.moe_bytes(2, 4096, 1536, 8, 14)
    q = traffic.moe_w4a4_bytes(2, 4096, 1536, 8, 14)
    assert q - routed == 2 * 2 * 4096 * 2 + 2 * 16 * 1536 * 2 + 8
    with_shared = traffic.moe_w4a4_bytes(2, 4096, 1536, 8, 14, 768)
    assert with_shared - q == traffic.moe_shared_bytes(2, 4096, 1536, 8, 14, 768) - routed
    # one token: h goes onto its grid inside gate|up (no second read of h)
    one = traffic.moe_w4a4_bytes(1, 4096, 1536, 8, 8) - traffic.moe_bytes(1, 4096, 1536, 8, 8)
    assert one == 2 * 4096 * 2 + 8 * 1536 * 2 + 8
