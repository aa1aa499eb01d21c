"""The matrix-core GEMV kernels issue their weight loads through inline asm;
their compiled gfx950 code must never touch a load's destination registers
before a vmcnt wait has retired that load (a tail that issued loads nobody
consumed once let the epilogue reuse those registers while the data was still
in flight). Compiles the kernels with hipcc (no GPU needed) and walks the
assembly."""
import os
import shutil
import subprocess

import pytest

from isa_pending import check_asm, violations

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_gemv_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def test_walker_flags_a_touch_before_the_wait():
    body = ["global_load_dwordx4 v[4:7], v[0:1], off nt",
            "v_add_u32_e32 v5, v5, v2",            # touches a pending dest
            "s_waitcnt vmcnt(0)",
            "v_add_u32_e32 v6, v6, v2"]
    found = violations(body)
    assert [f[0] for f in found] == [1]
    ok = ["global_load_dwordx4 v[4:7], v[0:1], off nt",
          "global_load_lds_dwordx4 v[0:1], off",
          "s_waitcnt vmcnt(1)",
          "v_add_u32_e32 v5, v5, v2"]
    assert violations(ok) == []
    # a load into registers another load still has pending is a write after
    # write (returns are in order), but its address must not be pending
    waw = ["global_load_dwordx4 v[40:43], v[0:1], off",
           "global_load_ushort v40, v[4:5], off"]
    assert violations(waw) == []
    raw = ["global_load_dwordx4 v[40:43], v[0:1], off",
           "global_load_ushort v50, v[40:41], off"]
    assert [f[0] for f in violations(raw)] == [1]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_splitk_kernels_leave_pending_loads_alone(tmp_path):
    out = tmp_path / "splitk.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, "gemv_splitk.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    text = out.read_text()
    res = check_asm(text, r"_Z\S*k_gemv_splitk\S*")
    # M = 3..8 x (one x slice held with a ring of 3, two with a ring of 4,
    # x streamed with rings of 3 and 4)
    assert len(res) == 24, sorted(res)
    bad = {k: v[:3] for k, v in res.items() if v}
    assert not bad, bad
    # the loads are really there and waited for by count, not drained
    assert text.count("global_load_dwordx4") >= 24 * 11
    for n in (3, 12, 11, 22):   # (ring - 2) x loads per item of each variant
        assert f"vmcnt({n})" in text, n
    # no spills: a spilled ring register would be stored while its load is pending
    assert "scratch_" not in text


# The other kernel with hand-placed waits: the matrix-core GEMV for K not a
# multiple of 256 copies x into LDS by DMA and reads it with inline-asm LDS
# reads, ordered by an explicit vmcnt wait. (The remaining kernels issue
# every load through the compiler, whose own wait insertion tracks them; the
# walk is linear and would see the two sides of their branches as one path.)
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_mfma_kernel_leaves_pending_loads_alone(tmp_path):
    out = tmp_path / "mfma.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, "gemv_mfma.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    text = out.read_text()
    res = check_asm(text, r"_Z\S*k_gemv_mfma\S*")
    assert len(res) == 1, sorted(res)
    bad = {k: v[:3] for k, v in res.items() if v}
    assert not bad, bad
    # the x copies go by LDS DMA and the A operands come from asm LDS reads
    assert "global_load_lds_dwordx4" in text and "ds_read_b128" in text
    assert "scratch_" not in text


KERNEL_FILES = ["gemv.hip", "gemv_g8.hip", "gemv_g8r.hip", "gemv_mfma.hip", "gemv_splitk.hip", "gemv_mt.hip",
                "moe.hip", "w4a4.hip", "pack.hip", "stream_read.hip"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_no_kernel_spills_registers(tmp_path):
    """Every kernel fits its registers: no VGPR spills and no private
    (scratch) memory. A spill costs a round trip to memory per use; a size
    bound shared between kernels once grew a per-token array of the MoE down
    pass to 128 entries and spilled it whole."""
    import re
    procs = {}
    for f in KERNEL_FILES:
        out = tmp_path / (f + ".s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
               "-o", str(out), os.path.join(CSRC, f)]
        procs[f] = (subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE), out)
    kernels = 0
    g8_one_slice = 0
    for f, (p, out) in procs.items():
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, (f, err[-2000:])
        text = out.read_text()
        for block in text.split("- .agpr_count:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", block).group(1)
            spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1))
            priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
            assert spill == 0 and priv == 0, (f, name, spill, priv)
            kernels += 1
            # the eight-token kernel with one slice per wavefront and one or
            # two tiles runs 16-wavefront workgroups two to a CU only within
            # 64 registers (eight wavefronts per SIMD); at 70 the LM head at
            # M = 8 took 87.6 instead of 73.3 us
            m = re.match(r"_ZN5nvfp49k_gemv_g8ILi\d+ELi([12])ELi1EEE", name)
            if m:
                vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
                assert vgpr <= 64, (name, vgpr)
                g8_one_slice += 1
    assert kernels >= 40, kernels
    assert g8_one_slice == 14, g8_one_slice   # M = 2 .. 8, one or two tiles
