"""The slot protocol of the split-K GEMV's reduction (splitk_slots.h), built
for the host with g++ and run as a model under random interleavings of W
wavefronts: every tile is summed exactly once from its own W partials, and
when the bounded slot wait gives up, no wait runs forever and every wrong
result comes with the fault recorded."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_gemv_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_slot_protocol_model(tmp_path):
    exe = tmp_path / "slot_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", CSRC, "-o", str(exe),
                    os.path.join(ROOT, "tests", "slot_check.cpp")],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_slot_model_catches_a_wrong_last_arrival(tmp_path):
    """The model is not vacuous: with the last-arrival test off by one (a
    plausible slip) it fails."""
    src = open(os.path.join(CSRC, "splitk_slots.h")).read()
    bad = src.replace("round * (uint32_t)W + (uint32_t)(W - 1)", "round * (uint32_t)W + (uint32_t)W")
    assert bad != src
    d = tmp_path / "inc"
    d.mkdir()
    (d / "splitk_slots.h").write_text(bad)
    shutil.copy(os.path.join(CSRC, "segments.h"), d / "segments.h")
    exe = tmp_path / "slot_check_bad"
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", str(d), "-o", str(exe),
                    os.path.join(ROOT, "tests", "slot_check.cpp")],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode != 0 and out.stdout.startswith("FAIL"), out.stdout
