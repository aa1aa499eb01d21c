"""The segment cursor of the split-K GEMV kernel (segments.h), built for the
host with g++ and walked over random segment tables the way the kernel walks
it: every tile of every workgroup range lands in the segment a plain scan of
the table names, and a step past the last tile leaves the cursor on the last
segment (an earlier cursor read past the table there, and a pointer it loaded
from beyond the table was then dereferenced)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_gemv_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_cursor_stays_in_the_table(tmp_path):
    exe = tmp_path / "cursor_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", CSRC, "-o", str(exe),
                    os.path.join(ROOT, "tests", "cursor_check.cpp")],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout
