"""The boundary from plain C: tests/c_abi_check.c is compiled with gcc as
strict C99 against include/nvfp4_gemv.h, linked to the built library and run
(host-side paths only; no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "nvfp4_block_scaled_gemv_amd")
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.skipif(not os.path.exists(os.path.join(LIBDIR, "libnvfp4_gemv.so")),
                    reason="library not built")
def test_c_program_uses_the_abi(tmp_path):
    exe = tmp_path / "c_abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe),
           "-L", LIBDIR, "-lnvfp4_gemv", f"-Wl,-rpath,{LIBDIR}"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=120)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
