"""bench.py's command line on the CPU: more than one GPU is refused with a
message and exit status 2 before anything touches a device, and the profile
summaries parse the CSV layout rocprofv3 writes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


STATS = (
    '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
    '"void nvfp4::k_gemv<1, 4, false>",3,165000,55000,80.0,54000,56000,800\n'
    '"nvfp4::k_amax",2,20000,10000,20.0,9000,11000,1000\n')
TRACE = (
    '"Kernel_Name","Start_Timestamp","End_Timestamp","Grid_Size_Y"\n'
    '"void nvfp4::k_gemv<1, 4, false>",0,54000,1\n'
    '"void nvfp4::k_gemv<1, 4, false>",60000,115000,1\n'
    '"void nvfp4::k_gemv<1, 4, false>",120000,176000,1\n'
    '"void nvfp4::k_moe_gate_up<1>",200000,212000,8\n'
    '"void nvfp4::k_moe_down<2, 2>",212500,222500,1\n')


def _summarize(stats, out):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-stats",
                           str(stats), str(out), "--cmd", "the command"],
                          capture_output=True, text=True, timeout=120)


def test_stats_summary_with_trace(tmp_path):
    """Medians come from the kernel trace beside the stats file, and the MoE
    pass sums from its gate|up and down dispatches."""
    (tmp_path / "b_kernel_stats.csv").write_text(STATS)
    (tmp_path / "b_kernel_trace.csv").write_text(TRACE)
    out = tmp_path / "summary.txt"
    r = _summarize(tmp_path / "b_kernel_stats.csv", out)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    assert "the command" in text
    row = [l for l in text.splitlines() if "k_gemv<1, 4, false>" in l][0].split()
    assert row[0] == "3" and row[2] == "55.00"          # calls, median over the trace
    assert "gate|up grid.y=8, W4A16, 2 launches" in text
    line = [l for l in text.splitlines() if "grid.y=8" in l][0].split()
    assert line[1] == "22.00"                              # 12 + 10 us


def test_stats_summary_without_trace(tmp_path):
    """A stats file with no trace beside it (or not named like rocprofv3's)
    still gives the table, without medians."""
    csv = tmp_path / "stats.csv"
    csv.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void nvfp4::k_gemv<1, 4, false>",3,165000,55000,80.0,54000,56000,800\n'
        '"nvfp4::k_amax",2,20000,10000,20.0,9000,11000,1000\n')
    out = tmp_path / "summary.txt"
    r = _summarize(csv, out)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    assert "the command" in text and "k_gemv<1, 4, false>" in text and "k_amax" in text


def _pmc_csv(path, counter, rows):
    """rows: (kernel name, counter value[, grid size])."""
    lines = ['"Dispatch_Id","Grid_Size","Kernel_Name","Counter_Name","Counter_Value"']
    lines += [f'{i},{r[2] if len(r) > 2 else 1024},"{r[0]}","{counter}",{r[1]}'
              for i, r in enumerate(rows)]
    path.write_text("\n".join(lines) + "\n")


def test_traffic_summary_scales_by_the_copy_kernel(tmp_path):
    """FETCH_SIZE and WRITE_SIZE of the LM-head kernel are turned into bytes
    with the bytes per counter unit that the copy kernel of known size (512
    MiB read and 512 MiB written per launch) gives; the header carries the
    hash of the kernel sources that stored traffic is keyed on."""
    lm = "void nvfp4::k_gemv<1, 4, false>(nvfp4::SegTable, unsigned short const*, long)"
    cp = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>()"
    # the same elementwise kernel on a smaller tensor (another leg) is not the copy
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(lm, 171000.0), (lm, 171002.0),
                                                (cp, 262144.0, 33554432), (cp, 999.0, 4096)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(lm, 600.0), (lm, 600.0),
                                                (cp, 524288.0, 33554432), (cp, 7.0, 4096)])
    out = tmp_path / "traffic.txt"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-pmc",
                        str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out),
                        "--cmd", "pass 1", "--cmd", "pass 2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    kv = dict(l.split(":", 1) for l in out.read_text().splitlines()
              if ":" in l and not l.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    # 512 MiB over 262144 and over 524288 counter units
    assert kv["calibration_bytes_per_unit"] == "fetch 2048.00, write 1024.00"
    kv = {k: v.split()[0] for k, v in kv.items()}
    assert int(kv["read_bytes_per_launch"]) == 171001 * 2048
    assert int(kv["write_bytes_per_launch"]) == 600 * 1024
    assert int(kv["traffic_bytes_per_launch"]) == 171001 * 2048 + 600 * 1024
    h = subprocess.run([sys.executable, "-c", "import bench; print(bench.kernel_source_hash())"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120).stdout.strip()
    assert kv["kernel_source_sha256_16"] == h
