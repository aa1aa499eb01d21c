#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s and % of the HBM roofline of the NVFP4 g16
W4A16 GEMV on one MI355X.

Headline leg (``value``): the LM-head-sized GEMV, M=1, N=151936, K=4096 (the
llama.cpp trace page's output.weight at one token). A step is one GEMV call.
Secondary legs, measured the same way and reported in the same JSON line:
  m8    - the stress GEMV pair at M=8 (12288x4096 and 4096x12288, Student-t
          weights with 1% zero blocks), one step = both calls;
  layer - the dense decode layer at M=5 (q, k, v, o, gate, up, down), one
          step = the seven calls;
  w4a4  - the pages' W4A4 dense FFN at M=2 (gate, up, down 4096x4096): one
          step = quantizing x with a static input scale and the three calls;
  moe   - the 288-expert MoE expert-slot pass at M=8 (and M=1), top-8, and
          the same pass with the pages' shared expert (768 wide) fused in;
  copy  - a plain fp32 copy kernel of 2 x 512 MiB per launch: the measured
          bandwidth that the other legs are also reported against, and the
          calibration of the HBM byte counters.
Throughput counts algorithmic bytes (codes + scales + tensor scale + x + y;
for the MoE every distinct expert's weights once) per second, inputs already
resident in HBM. Weight copies are rotated so that each call reads memory
the previous calls did not (the 256 MB MALL cannot serve repeats).

Timing: W warm-up steps, then exactly K steps between two device
synchronisations (wall clock -> ms_per_step, value). Two HIP events on the
launch stream bracket the timed launches; their elapsed time over K is the
kernel's average launch duration (gaps between back-to-back launches
included) used for ``roofline.achieved``.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X published HBM3E bandwidth
METRIC = "achieved HBM GB/s and % of roofline, NVFP4 W4A16 GEMV at M=1 and M=8"
MIN_ROTATION_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                              capture_output=True, text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


def library_source_hash():
    """Hash of the library's sources and public header (identifies the build
    where the tree carries no git metadata)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "nvfp4_block_scaled_gemv_amd", "csrc", "*"))
                       + [os.path.join(ROOT, "include", "nvfp4_gemv.h")]):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


def timed_steps(torch, step, steps, warmup):
    """Run `warmup` untimed steps, then exactly `steps` timed ones between two
    device synchronisations. Two HIP events on the launch stream (torch's
    current stream, which every call of the library uses) bracket the timed
    launches. Returns (wall ms per step, event ms per step)."""
    for i in range(warmup):
        step(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


_SLEEP_CYCLES_PER_MS = None


def queued_steps(torch, step, steps, first, wall_ms_per_step):
    """Device time per step (us) with every launch queued ahead of the GPU.
    A bounded sleep kernel (torch.cuda._sleep) holds the stream while the
    host issues the steps; they then run back to back, so host time between
    launches (the Python binding takes several microseconds per call) is not
    counted. The events sit after the sleep, around the steps. Returns None
    when the host did not finish issuing before the sleep ended (the number
    would include host gaps) or when the sleep kernel is unavailable."""
    global _SLEEP_CYCLES_PER_MS
    if not hasattr(torch.cuda, "_sleep"):
        return None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if _SLEEP_CYCLES_PER_MS is None:
        c0 = 1 << 22
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(c0)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = c0 / max(e0.elapsed_time(e1), 1e-3)
    hold_ms = 2.0 + 2.0 * wall_ms_per_step * steps
    torch.cuda.synchronize()
    torch.cuda._sleep(int(hold_ms * _SLEEP_CYCLES_PER_MS))
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(first + i)
    e1.record()
    issue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    if issue_ms > 0.8 * hold_ms:
        return None
    return e0.elapsed_time(e1) / steps * 1e3


def back_to_back(torch, step, steps, warmup, wall_ms, nbytes):
    """The queued measurement as bench fields (at most 100 steps, so that the
    launches fit in the stream's hardware queue)."""
    n = min(steps, 100)
    us = queued_steps(torch, step, n, warmup, wall_ms)
    if us is None:
        return {"device_us_back_to_back": None}
    return {"device_us_back_to_back": us,
            "frac_of_peak_back_to_back": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


# ------------------------------------------------------------------- legs

def leg_lm_head(torch, nv, workloads, traffic, steps, warmup, want_cpu):
    import oracle
    M, N, K = 1, 151936, 4096
    log(f"[bench] lm head: generating W {N}x{K}")
    W = workloads.dense_weights(3, 0, 0, N, K)
    Wd = torch.from_numpy(W).cuda()
    codes, scales, g = nv.pack(Wd)
    del Wd
    x_bits = workloads.x_bf16(3, 0, 0, M, K)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    wbytes = traffic.weight_bytes(N, K)
    R = max(2, -(-MIN_ROTATION_BYTES // wbytes))
    copies = [(codes, scales, g)] + [(codes.clone(), scales.clone(), g.clone())
                                     for _ in range(R - 1)]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step(i):
        c, s, gg = copies[i % R]
        nv.gemv_into(c, s, gg, x, y)

    ms, kms = timed_steps(torch, step, steps, warmup)
    B = traffic.gemv_bytes(M, N, K)
    out = {
        "bytes_per_step": B, "ms_per_step": ms, "kernel_us_events": kms * 1e3,
        "gbs_wall": B / (ms * 1e-3) / 1e9, "gbs_kernel": B / (kms * 1e-3) / 1e9,
        "tokens_per_s": M / (ms * 1e-3), "rotate_copies": R,
    }
    # parity of the timed configuration: pack bit-exact, sampled rows in tolerance
    log("[bench] lm head: oracle pack + sampled-row parity")
    t = time.perf_counter()
    c0, s0, g0 = oracle.pack(W)
    pack_s = time.perf_counter() - t
    del W
    torch.cuda.synchronize()
    pack_ok = bool(np.array_equal(codes.cpu().numpy(), c0) and
                   np.array_equal(scales.cpu().numpy(), s0) and
                   np.float32(g.cpu().numpy()[0]) == g0)
    nv.gemv_into(codes, scales, g, x, y)
    yh = y.cpu().numpy()
    rows = np.random.default_rng(0).choice(N, 2048, replace=False)
    yr, ad = oracle.gemv(c0, s0, g0, x_bits, rows=rows)
    worst = float((np.abs(yh[:, rows] - yr) / (1e-3 * ad + 1e-6)).max())
    out["parity"] = {"pack_bit_exact": pack_ok, "sampled_rows": int(len(rows)),
                     "max_err_over_tol": worst, "ok": pack_ok and worst <= 1.0}
    if want_cpu:
        out["cpu_baseline"] = cpu_baseline(c0, s0, g0, x_bits, B, M)
        out["cpu_baseline"]["pack_s"] = pack_s
    return out


def cpu_baseline(c0, s0, g0, x_bits, B, M):
    """The oracle as it stands (fp64, OpenMP over rows) on the host cores:
    the full 151936 x 4096 M=1 GEMV, repeated until about 10 s have passed."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    times = []
    t_end = time.perf_counter() + 10.0
    while len(times) < 2 or (time.perf_counter() < t_end and len(times) < 50):
        t = time.perf_counter()
        oracle.gemv(c0, s0, g0, x_bits)
        times.append(time.perf_counter() - t)
    tm = float(np.median(times))
    out = {"value": B / tm / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"full 151936x4096 M=1 GEMV, {len(times)} runs, median {tm:.3f} s",
           "tokens_per_s": M / tm, "cpu": cpu_model(), "host_cpus": os.cpu_count()}
    # the same oracle on one thread (one run of the full matrix)
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        t = time.perf_counter()
        oracle.gemv(c0, s0, g0, x_bits)
        t1 = time.perf_counter() - t
        gomp.omp_set_num_threads(threads)
        out["one_thread"] = {"value": B / t1 / 1e9, "unit": "GB/s", "seconds": t1}
    except OSError:
        pass
    return out


def leg_m8(torch, nv, workloads, traffic, steps, warmup):
    M = 8
    mats = [(0, 12288, 4096), (1, 4096, 12288)]
    packed, B, wb = [], 0, 0
    for i, N, K in mats:
        log(f"[bench] m8: generating W {N}x{K} (Student-t)")
        W = workloads.dense_weights(5, 0, i, N, K)
        c, s, g = nv.pack(torch.from_numpy(W).cuda())
        x = torch.from_numpy(workloads.x_bf16(5, 0, i, M, K).view(np.int16)).cuda().view(
            torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        packed.append((c, s, g, x, y))
        B += traffic.gemv_bytes(M, N, K)
        wb += traffic.weight_bytes(N, K)
    R = max(2, -(-MIN_ROTATION_BYTES // wb))
    copies = [packed] + [[(c.clone(), s.clone(), g.clone(), x, y) for c, s, g, x, y in packed]
                         for _ in range(R - 1)]

    def step(i):
        for c, s, g, x, y in copies[i % R]:
            nv.gemv_into(c, s, g, x, y)

    ms, kt = timed_steps(torch, step, steps, warmup)
    return {"workload": "stress_m8_t3 (12288x4096 + 4096x12288)", "M": M,
            "bytes_per_step": B, "ms_per_step": ms, "step_us_events": kt * 1e3,
            "gbs_wall": B / (ms * 1e-3) / 1e9, "gbs_kernel": B / (kt * 1e-3) / 1e9,
            "frac_of_peak": B / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS,
            **back_to_back(torch, step, steps, warmup, ms, B),
            "tokens_per_s": M / (ms * 1e-3), "rotate_copies": R}


def leg_layer(torch, nv, workloads, traffic, steps, warmup):
    """The dense decode layer at M=5: q, k, v, o, gate, up, down, each matrix
    from its own weight stream. Timed twice: seven separate calls (each with its
    own x), and fused into four launches (q|k|v and gate|up as one
    multi-projection call each, sharing the group's x)."""
    M = 5
    names = [n for n, _, _ in workloads.DECODE_LAYER]
    packed, B, wb = {}, 0, 0
    for si, (name, N, K) in enumerate(workloads.DECODE_LAYER):
        log(f"[bench] layer: generating {name} {N}x{K}")
        W = workloads.dense_weights(2, 0, si, N, K)
        c, s, g = nv.pack(torch.from_numpy(W).cuda())
        del W
        x = torch.from_numpy(workloads.x_bf16(2, 0, si, M, K).view(np.int16)).cuda().view(
            torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        packed[name] = (c, s, g, x, y)
        B += traffic.gemv_bytes(M, N, K)
        wb += traffic.weight_bytes(N, K)
    R = max(2, -(-MIN_ROTATION_BYTES // wb))
    copies = [packed] + [{k: (c.clone(), s.clone(), g.clone(), x, y)
                          for k, (c, s, g, x, y) in packed.items()} for _ in range(R - 1)]
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    # fused: x read once per launch
    Bf = B - sum((len(gr) - 1) * M * 4096 * 2 for gr in groups)

    def step(i):
        cp = copies[i % R]
        for n in names:
            c, s, g, x, y = cp[n]
            nv.gemv_into(c, s, g, x, y)

    def step_fused(i):
        cp = copies[i % R]
        for gr in groups:
            mats = [cp[n][:3] for n in gr]
            nv.gemv_segments_into(mats, cp[gr[0]][3], [cp[n][4] for n in gr])

    ms, kt = timed_steps(torch, step, steps, warmup)
    msf, ktf = timed_steps(torch, step_fused, steps, warmup)
    return {"workload": "decode_layer_m5 (q,k,v,o 4096/1024 x 4096; gate, up 12288x4096; "
                        "down 4096x12288)", "M": M, "launches_per_step": len(names),
            "bytes_per_step": B, "ms_per_step": ms, "step_us_events": kt * 1e3,
            "gbs_wall": B / (ms * 1e-3) / 1e9, "gbs_kernel": B / (kt * 1e-3) / 1e9,
            "frac_of_peak": B / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS,
            **back_to_back(torch, step, steps, warmup, ms, B),
            "tokens_per_s": M / (ms * 1e-3), "rotate_copies": R,
            "fused": {"launches_per_step": len(groups), "bytes_per_step": Bf,
                      "ms_per_step": msf, "step_us_events": ktf * 1e3,
                      "gbs_kernel": Bf / (ktf * 1e-3) / 1e9,
                      "frac_of_peak": Bf / (ktf * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      **back_to_back(torch, step_fused, steps, warmup, msf, Bf),
                      "tokens_per_s": M / (msf * 1e-3)}}


def leg_w4a4(torch, nv, workloads, traffic, steps, warmup):
    """The pages' W4A4 dense FFN (gate, up, down 4096x4096 at M=2): one step =
    quantizing the activations with a static input scale and the three W4A4
    GEMVs on them, gate|up as one multi-projection call."""
    wl = workloads.WORKLOADS[6]
    M = wl["M"]
    mats = []
    for i, (name, N, K) in enumerate(wl["mats"]):
        log(f"[bench] w4a4: packing {name} {N}x{K}")
        W = torch.from_numpy(workloads.dense_weights(6, 0, i, N, K)).cuda()
        mats.append((nv.pack(W), N, K))
        del W
    K = wl["mats"][0][2]
    wb = sum(traffic.weight_bytes(N, K) for _, N, K in mats)
    reps = max(2, (1 << 30) // wb + 1)
    copies = [mats] + [[(tuple(t.clone() for t in p), N, K) for p, N, K in mats]
                       for _ in range(reps - 1)]
    x = torch.from_numpy(workloads.x_bf16(6, 0, 0, M, K).view(np.int16)).cuda().view(
        torch.bfloat16)
    calib = workloads.x_bf16(6, 1, 0, M, K)
    gx = torch.tensor([np.abs(((calib.astype(np.uint32) << 16).view(np.float32))).max()
                       / 2688.0], dtype=torch.float32, device="cuda")
    cx, sx = nv.quantize_act(x, gx)
    ws = torch.empty(nv.gemv_w4a4_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, N, _ in mats]

    def step(i):
        # gate|up share the activations: one multi-projection call; then down
        nv.quantize_act_into(x, gx, cx, sx)
        cp = copies[i % reps]
        nv.gemv_w4a4_segments_into([cp[0][0], cp[1][0]], cx, sx, gx, ys[:2], ws)
        nv.gemv_w4a4_into(*cp[2][0], cx, sx, gx, ys[2], ws)

    ms, kms = timed_steps(torch, step, steps, warmup)
    B = traffic.quantize_act_bytes(M, K) + sum(traffic.gemv_w4a4_bytes(M, N, K)
                                               for _, N, K in mats)
    return {"workload": "w4a4_ffn_m2 (gate, up, down 4096x4096; static input scale)", "M": M,
            "launches_per_step": 1 + (1 if M <= 2 else 2) * 2, "bytes_per_step": B,
            "ms_per_step": ms,
            "step_us_events": kms * 1e3, "gbs_wall": B / (ms * 1e-3) / 1e9,
            "gbs_kernel": B / (kms * 1e-3) / 1e9,
            "frac_of_peak": B / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            **back_to_back(torch, step, steps, warmup, ms, B),
            "tokens_per_s": M / (ms * 1e-3), "rotate_copies": reps}


def gpu_clock_state():
    """Best-effort read of the DPM clock tables (read-only sysfs)."""
    import glob
    out = {}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_*clk"))[:8]:
        try:
            with open(f) as fh:
                cur = [l.strip() for l in fh if "*" in l]
            out[f.split("/")[-1] + "@" + f.split("/")[-3]] = cur[0] if cur else None
        except OSError:
            pass
    return out or None


def leg_moe(torch, nv, workloads, traffic, steps, warmup, M):
    E, H, I, topk = 288, 4096, 1536, 8
    log(f"[bench] moe M={M}: generating {E} experts on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4_000 + M)
    c13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device="cuda")
    g13 = torch.empty((E,), dtype=torch.float32, device="cuda")
    c2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((E, H, I // 16), dtype=torch.uint8, device="cuda")
    g2 = torch.empty((E,), dtype=torch.float32, device="cuda")
    for e in range(E):
        w = torch.randn((2 * I, H), generator=gen, device="cuda") * 0.02
        nv.pack_into(w, c13[e], s13[e], g13[e:e + 1])
        w = torch.randn((H, I), generator=gen, device="cuda") * 0.02
        nv.pack_into(w, c2[e], s2[e], g2[e:e + 1])
    del w
    nb = 16
    batches = []
    for b in range(nb):
        ids, gw = workloads.moe_routing(4, b, M, E, topk)
        x = torch.from_numpy(workloads.x_bf16(4, b, 0, M, H).view(np.int16)).cuda().view(
            torch.bfloat16)
        batches.append((torch.from_numpy(ids).cuda(), torch.from_numpy(gw).cuda(), x,
                        len(set(ids.ravel().tolist()))))
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    D = float(np.mean([batches[(warmup + i) % nb][3] for i in range(steps)]))

    def run(step, nbytes, workload):
        ms, kms = timed_steps(torch, step, steps, warmup)
        # bytes of the steps actually timed (each step's own distinct-expert count)
        B = float(np.mean([nbytes(batches[(warmup + i) % nb][3]) for i in range(steps)]))
        return {"workload": workload, "M": M,
                "distinct_experts_mean": D, "bytes_per_step": B, "ms_per_step": ms,
                "pass_us": kms * 1e3, "gbs_wall": B / (ms * 1e-3) / 1e9,
                "gbs_pass": B / (kms * 1e-3) / 1e9,
                "frac_of_peak": B / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                **back_to_back(torch, step, steps, warmup, ms, float(np.mean(
                    [nbytes(batches[(warmup + i) % nb][3]) for i in range(min(steps, 100))]))),
                "tokens_per_s": M / (ms * 1e-3), "rotating_batches": nb}

    ws = torch.empty(nv.moe_workspace_bytes(M, H, I, topk), dtype=torch.uint8, device="cuda")

    def step(i):
        ids, gw, x, _ = batches[i % nb]
        nv.moe_gemv_into(c13, s13, g13, c2, s2, g2, x, ids, gw, y, ws)

    routed = run(step, lambda d: traffic.moe_bytes(M, H, I, topk, d),
                 f"moe_288x(3072x4096,4096x1536)_top8_m{M}")

    # the same call with the shared expert of the pages (gate|up 768+768 x
    # 4096, down 4096 x 768) in the same two launches
    Is = 768
    w = torch.randn((2 * Is, H), generator=gen, device="cuda") * 0.02
    sh13 = nv.pack(w)
    w = torch.randn((H, Is), generator=gen, device="cuda") * 0.02
    sh2 = nv.pack(w)
    del w
    shared = (*sh13, *sh2)
    wss = torch.empty(nv.moe_shared_workspace_bytes(M, H, I, topk, Is), dtype=torch.uint8,
                      device="cuda")

    def step_shared(i):
        ids, gw, x, _ = batches[i % nb]
        nv.moe_shared_gemv_into(c13, s13, g13, c2, s2, g2, x, ids, gw, shared, y, wss)

    with_shared = run(step_shared, lambda d: traffic.moe_shared_bytes(M, H, I, topk, d, Is),
                      f"moe_288x(3072x4096,4096x1536)_top8_shared768_m{M}")

    # W4A4 routed experts (static input scales for x and h, calibrated on
    # another batch of the same distributions) with the W4A16 shared expert
    xc = torch.from_numpy(workloads.x_bf16(4, nb, 0, M, H).view(np.int16)).cuda().view(
        torch.bfloat16)
    gx = (xc.float().abs().max() / 2688.0).reshape(1)
    idc, gwc = (torch.from_numpy(a).cuda() for a in workloads.moe_routing(4, nb, M, E, topk))
    nv.moe_shared_gemv_into(c13, s13, g13, c2, s2, g2, xc, idc, gwc, shared, y, wss)
    hc = wss[:M * topk * I * 2].view(torch.bfloat16).float()
    gh = (hc.abs().max() / 2688.0).reshape(1)
    wsq = torch.empty(nv.moe_w4a4_workspace_bytes(M, H, I, topk, Is), dtype=torch.uint8,
                      device="cuda")

    def step_w4a4(i):
        ids, gw, x, _ = batches[i % nb]
        nv.moe_w4a4_gemv_into(c13, s13, g13, c2, s2, g2, x, gx, gh, ids, gw, y, wsq,
                              shared=shared)

    w4a4 = run(step_w4a4, lambda d: traffic.moe_w4a4_bytes(M, H, I, topk, d, Is),
               f"moe_w4a4_288x(3072x4096,4096x1536)_top8_shared768_m{M}")
    w4a4["launches_per_step"] = 3 if M == 1 else 4
    return routed, with_shared, w4a4


def leg_copy(torch, steps, warmup):
    """Calibration for the HBM byte counters: a plain fp32 copy kernel
    (dst = src * 1) of known size, 512 MiB read and 512 MiB written per
    launch, two buffer pairs alternating so the MALL cannot serve repeats."""
    n = (512 << 20) // 4
    bufs = [(torch.ones(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(2)]

    def step(i):
        src, dst = bufs[i % 2]
        torch.mul(src, 1.0, out=dst)

    ms, kms = timed_steps(torch, step, steps, warmup)
    return {"bytes_read": n * 4, "bytes_written": n * 4, "us_events": kms * 1e3,
            "gbs": 2 * n * 4 / (kms * 1e-3) / 1e9}


# ------------------------------------------------------- profile summaries

LM_KERNEL = "nvfp4::k_gemv<1, 4, false>"
COPY_KERNEL = "MulFunctor<float>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gemv_lm_head_m1_151936x4096.txt")
KERNEL_SOURCES = ["gemv.hip", "gemv_core.h", "device.h"]


def kernel_source_hash():
    """Hash of the LM-head kernel's sources with comments and whitespace
    removed, so that the stored traffic counters stay valid across edits
    that do not change the code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_gemv_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                  # line comments
        h.update(f.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _pmc_means(csv_path, counter):
    """Mean per-dispatch value of `counter` for each kernel name."""
    import csv
    acc = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _copy_units(csv_path, counter):
    """Mean per-dispatch value of `counter` for the copy kernel: among the
    dispatches whose kernel name contains COPY_KERNEL, those with the largest
    grid (other legs run the same elementwise kernel on smaller tensors).
    Returns (mean, dispatches) or None."""
    import csv
    rows = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and COPY_KERNEL in row["Kernel_Name"]:
                rows.append((int(row.get("Grid_Size") or 0), float(row["Counter_Value"])))
    if not rows:
        return None
    top = max(g for g, _ in rows)
    vals = [v for g, v in rows if g == top]
    return sum(vals) / len(vals), len(vals)


def _pick(means, key):
    hits = [(k, v) for k, v in means.items() if key in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {[k for k, _ in hits]}")
    return hits[0][1]


def summarize_pmc(fetch_csv, write_csv, cmd, out):
    """HBM traffic of the LM-head kernel per launch from two rocprofv3 --pmc
    passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what
    the same counter reads for the copy kernel of known size."""
    from nvfp4_block_scaled_gemv_amd import traffic
    f_k, nf = _pick(_pmc_means(fetch_csv, "FETCH_SIZE"), LM_KERNEL)
    w_k, nw = _pick(_pmc_means(write_csv, "WRITE_SIZE"), LM_KERNEL)
    fc, wc = _copy_units(fetch_csv, "FETCH_SIZE"), _copy_units(write_csv, "WRITE_SIZE")
    if fc is None or wc is None:
        raise SystemExit("no copy kernel dispatches in the counter CSVs")
    (f_c, nfc), (w_c, nwc) = fc, wc
    copy_bytes = 512 << 20
    fr, fw = copy_bytes / f_c, copy_bytes / w_c        # bytes per counter unit
    read_b, write_b = f_k * fr, w_k * fw
    alg = traffic.gemv_bytes(1, 151936, 4096)
    lines = [
        "# HBM traffic of the LM-head GEMV kernel, LM head M=1 N=151936 K=4096",
        "# commands (run from /tmp with TMPDIR=/tmp):",
        *[f"#   {c}" for c in cmd],
        f"kernel_source_sha256_16: {kernel_source_hash()}",
        f"fetch_kib_per_dispatch: {f_k:.1f}  (mean of {nf} dispatches)",
        f"write_kib_per_dispatch: {w_k:.1f}  (mean of {nw} dispatches)",
        f"copy_fetch_kib_per_dispatch: {f_c:.1f}  (mean of {nfc}; 512 MiB read)",
        f"copy_write_kib_per_dispatch: {w_c:.1f}  (mean of {nwc}; 512 MiB written)",
        f"calibration_bytes_per_unit: fetch {fr:.2f}, write {fw:.2f}",
        f"read_bytes_per_launch: {read_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {read_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {(read_b + write_b) / alg:.4f}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic():
    """traffic bytes per launch from the committed counter summary, or None
    when it is missing or was taken on different kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip().split()[0]
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def summarize_stats(stats_csv, cmd, out, top=16):
    """Short text table from a rocprofv3 --stats kernel summary, with the
    per-dispatch median, p10 and p90 from the kernel trace next to it."""
    import csv
    rows = []
    with open(stats_csv, newline="") as f:
        for r in csv.DictReader(f):
            rows.append(r)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    durs = {}
    # rocprofv3 writes <prefix>_kernel_trace.csv beside <prefix>_kernel_stats.csv
    trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
    if trace_csv == stats_csv:
        trace_csv = ""
    if trace_csv and os.path.exists(trace_csv):
        with open(trace_csv, newline="") as f:
            for r in csv.DictReader(f):
                durs.setdefault(r["Kernel_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 --kernel-trace --stats kernel summary (durations in us;",
             "# median/p10/p90 over the dispatches in the kernel trace)",
             "# commands (run from /tmp with TMPDIR=/tmp):", *[f"#   {c}" for c in cmd],
             f"{'calls':>7} {'avg':>9} {'median':>9} {'p10':>9} {'p90':>9} {'min':>9} "
             f"{'max':>9} {'pct':>6}  kernel"]
    for r in rows[:top]:
        name = r["Name"]
        short = name.split("(")[0] if name.startswith(("nvfp4", "void nvfp4")) else name[:90]
        d = np.sort(np.array(durs.get(name, [float("nan")])))
        med, p10, p90 = (float(np.percentile(d, q)) for q in (50, 10, 90))
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.2f} {med:9.2f} "
                     f"{p10:9.2f} {p90:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}  {short}")
    if trace_csv and os.path.exists(trace_csv):
        lines += moe_pass_sums(trace_csv)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def moe_pass_sums(trace_csv):
    """MoE passes from a kernel trace, in dispatch order: each pass is
    [k_quantize_decode] k_moe_gate_up [k_quantize_decode] k_moe_down, and
    its time is the sum of its kernels' durations (gaps between launches
    excluded). Grouped by the gate|up grid's y size (slots M*topk, plus one
    row when a shared expert rides along) and by whether the activations
    are quantized (W4A4)."""
    import csv
    with open(trace_csv, newline="") as f:
        rows = [r for r in csv.DictReader(f)
                if any(k in r["Kernel_Name"] for k in
                       ("k_moe_gate_up", "k_moe_down", "k_quantize_decode"))]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    passes, cur = {}, None
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        name = r["Kernel_Name"]
        if cur is None:
            cur = {"w4a4": "k_quantize_decode" in name, "gy": None, "us": 0.0, "n": 0}
        cur["us"] += d
        cur["n"] += 1
        if "k_moe_gate_up" in name:
            cur["gy"] = int(r.get("Grid_Size_Y", 0) or 0)
        if "k_moe_down" in name:
            key = (cur["gy"], cur["w4a4"], cur["n"])
            passes.setdefault(key, []).append(cur["us"])
            cur = None
    out = ["", "# MoE passes: sum of the kernel durations of each pass (us), by gate|up",
           "# grid.y (slots M*topk, +1 with a shared expert) and W4A4 or not",
           f"{'passes':>7} {'median':>9} {'p10':>9} {'p90':>9}  pass"]
    for (gy, w4, n), v in sorted(passes.items(), key=lambda kv: (kv[0][0] or 0, kv[0][1])):
        a = np.array(v)
        out.append(f"{len(v):7d} {np.median(a):9.2f} {np.percentile(a, 10):9.2f} "
                   f"{np.percentile(a, 90):9.2f}  gate|up grid.y={gy}, "
                   f"{'W4A4' if w4 else 'W4A16'}, {n} launches")
    return out


def summarize_counters(csvs, cmd, out, match="nvfp4::"):
    """Per-kernel means of every counter in rocprofv3 --pmc CSVs (one per
    pass), for kernels whose name contains `match`. FETCH_SIZE is also given
    in bytes, scaled by what it reads for the copy kernel of known size when
    that kernel is in the same CSV, and divided by TCP_TCC_READ_REQ_sum where
    both were collected (HBM bytes per L1-to-L2 read request)."""
    import csv
    fetch_scale = None
    for path in csvs:
        fc = _copy_units(path, "FETCH_SIZE")
        if fc is not None:
            fetch_scale = (512 << 20) / fc[0]
    vals = {}
    for path in csvs:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if match not in name:
                    continue
                short = name.split("(")[0].replace("void ", "")
                vals.setdefault(short, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    lines = ["# rocprofv3 --pmc counter means per dispatch (one pass per command)",
             "# commands (run from /tmp with TMPDIR=/tmp):", *[f"#   {c}" for c in cmd],
             f"# FETCH_SIZE calibration: {fetch_scale:.2f} bytes per unit (copy kernel)"
             if fetch_scale else "# FETCH_SIZE calibration: no copy kernel in the CSVs"]
    for kern in sorted(vals):
        c = {k: float(np.mean(v)) for k, v in vals[kern].items()}
        n = min(len(v) for v in vals[kern].values())
        lines.append(f"kernel {kern}  ({n}+ dispatches)")
        for k in sorted(c):
            lines.append(f"  {k:40s} {c[k]:14.6g}")
        if "FETCH_SIZE" in c and fetch_scale:
            fb = c["FETCH_SIZE"] * fetch_scale
            lines.append(f"  {'HBM bytes read (calibrated FETCH_SIZE)':40s} {fb:14.6g}")
            if c.get("TCP_TCC_READ_REQ_sum"):
                lines.append(f"  {'HBM bytes per L1->L2 read request':40s} "
                             f"{fb / c['TCP_TCC_READ_REQ_sum']:14.1f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--legs", default="lm_head,m8,layer,w4a4,moe,copy",
                    help="comma list of lm_head, m8, layer, w4a4, moe, copy (lm_head is the "
                         "headline; copy is a plain copy kernel: the byte-counter "
                         "calibration and the measured-bandwidth reference)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"),
                    help="write the traffic summary from two rocprofv3 --pmc passes")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "OUT"),
                    help="write a short table from a rocprofv3 --stats kernel summary")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV_THEN_OUT",
                    help="write per-kernel counter means from rocprofv3 --pmc CSVs "
                         "(last argument: the output file)")
    ap.add_argument("--cmd", action="append", default=[],
                    help="command line(s) that produced the profile, for the summary header")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc[:2], args.cmd, args.summarize_pmc[2])
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.cmd, args.summarize_stats[1])
        return
    if args.summarize_counters:
        if len(args.summarize_counters) < 2:
            ap.error("--summarize-counters needs at least one CSV and the output file")
        summarize_counters(args.summarize_counters[:-1], args.cmd, args.summarize_counters[-1])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported; the GEMV is sharded by output rows across GPUs and each GPU's share "
              "is this single-GPU kernel at a smaller N.", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_block_scaled_gemv_amd as nv
    from nvfp4_block_scaled_gemv_amd import traffic
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nv.lib()   # fail loudly if the HIP library is not built
    legs = [s.strip() for s in args.legs.split(",") if s.strip()]
    props = torch.cuda.get_device_properties(0)
    result = {
        "metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "lm_head_m1_151936x4096", "M": 1, "N": 151936, "K": 4096,
                   "weights": "nvfp4 g16 from N(0,0.02) fp32, packed on the GPU",
                   "x": "bf16 N(0,1)", "y": "fp32"},
    }
    if "lm_head" in legs:
        lm = leg_lm_head(torch, nv, workloads, traffic, args.steps, args.warmup,
                         not args.no_cpu_baseline)
        result["value"] = lm["gbs_wall"]
        result["ms_per_step"] = lm["ms_per_step"]
        result["tokens_per_s"] = lm["tokens_per_s"]
        result["frac_of_peak_wall"] = lm["gbs_wall"] / HBM_PEAK_GBS
        result["roofline"] = {"bound": "hbm", "achieved": lm["gbs_kernel"],
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": lm["gbs_kernel"] / HBM_PEAK_GBS,
                              "traffic": read_traffic(),
                              "kernel": LM_KERNEL,
                              "kernel_avg_us": lm["kernel_us_events"],
                              "bytes_per_launch": lm["bytes_per_step"]}
        result["config"]["rotate_copies"] = lm["rotate_copies"]
        result["parity"] = lm["parity"]
        if "cpu_baseline" in lm:
            result["cpu_baseline"] = lm["cpu_baseline"]
    if "m8" in legs:
        result["m8"] = leg_m8(torch, nv, workloads, traffic, args.steps, args.warmup)
    if "layer" in legs:
        result["layer_m5"] = leg_layer(torch, nv, workloads, traffic, args.steps, args.warmup)
    if "w4a4" in legs:
        result["w4a4_ffn_m2"] = leg_w4a4(torch, nv, workloads, traffic, args.steps, args.warmup)
    if "copy" in legs:
        cp = leg_copy(torch, min(args.steps, 50), min(args.warmup, 5))
        result["copy_calibration"] = cp
        # fractions of the measured copy bandwidth (read + write bytes per second)
        if result.get("roofline"):
            result["roofline"]["frac_of_measured_copy"] = result["roofline"]["achieved"] / cp["gbs"]
        for k in ("m8", "layer_m5", "w4a4_ffn_m2"):
            if k in result:
                result[k]["frac_of_measured_copy"] = result[k]["gbs_kernel"] / cp["gbs"]
    if "moe" in legs:
        result["moe"], result["moe_shared"], result["moe_w4a4"] = {}, {}, {}
        for M in (1, 8):
            routed, with_shared, w4a4 = leg_moe(torch, nv, workloads, traffic, args.steps,
                                                args.warmup, M)
            result["moe"][f"m{M}"] = routed
            result["moe_shared"][f"m{M}"] = with_shared
            result["moe_w4a4"][f"m{M}"] = w4a4
    result["env"] = {"gpu": props.name, "cus": props.multi_processor_count,
                     "dpm_clocks": gpu_clock_state(),
                     "hip": torch.version.hip, "torch": torch.__version__, "git": git_sha(),
                     "library_sources_sha256_16": library_source_hash(),
                     "argv": sys.argv[1:]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
