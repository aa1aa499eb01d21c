#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s and % of roofline of the NVFP4 g16 W4A16 GEMV
on one MI355X, for every workload of the method.

Headline (``value``): the LM-head-sized GEMV, M=1, N=151936, K=4096 (the
llama.cpp trace page's output.weight at one token); a step is one GEMV call.
Every other workload is measured the same way and reported in the same JSON
line under ``configs``:
  1  gemv_m1_1024x4096   - one small GEMV (launch-bound: its HBM time is 0.3 us);
  2  decode_layer_m5     - q, k, v, o, gate, up, down at M=5, seven calls, and
                           fused into four launches (q|k|v and gate|up);
  3  lm_head_m1          - the headline;
  4  moe_m1, moe_m8      - the 288-expert MoE expert-slot pass, top-8;
  5  stress_m8           - 12288x4096 and 4096x12288 at M=8, Student-t weights;
and the wider rows of the method: the LM head at M=8, the stress pair at
M=16 and M=128, the W4A4 dense FFN, the MoE with the pages' 768-wide shared
expert, and the W4A4 MoE.

Throughput counts algorithmic bytes (codes + scales + tensor scale + x + y;
for the MoE every distinct expert's weights once) per second, inputs already
resident in HBM. Weight copies are rotated so that each call reads memory the
previous calls did not (the 256 MB MALL cannot serve repeats).

Timing of each leg:
  * wall: W warm-up steps, then exactly K timed steps between two device
    synchronisations -> ms_per_step and ``value``;
  * step_us (the basis of every GB/s and roofline fraction): a fixed number
    of steps (independent of K) queued on the launch stream behind a busy
    hold of pure-read launches, then run back to back, bracketed by two HIP
    events on that stream. The hold keeps the GPU loaded while the host
    queues: after any idle period the GPU runs its first ~10 ms of kernels
    up to 15% slower, which an idle hold (a sleep kernel) would fold in;
  * window_us: LAUNCH_WINDOW steps issued by the host back to back between
    two events (GPU-bound for long steps, host-bound for short ones).
Each leg also carries its parity against the oracle (all outputs of the timed
configuration), the oracle's own time on the host cores (``cpu``: all threads,
and one thread on a bounded sample) and the fraction of the measured read
ceiling (``nvfp4_stream_read``: a pure read of the same byte count).

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
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X published HBM3E bandwidth
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
METRIC = "achieved HBM GB/s and % of roofline, NVFP4 W4A16 GEMV at M=1 and M=8"
MIN_ROTATION_BYTES = 1 << 30
LAUNCH_WINDOW = 400        # steps in the issue-gated event window of every leg
QUEUED_WINDOW = 200        # steps queued back to back behind a busy hold
QUEUED_LAUNCHES = 400      # at most this many launches queued at once
ALL_LEGS = "lm_head,small,stress,layer,moe,moe_skew,w4a4,wide,copy"
# legs that only run when named: one skewed-routing case each (for counters)
EXTRA_LEGS = "moe_skew_one,moe_skew_same"


HOLD = None               # the BusyHold of this run


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


def oracle_threads():
    return int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)


# ------------------------------------------------------------------ timing

def timed_steps(torch, step, steps, warmup):
    """Run `warmup` untimed steps, then exactly `steps` timed ones between two
    device synchronisations. Returns the wall ms per step."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def launch_window(torch, step, first, n=LAUNCH_WINDOW):
    """Average device time per step (us) over a fixed window of n steps
    issued back to back, bracketed by two HIP events on the launch stream
    (torch's current stream, which the library launches on). While a step
    takes longer on the GPU than the host needs to issue it, the window is
    GPU-bound and the first launch's host latency is spread over n steps;
    for shorter steps the window measures the host, and the queued
    measurement below is the device time."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(n):
        step(first + i)
    e1.record()
    issue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3, issue_ms / n


class BusyHold:
    """Keeps the GPU at full load while the host queues the steps to be
    timed: pure-read launches over a 1 GiB buffer (nvfp4_stream_read). The
    GPU runs the first ~10 ms after any idle period up to 15% slower (a
    clock ramp, seen in rocprofv3 traces after a sleep kernel or a host
    pause), so an idle hold would bias every queued measurement."""

    def __init__(self, torch, nv):
        self.torch, self.nv = torch, nv
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        self.buf.fill_(0x3C)
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        for _ in range(5):
            self.read()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            self.read()
        e1.record()
        torch.cuda.synchronize()
        self.read_ms = e0.elapsed_time(e1) / 20

    def read(self):
        self.nv.stream_read(self.buf, self.sink)

    def hold(self, ms):
        """Queue about `ms` of reads; returns the queued hold in ms."""
        n = max(2, int(np.ceil(ms / self.read_ms)))
        for _ in range(n):
            self.read()
        return n * self.read_ms


def queued_steps(torch, hold, step, steps, first, issue_ms_per_step):
    """Device time per step (us) with the steps queued ahead of the GPU
    behind a busy hold, so that they run back to back with no host time
    between launches. Returns None if the host did not finish issuing them
    before the hold ran out (the number would include host gaps)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold_ms = hold.hold(1.0 + 1.5 * issue_ms_per_step * steps)
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


def measure(torch, hold, step, steps, warmup, nbytes, tokens, launches, ceiling=None):
    """The timing fields of one leg: wall clock over K steps; device time per
    step from a fixed number of steps queued back to back behind a busy hold
    (``step_us``, the basis of every GB/s and fraction below; the
    issue-gated window of LAUNCH_WINDOW steps stands in where the host could
    not queue them in time). `nbytes` = algorithmic bytes per step, `tokens`
    = activation rows per step, `launches` = kernel launches per step,
    `ceiling` = pure-read time (us) of the same bytes."""
    ms = timed_steps(torch, step, steps, warmup)
    win, issue = launch_window(torch, step, warmup + steps)
    nq = max(40, min(QUEUED_WINDOW, QUEUED_LAUNCHES // launches))
    b2b = queued_steps(torch, hold, step, nq, warmup + steps + LAUNCH_WINDOW, issue)
    us = b2b if b2b else win
    out = {"bytes_per_step": nbytes, "launches_per_step": launches, "ms_per_step": ms,
           "gbs_wall": nbytes / (ms * 1e-3) / 1e9,
           "step_us": us, "step_us_basis": (f"{nq} steps queued back to back behind a busy "
                                            "hold" if b2b else
                                            f"{LAUNCH_WINDOW}-step event window"),
           "window_us": win, "host_issue_us_per_step": issue * 1e3,
           "device_us_back_to_back": b2b,
           "gbs": nbytes / (us * 1e-6) / 1e9,
           "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "tokens_per_s": tokens / (ms * 1e-3),
           "tokens_per_s_device": tokens / (us * 1e-6)}
    if ceiling:
        out["read_ceiling_us"] = ceiling
        out["frac_of_read_ceiling"] = ceiling / us
    return out


# ----------------------------------------------------------- read ceiling

class ReadCeiling:
    """Pure-read time of a byte count: nvfp4_stream_read over R buffers of
    that size (R * size >= 1 GiB, rotated), measured like the legs (launches
    queued back to back); the mean device time per launch in us."""

    def __init__(self, torch, nv, hold):
        self.torch, self.nv, self.hold, self.cache = torch, nv, hold, {}
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def us(self, nbytes):
        torch = self.torch
        n16 = -(-int(nbytes) // 16) * 16
        if n16 not in self.cache:
            R = max(2, -(-MIN_ROTATION_BYTES // n16))
            R = min(R, 512)
            bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda") for _ in range(R)]
            for b in bufs:
                b.fill_(0x5A)

            def step(i):
                self.nv.stream_read(bufs[i % R], self.sink)

            win, issue = launch_window(torch, step, 0, 50)
            us = queued_steps(torch, self.hold, step, QUEUED_WINDOW, 50, issue)
            self.cache[n16] = us if us else win
            del bufs
        return self.cache[n16]

    def table(self):
        return {str(b): {"us": us, "gbs": b / (us * 1e-6) / 1e9,
                         "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
                for b, us in sorted(self.cache.items())}


# -------------------------------------------------------------- cpu oracle

def cpu_timed(fn, budget_s=3.0, max_runs=20):
    """Median wall time (s) of fn() on the host, repeated until `budget_s`
    has passed (at least twice)."""
    times = []
    t_end = time.perf_counter() + budget_s
    while len(times) < 2 or (time.perf_counter() < t_end and len(times) < max_runs):
        t = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t)
    return float(np.median(times)), len(times)


def one_thread(fn):
    """Wall time (s) of one call of fn() with the oracle's OpenMP pool cut to
    one thread (None where libgomp cannot be reached)."""
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    gomp.omp_set_num_threads(1)
    try:
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t
    finally:
        gomp.omp_set_num_threads(oracle_threads())


def cpu_baseline(full, nbytes, tokens, what, sample_1t=None, frac_1t=1.0):
    """The oracle as it stands (fp64, OpenMP over rows) timed on the host
    cores: `full()` runs the whole step; `sample_1t()` a bounded part of it
    (fraction `frac_1t` of the work) on one thread, scaled to the whole."""
    tm, runs = cpu_timed(full)
    out = {"value": nbytes / tm / 1e9, "unit": "GB/s", "cores": oracle_threads(),
           "kind": "oracle", "sample": f"{what}: {runs} runs, median {tm:.4f} s",
           "seconds_per_step": tm, "tokens_per_s": tokens / tm, "cpu": cpu_model(),
           "host_cpus": os.cpu_count()}
    t1 = one_thread(sample_1t or full)
    if t1 is not None:
        s = t1 / frac_1t
        out["one_thread"] = {"value": nbytes / s / 1e9, "unit": "GB/s", "cores": 1,
                             "seconds_per_step": s,
                             "sample": (f"{frac_1t:.4g} of the step on one thread "
                                        f"({t1:.3f} s), scaled") if frac_1t != 1.0
                             else f"the whole step on one thread ({t1:.3f} s)"}
    return out


def tol_ratio(y, y_ref, ad):
    """Largest |y - y_ref| / (1e-3 * sum|w x| + 1e-6) and the count above 1."""
    r = np.abs(np.asarray(y, np.float64) - y_ref) / (1e-3 * ad + 1e-6)
    return (float(r.max()) if r.size else 0.0), int((~(r <= 1.0)).sum())


def x_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(
        torch.bfloat16)


# -------------------------------------------------------------- dense legs

class Dense:
    """Packed matrices of one dense workload on the device, their oracle
    packs on the host (for parity), and R rotated device copies."""

    def __init__(self, torch, nv, workloads, traffic, wl, mats, M, rep=0, xs_per_mat=True):
        self.M, self.mats = M, mats
        self.dev, self.host, self.x, self.xbits = [], [], [], []
        wb = 0
        for si, (name, N, K) in enumerate(mats):
            log(f"[bench] workload {wl}: {name} {N}x{K}")
            W = workloads.dense_weights(wl, rep, si, N, K)
            self.dev.append(nv.pack(torch.from_numpy(W).cuda()))
            self.host.append(_oracle().pack(W))
            del W
            xb = workloads.x_bf16(wl, rep, si if xs_per_mat else 0, M, K)
            self.xbits.append(xb)
            self.x.append(x_dev(torch, xb))
            wb += traffic.weight_bytes(N, K)
        self.R = max(2, -(-MIN_ROTATION_BYTES // wb))
        self.copies = [self.dev] + [[tuple(t.clone() for t in p) for p in self.dev]
                                    for _ in range(self.R - 1)]
        self.y = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, N, _ in mats]
        self.bytes = [traffic.gemv_bytes(M, N, K) for _, N, K in mats]

    def pack_exact(self):
        import torch
        torch.cuda.synchronize()
        return all(np.array_equal(d[0].cpu().numpy(), h[0]) and
                   np.array_equal(d[1].cpu().numpy(), h[1]) and
                   np.float32(d[2].cpu().numpy()[0]) == h[2]
                   for d, h in zip(self.dev, self.host))

    def parity(self, ys=None):
        """All outputs of every matrix against the oracle."""
        import torch
        torch.cuda.synchronize()
        ys = ys or self.y
        worst, bad, n = 0.0, 0, 0
        for (c, s, g), xb, y in zip(self.host, self.xbits, ys):
            yr, ad = _oracle().gemv(c, s, g, xb)
            w, b = tol_ratio(y.cpu().numpy(), yr, ad)
            worst, bad, n = max(worst, w), bad + b, n + yr.size
        return {"outputs": n, "max_err_over_tol": worst, "outside_tol": bad,
                "ok": bad == 0}

    def oracle_step(self):
        for (c, s, g), xb in zip(self.host, self.xbits):
            _oracle().gemv(c, s, g, xb)

    def oracle_sample(self, frac):
        """The first `frac` of every matrix's rows."""
        for (c, s, g), xb in zip(self.host, self.xbits):
            n = max(1, int(round(c.shape[0] * frac)))
            _oracle().gemv(c, s, g, xb, rows=np.arange(n))


def _oracle():
    import oracle
    return oracle


def dense_leg(torch, nv, D, steps, warmup, ceil, want_cpu, label, segments=None):
    """One step = every matrix of D, one nvfp4_gemv call each (or, with
    `segments`, one nvfp4_gemv_segments call per group of matrix indices,
    the group sharing the first matrix's x)."""
    M = D.M
    if segments is None:
        def step(i):
            for (c, s, g), x, y in zip(D.copies[i % D.R], D.x, D.y):
                nv.gemv_into(c, s, g, x, y)
        nbytes = sum(D.bytes)
        launches = len(D.mats)
        ceiling = sum(ceil.us(b) for b in D.bytes)
    else:
        def step(i):
            cp = D.copies[i % D.R]
            for grp in segments:
                nv.gemv_segments_into([cp[j] for j in grp], D.x[grp[0]], [D.y[j] for j in grp])
        K = D.mats[0][2]
        nbytes = sum(D.bytes) - sum((len(g) - 1) * M * K * 2 for g in segments)
        launches = len(segments)
        ceiling = sum(ceil.us(sum(D.bytes[j] for j in g)) for g in segments)
    out = {"workload": label, "M": M, "rotate_copies": D.R,
           **measure(torch, HOLD, step, steps, warmup, nbytes, M, launches, ceiling)}
    if segments is None:
        out["parity"] = D.parity()
    else:
        # the fused launches read the group's first x: compare against the
        # oracle on that x
        step(0)
        torch.cuda.synchronize()
        worst, bad, n = 0.0, 0, 0
        for grp in segments:
            for j in grp:
                c, s, g = D.host[j]
                yr, ad = _oracle().gemv(c, s, g, D.xbits[grp[0]])
                w, b = tol_ratio(D.y[j].cpu().numpy(), yr, ad)
                worst, bad, n = max(worst, w), bad + b, n + yr.size
        out["parity"] = {"outputs": n, "max_err_over_tol": worst, "outside_tol": bad,
                         "ok": bad == 0}
    if want_cpu and segments is None:
        frac = min(1.0, 2.0e8 / max(1, sum(N * K for _, N, K in D.mats) * M))
        out["cpu"] = cpu_baseline(D.oracle_step, nbytes, M, f"the whole step ({label})",
                                  lambda: D.oracle_sample(frac), frac)
    return out


# ------------------------------------------------------------------- moe

class Moe:
    """The 288-expert MoE workload on the device: every expert packed on the
    GPU from its seeded fp32 stream (workloads.moe_expert_weights), the pages'
    768-wide shared expert, and rotating batches of routing and x."""

    E, H, I, TOPK, IS = 288, 4096, 1536, 8, 768

    def __init__(self, torch, nv, workloads):
        self.torch, self.nv, self.wl = torch, nv, workloads
        E, H, I = self.E, self.H, self.I
        log(f"[bench] moe: packing {E} experts from their seeded streams")
        d = "cuda"
        self.c13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=d)
        self.s13 = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=d)
        self.g13 = torch.empty((E,), dtype=torch.float32, device=d)
        self.c2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=d)
        self.s2 = torch.empty((E, H, I // 16), dtype=torch.uint8, device=d)
        self.g2 = torch.empty((E,), dtype=torch.float32, device=d)

        def gen(e):
            return e, workloads.moe_expert_weights(4, 0, e, H, I, threads=1)

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            for c0 in range(0, E, 16):
                for e, (w13, w2) in ex.map(gen, range(c0, min(E, c0 + 16))):
                    nv.pack_into(torch.from_numpy(w13).cuda(), self.c13[e], self.s13[e],
                                 self.g13[e:e + 1])
                    nv.pack_into(torch.from_numpy(w2).cuda(), self.c2[e], self.s2[e],
                                 self.g2[e:e + 1])
        ws13, ws2 = workloads.moe_shared_weights(4, 0, H, self.IS)
        self.shared_host_w = (ws13, ws2)
        self.shared = (*nv.pack(torch.from_numpy(ws13).cuda()),
                       *nv.pack(torch.from_numpy(ws2).cuda()))
        self.routed = (self.c13, self.s13, self.g13, self.c2, self.s2, self.g2)
        torch.cuda.synchronize()

    def batches(self, M, nb=16):
        out = []
        for b in range(nb):
            ids, gw = self.wl.moe_routing(4, b, M, self.E, self.TOPK)
            xb = self.wl.x_bf16(4, b, 0, M, self.H)
            out.append((self.torch.from_numpy(ids).cuda(), self.torch.from_numpy(gw).cuda(),
                        x_dev(self.torch, xb), len(set(ids.ravel().tolist())), ids, gw, xb))
        return out

    def host_stacks(self, ids):
        """Oracle packs of the experts `ids` names (the rest zero, g = 1),
        each regenerated from its seeded stream: the oracle's input, built
        without the GPU."""
        E, H, I = self.E, self.H, self.I
        hc13 = np.zeros((E, 2 * I, H // 2), np.uint8)
        hs13 = np.zeros((E, 2 * I, H // 16), np.uint8)
        hg13 = np.ones(E, np.float32)
        hc2 = np.zeros((E, H, I // 2), np.uint8)
        hs2 = np.zeros((E, H, I // 16), np.uint8)
        hg2 = np.ones(E, np.float32)
        for e in sorted(set(int(v) for v in np.ravel(ids) if 0 <= v < E)):
            w13, w2 = self.wl.moe_expert_weights(4, 0, e, H, I)
            hc13[e], hs13[e], hg13[e] = _oracle().pack(w13)
            hc2[e], hs2[e], hg2[e] = _oracle().pack(w2)
        return hc13, hs13, hg13, hc2, hs2, hg2

    def host_shared(self):
        ws13, ws2 = self.shared_host_w
        return (*_oracle().pack(ws13), *_oracle().pack(ws2))


def moe_legs(torch, nv, traffic, mo, M, steps, warmup, ceil, want_cpu):
    """The routed MoE pass at M tokens, the same with the shared expert, and
    the W4A4 routed experts with the W4A16 shared expert."""
    E, H, I, topk, Is = mo.E, mo.H, mo.I, mo.TOPK, mo.IS
    bt = mo.batches(M)
    nb = len(bt)
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")

    def mean_bytes(fn, first, n):
        return float(np.mean([fn(bt[(first + i) % nb][3]) for i in range(n)]))

    def run(step, fn, label, launches):
        # bytes of the steps timed by the launch window (each step's own
        # distinct-expert count)
        first = warmup + steps + LAUNCH_WINDOW
        nbytes = mean_bytes(fn, first, QUEUED_WINDOW)
        out = {"workload": label, "M": M, "rotating_batches": nb,
               "distinct_experts_mean": mean_bytes(lambda d: d, first, QUEUED_WINDOW),
               **measure(torch, HOLD, step, steps, warmup, nbytes, M, launches, ceil.us(nbytes))}
        return out

    # host stacks for the parity batch (batch 0): routed experts + shared
    ids0, gw0, xb0 = bt[0][4], bt[0][5], bt[0][6]
    log(f"[bench] moe M={M}: oracle packs of the {bt[0][3]} experts of batch 0")
    hw = mo.host_stacks(ids0)
    hsh = mo.host_shared()

    ws = torch.empty(nv.moe_workspace_bytes(M, H, I, topk), dtype=torch.uint8, device="cuda")

    def step(i):
        ids, gw, x = bt[i % nb][:3]
        nv.moe_gemv_into(*mo.routed, x, ids, gw, y, ws)

    routed = run(step, lambda d: traffic.moe_bytes(M, H, I, topk, d),
                 f"moe_288x(3072x4096,4096x1536)_top8_m{M}", 2)
    step(0)
    yr, bound = _oracle().moe(*hw, xb0, ids0, gw0)
    w, b = tol_ratio(y.cpu().numpy(), yr, bound)
    routed["parity"] = {"batch": 0, "outputs": int(yr.size), "max_err_over_tol": w,
                        "outside_tol": b, "ok": b == 0}
    if want_cpu:
        D0 = bt[0][3]
        # the oracle loops over (token, slot): one token is 1/M of its work
        routed["cpu"] = cpu_baseline(lambda: _oracle().moe(*hw, xb0, ids0, gw0),
                                     traffic.moe_bytes(M, H, I, topk, D0), M,
                                     f"the whole pass of batch 0 ({D0} experts)",
                                     lambda: _oracle().moe(*hw, xb0[:1], ids0[:1], gw0[:1]),
                                     1.0 / M)

    wss = torch.empty(nv.moe_shared_workspace_bytes(M, H, I, topk, Is), dtype=torch.uint8,
                      device="cuda")

    def step_shared(i):
        ids, gw, x = bt[i % nb][:3]
        nv.moe_shared_gemv_into(*mo.routed, x, ids, gw, mo.shared, y, wss)

    with_shared = run(step_shared, lambda d: traffic.moe_shared_bytes(M, H, I, topk, d, Is),
                      f"moe_288x(3072x4096,4096x1536)_top8_shared768_m{M}", 2)
    step_shared(0)
    yr, bound = _oracle().moe_shared(*hw, xb0, ids0, gw0, hsh)
    w, b = tol_ratio(y.cpu().numpy(), yr, bound)
    with_shared["parity"] = {"batch": 0, "outputs": int(yr.size), "max_err_over_tol": w,
                             "outside_tol": b, "ok": b == 0}

    # W4A4 routed experts: static input scales for x and h, calibrated on
    # another batch of the same distributions (batch nb, never timed)
    xc = mo.wl.x_bf16(4, nb, 0, M, H)
    gx_v = np.float32(np.abs((xc.astype(np.uint32) << 16).view(np.float32)).max() / 2688.0)
    idc, gwc = mo.wl.moe_routing(4, nb, M, E, topk)
    hwc = mo.host_stacks(idc)
    _, _, hcal = _oracle().moe(*hwc, xc, idc, gwc, want_h=True)
    hcal_f = (hcal.astype(np.uint32) << 16).view(np.float32)
    gh_v = np.float32(np.abs(hcal_f).max() / 2688.0)
    del hwc
    gx = torch.tensor([gx_v], dtype=torch.float32, device="cuda")
    gh = torch.tensor([gh_v], dtype=torch.float32, device="cuda")
    wsq = torch.empty(nv.moe_w4a4_workspace_bytes(M, H, I, topk, Is), dtype=torch.uint8,
                      device="cuda")

    def step_w4a4(i):
        ids, gw, x = bt[i % nb][:3]
        nv.moe_w4a4_gemv_into(*mo.routed, x, gx, gh, ids, gw, y, wsq, shared=mo.shared)

    w4a4 = run(step_w4a4, lambda d: traffic.moe_w4a4_bytes(M, H, I, topk, d, Is),
               f"moe_w4a4_288x(3072x4096,4096x1536)_top8_shared768_m{M}", 3 if M == 1 else 4)
    step_w4a4(0)
    yq = y.cpu().numpy()
    yr, bound, _, hc, hs = _oracle().moe_w4a4(*hw, xb0, ids0, gw0, gx_v, gh_v, shared=hsh)
    # tokens whose h landed on the same NVFP4 grid values as the oracle's must
    # be within tolerance; a token whose gate|up sum (fp32 here, fp64 in the
    # oracle) rounded one bf16 ulp across a grid decision may differ more
    lay = nv.moe_w4a4_workspace_layout(M, H, I, topk, Is)
    hq = wsq[lay["hq"]:lay["hq"] + M * topk * I * 2].view(torch.int16).cpu().numpy()
    hq = hq.view(np.uint16).reshape(M, topk, I)
    hq_ref = _oracle_hq_bits(hc, hs).reshape(M, topk, I)
    valid = (ids0 >= 0) & (ids0 < E)
    same_tok = np.array([np.array_equal(hq[m][valid[m]], hq_ref[m][valid[m]])
                         for m in range(M)])
    r = np.abs(yq.astype(np.float64) - yr) / (1e-3 * bound + 1e-6)
    w = float(r[same_tok].max()) if same_tok.any() else 0.0
    b = int((~(r[same_tok] <= 1.0)).sum())
    w4a4["parity"] = {"batch": 0, "outputs": int(yr.size), "tokens_with_equal_h_grid":
                      int(same_tok.sum()), "max_err_over_tol_equal_h_grid": w,
                      "outside_tol_equal_h_grid": b,
                      "max_err_over_tol_all": float(r.max()), "ok": b == 0}
    return routed, with_shared, w4a4


def skewed_routing(ids, case, b, E):
    """Skewed variants of a routing batch (ids int32[M, topk]): case
    "one_expert_all_tokens" puts expert b % E in slot 0 of every token (the
    token's other slots keep their distinct experts); "same_experts_all_tokens"
    has every token name the same topk experts, each token in its own order."""
    M, topk = ids.shape
    r = np.random.default_rng(1000 + b)
    if case == "one_expert_all_tokens":
        e0 = b % E
        out = np.empty_like(ids)
        for m in range(M):
            rest = [int(e) for e in ids[m] if e != e0][:topk - 1]
            while len(rest) < topk - 1:
                c = int(r.integers(0, E))
                if c != e0 and c not in rest:
                    rest.append(c)
            out[m] = [e0] + rest
        return out.astype(np.int32)
    base = (topk * b + np.arange(topk)) % E
    return np.stack([r.permutation(base) for _ in range(M)]).astype(np.int32)


def moe_skew_legs(torch, nv, traffic, mo, steps, warmup, ceil,
                  cases=("one_expert_all_tokens", "same_experts_all_tokens")):
    """The routed MoE pass at M = 8 under skewed routing (skewed_routing):
    the weights each distinct expert contributes are what the bytes count, so
    a pass that re-read a shared expert's rows per token would show here as
    a lower fraction of the read ceiling. Parity on batch 0 of each case."""
    E, H, I, topk, M = mo.E, mo.H, mo.I, mo.TOPK, 8
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(nv.moe_workspace_bytes(M, H, I, topk), dtype=torch.uint8, device="cuda")
    out = {}
    for case in cases:
        bt = []
        for b in range(16):
            ids, gw = mo.wl.moe_routing(4, 100 + b, M, E, topk)
            ids = skewed_routing(ids, case, b, E)
            xb = mo.wl.x_bf16(4, 100 + b, 0, M, H)
            bt.append((torch.from_numpy(ids).cuda(), torch.from_numpy(gw).cuda(),
                       x_dev(torch, xb), len(set(ids.ravel().tolist())), ids, gw, xb))
        nb = len(bt)

        def step(i, bt=bt):
            ids, gw, x = bt[i % nb][:3]
            nv.moe_gemv_into(*mo.routed, x, ids, gw, y, ws)

        first = warmup + steps + LAUNCH_WINDOW
        ds = [bt[(first + i) % nb][3] for i in range(QUEUED_WINDOW)]
        nbytes = float(np.mean([traffic.moe_bytes(M, H, I, topk, d) for d in ds]))
        res = {"workload": f"moe_288x(3072x4096,4096x1536)_top8_m8_{case}", "M": M,
               "rotating_batches": nb, "distinct_experts_mean": float(np.mean(ds)),
               **measure(torch, HOLD, step, steps, warmup, nbytes, M, 2, ceil.us(nbytes))}
        ids0, gw0, xb0 = bt[0][4], bt[0][5], bt[0][6]
        hw = mo.host_stacks(ids0)
        step(0)
        yr, bound = _oracle().moe(*hw, xb0, ids0, gw0)
        w, bo = tol_ratio(y.cpu().numpy(), yr, bound)
        res["parity"] = {"batch": 0, "outputs": int(yr.size), "max_err_over_tol": w,
                         "outside_tol": bo, "ok": bo == 0}
        del hw
        out[case] = res
    return out


def _oracle_hq_bits(hc, hs):
    """bf16 bits of e2m1 * s for quantized rows (codes [R, I/2], scales
    [R, I/16]) from the oracle's element tables: the values the kernel's
    quantizer writes to the workspace."""
    o = _oracle()
    e2 = np.array([o.e2m1_value(c) for c in range(16)], np.float64)
    e4 = np.array([o.e4m3_value(b) for b in range(256)], np.float64)
    lo, hi = hc & 0xF, hc >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(hc.shape[0], -1)
    vals = e2[codes] * np.repeat(e4[hs], 16, axis=1)
    return np.array([o.bf16_from_double(v) for v in vals.ravel()],
                    np.uint16).reshape(vals.shape)


# ------------------------------------------------------------------- w4a4

def leg_w4a4(torch, nv, workloads, traffic, steps, warmup, ceil, want_cpu):
    """The pages' W4A4 dense FFN (gate, up, down 4096x4096 at M=2): one step =
    quantizing the activations with a static input scale and the three W4A4
    GEMVs on them, gate|up as one multi-projection call."""
    wl = workloads.WORKLOADS[6]
    M = wl["M"]
    mats, host = [], []
    for i, (name, N, K) in enumerate(wl["mats"]):
        log(f"[bench] w4a4: packing {name} {N}x{K}")
        W = workloads.dense_weights(6, 0, i, N, K)
        mats.append((nv.pack(torch.from_numpy(W).cuda()), N, K))
        host.append(_oracle().pack(W))
        del W
    K = wl["mats"][0][2]
    wb = sum(traffic.weight_bytes(N, K) for _, N, K in mats)
    reps = max(2, (1 << 30) // wb + 1)
    copies = [mats] + [[(tuple(t.clone() for t in p), N, K) for p, N, K in mats]
                       for _ in range(reps - 1)]
    xb = workloads.x_bf16(6, 0, 0, M, K)
    x = x_dev(torch, xb)
    calib = workloads.x_bf16(6, 1, 0, M, K)
    gx_v = np.float32(np.abs(((calib.astype(np.uint32) << 16).view(np.float32))).max() / 2688.0)
    gx = torch.tensor([gx_v], dtype=torch.float32, device="cuda")
    cx, sx = nv.quantize_act(x, gx)
    ws = torch.empty(nv.gemv_w4a4_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, N, _ in mats]

    def step(i):
        nv.quantize_act_into(x, gx, cx, sx)
        cp = copies[i % reps]
        nv.gemv_w4a4_segments_into([cp[0][0], cp[1][0]], cx, sx, gx, ys[:2], ws)
        nv.gemv_w4a4_into(*cp[2][0], cx, sx, gx, ys[2], ws)

    nbytes = traffic.quantize_act_bytes(M, K) + sum(traffic.gemv_w4a4_bytes(M, N, K)
                                                    for _, N, K in mats)
    out = {"workload": "w4a4_ffn_m2 (gate, up, down 4096x4096; static input scale)", "M": M,
           "rotate_copies": reps,
           **measure(torch, HOLD, step, steps, warmup, nbytes, M, 1 + (1 if M <= 2 else 2) * 2,
                     ceil.us(nbytes))}
    step(0)
    torch.cuda.synchronize()
    hcx, hsx = _oracle().quantize_act(xb, gx_v)
    q_ok = bool(np.array_equal(cx.cpu().numpy(), hcx) and np.array_equal(sx.cpu().numpy(), hsx))
    worst, bad, n = 0.0, 0, 0
    for (c, s, g), yy in zip(host, ys):
        yr, ad = _oracle().gemv_w4a4(c, s, g, hcx, hsx, gx_v)
        w, b = tol_ratio(yy.cpu().numpy(), yr, ad)
        worst, bad, n = max(worst, w), bad + b, n + yr.size
    out["parity"] = {"quantize_bit_exact": q_ok, "outputs": n, "max_err_over_tol": worst,
                     "outside_tol": bad, "ok": q_ok and bad == 0}
    return out


# ------------------------------------------------------------------- copy

def leg_copy(torch, steps, warmup):
    """Calibration for the HBM byte counters: a plain fp32 copy kernel
    (dst = src * 1) of known size, 512 MiB read and 512 MiB written per
    launch, two buffer pairs alternating so the MALL cannot serve repeats."""
    n = (512 << 20) // 4
    bufs = [(torch.ones(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(2)]

    def step(i):
        src, dst = bufs[i % 2]
        torch.mul(src, 1.0, out=dst)

    timed_steps(torch, step, steps, warmup)
    us, _ = launch_window(torch, step, warmup + steps, 50)
    return {"bytes_read": n * 4, "bytes_written": n * 4, "us": us,
            "gbs": 2 * n * 4 / (us * 1e-6) / 1e9}


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
        bare = name.replace("(anonymous namespace)::", "")
        short = bare.split("(")[0] if bare.startswith(("nvfp4", "void nvfp4")) else name[:90]
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
                short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--legs", default=ALL_LEGS,
                    help="comma list of lm_head (the headline, config 3), small (config 1), "
                         "stress (config 5), layer (config 2), moe (config 4 with the shared "
                         "expert and W4A4 variants), w4a4 (the W4A4 dense FFN), wide (the LM "
                         "head at M=8 and the stress pair at M=16 and M=128), copy (a plain "
                         "copy kernel: the byte-counter calibration)")
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
    unknown = set(legs) - set(ALL_LEGS.split(",")) - set(EXTRA_LEGS.split(","))
    if unknown:
        ap.error(f"unknown legs {sorted(unknown)}")
    want_cpu = not args.no_cpu_baseline
    K_, W_ = args.steps, args.warmup
    props = torch.cuda.get_device_properties(0)
    global HOLD
    HOLD = BusyHold(torch, nv)
    ceil = ReadCeiling(torch, nv, HOLD)
    result = {
        "metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K_,
        "warmup": W_, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "lm_head_m1_151936x4096", "M": 1, "N": 151936, "K": 4096,
                   "weights": "nvfp4 g16 from N(0,0.02) fp32, packed on the GPU",
                   "x": "bf16 N(0,1)", "y": "fp32"},
    }
    configs = {}
    if "lm_head" in legs:
        D = Dense(torch, nv, workloads, traffic, 3, workloads.WORKLOADS[3]["mats"], 1)
        lm = dense_leg(torch, nv, D, K_, W_, ceil, want_cpu, "lm_head_m1_151936x4096")
        lm["parity"]["pack_bit_exact"] = D.pack_exact()
        lm["parity"]["ok"] = lm["parity"]["ok"] and lm["parity"]["pack_bit_exact"]
        configs["3_lm_head_m1"] = lm
        result["value"] = lm["gbs_wall"]
        result["ms_per_step"] = lm["ms_per_step"]
        result["tokens_per_s"] = lm["tokens_per_s"]
        result["frac_of_peak_wall"] = lm["gbs_wall"] / HBM_PEAK_GBS
        result["roofline"] = {
            "bound": "hbm", "achieved": lm["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": lm["frac_of_peak"], "traffic": read_traffic(), "kernel": LM_KERNEL,
            "kernel_avg_us": lm["step_us"],
            "basis": lm["step_us_basis"] + ": HIP events on the launch stream around a "
                     "fixed window of launches, independent of --steps",
            "kernel_avg_us_event_window": lm["window_us"],
            "event_window_launches": LAUNCH_WINDOW,
            "bytes_per_launch": lm["bytes_per_step"],
            "frac_of_read_ceiling": lm["frac_of_read_ceiling"]}
        result["config"]["rotate_copies"] = lm["rotate_copies"]
        result["parity"] = lm["parity"]
        if "cpu" in lm:
            result["cpu_baseline"] = lm["cpu"]
        del D
    if "small" in legs:
        D = Dense(torch, nv, workloads, traffic, 1, workloads.WORKLOADS[1]["mats"], 1)
        configs["1_gemv_m1_1024x4096"] = dense_leg(torch, nv, D, K_, W_, ceil, want_cpu,
                                                   "gemv_m1_1024x4096 (launch-bound)")
        del D
    if "stress" in legs:
        D = Dense(torch, nv, workloads, traffic, 5, workloads.WORKLOADS[5]["mats"], 8)
        configs["5_stress_m8"] = dense_leg(torch, nv, D, K_, W_, ceil, want_cpu,
                                           "stress_m8_t3 (12288x4096 + 4096x12288)")
        del D
    if "layer" in legs:
        D = Dense(torch, nv, workloads, traffic, 2, workloads.DECODE_LAYER, 5)
        lay = dense_leg(torch, nv, D, K_, W_, ceil, want_cpu,
                        "decode_layer_m5 (q,k,v,o 4096/1024 x 4096; gate, up 12288x4096; "
                        "down 4096x12288), seven calls")
        lay["fused"] = dense_leg(torch, nv, D, K_, W_, ceil, False,
                                 "decode_layer_m5, q|k|v and gate|up fused: four launches",
                                 segments=[(0, 1, 2), (3,), (4, 5), (6,)])
        configs["2_decode_layer_m5"] = lay
        del D
    skew_cases = tuple(c for leg, c in (("moe_skew_one", "one_expert_all_tokens"),
                                        ("moe_skew_same", "same_experts_all_tokens"))
                       if "moe_skew" in legs or leg in legs)
    if "moe" in legs or skew_cases:
        mo = Moe(torch, nv, workloads)
        if "moe" in legs:
            result["moe_shared"], result["moe_w4a4"] = {}, {}
            for M in (1, 8):
                routed, with_shared, w4a4 = moe_legs(torch, nv, traffic, mo, M, K_, W_, ceil,
                                                     want_cpu)
                configs[f"4_moe_m{M}"] = routed
                result["moe_shared"][f"m{M}"] = with_shared
                result["moe_w4a4"][f"m{M}"] = w4a4
        if skew_cases:
            result["moe_skew"] = moe_skew_legs(torch, nv, traffic, mo, K_, W_, ceil, skew_cases)
        del mo
    if "w4a4" in legs:
        result["w4a4_ffn_m2"] = leg_w4a4(torch, nv, workloads, traffic, K_, W_, ceil, want_cpu)
    if "wide" in legs:
        wide = {}
        if nv.MAX_M >= 8:
            D = Dense(torch, nv, workloads, traffic, 3, workloads.WORKLOADS[3]["mats"], 8,
                      xs_per_mat=False)
            wide["lm_head_m8"] = dense_leg(torch, nv, D, K_, W_, ceil, False,
                                           "lm_head_m8_151936x4096")
            del D
        for M in (16, 128):
            if nv.MAX_M >= M:
                D = Dense(torch, nv, workloads, traffic, 5, workloads.WORKLOADS[5]["mats"], M)
                leg = dense_leg(torch, nv, D, K_, W_, ceil, False,
                                f"stress_m{M}_t3 (12288x4096 + 4096x12288)")
                flops = sum(2 * M * N * K for _, N, K in D.mats)
                leg["tflops"] = flops / (leg["step_us"] * 1e-6) / 1e12
                leg["frac_of_bf16_mfma_peak"] = leg["tflops"] / BF16_MFMA_PEAK_TFLOPS
                # which roof binds: the weight bytes at the HBM peak or the
                # bf16 products at the dense matrix-core peak
                hbm_us = leg["bytes_per_step"] / (HBM_PEAK_GBS * 1e3)
                mfma_us = flops / (BF16_MFMA_PEAK_TFLOPS * 1e6)
                leg["roof"] = {"hbm_us": hbm_us, "mfma_us": mfma_us,
                               "bound": "mfma" if mfma_us > hbm_us else "hbm",
                               "frac_of_bound": max(hbm_us, mfma_us) / leg["step_us"]}
                wide[f"stress_m{M}"] = leg
                del D
        result["wide"] = wide
    if "copy" in legs:
        result["copy_calibration"] = leg_copy(torch, min(K_, 50), min(W_, 5))
    result["configs"] = configs
    result["read_ceiling"] = ceil.table()
    result["parity_ok_all"] = all(
        v["parity"]["ok"] for v in list(configs.values()) +
        [result.get("w4a4_ffn_m2") or {"parity": {"ok": True}}] +
        list((result.get("moe_shared") or {}).values()) +
        list((result.get("moe_w4a4") or {}).values()) +
        list((result.get("moe_skew") or {}).values()) +
        list((result.get("wide") or {}).values()) if "parity" in v)
    result["env"] = {"gpu": props.name, "cus": props.multi_processor_count,
                     "dpm_clocks": gpu_clock_state(),
                     "hip": torch.version.hip, "torch": torch.__version__, "git": git_sha(),
                     "library_sources_sha256_16": library_source_hash(),
                     "oracle_threads": oracle_threads(), "cpu": cpu_model(),
                     "argv": sys.argv[1:]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
