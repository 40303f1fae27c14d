#!/usr/bin/env python3
"""Throughput of the S4 filter path on one MI355X (gfx950).

A step is one call of ssm_forward on one batch of synthetic input: root values
by the Cauchy/Woodbury kernel, inverse transform to the kernel and its
convolution spectra, and the fused FFT convolution y = K * u + D u.  The
truncated-output vector C~ is formed once beforehand by ssm_discretize, off the
timer (the pages count filter evaluation from a supplied C~); its time is
reported separately.  All inputs are resident in HBM before timing starts.

Prints one JSON line: the headline metric (channel-steps/s = Bsz*H*L per
second), the roofline of the dominant kernel measured live with HIP events on
the launch stream, and the complex128 CPU oracle timed on a bounded sample on
this host.  --gpus N > 1 exits: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "channel-steps/sec (B·H·L) for S4 kernel-gen+FFT conv; % HBM/VALU roofline"
UNIT = "channel-steps/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X FP32: dense matrix (MFMA) and vector peaks are both 157.3
PEAK_FP64_TFLOPS = 78.6        # MI355X FP64 vector
PEAK_FP16_TFLOPS = 2500.0      # MI355X dense FP16 matrix (no sparsity)
DEFAULT_WORKLOAD = "s4-h1k-l16k"   # the largest workload: most channel-steps and bytes

KERNEL_SOURCES = {
    "filter": ["single_launch.hip", "roots.hpp", "fft.hpp", "common.hpp"],
    "cauchy": ["cauchy.hip", "roots.hpp", "wfft.hpp", "common.hpp"],
    "spectrum": ["wconv.hip", "wlarge.hip", "multipass.hip", "spectrum_conv.hip", "wfft.hpp", "fft.hpp",
                 "common.hpp"],
    "conv": ["wconv.hip", "wlarge.hip", "spectrum_conv.hip", "wfft.hpp", "fft.hpp", "common.hpp"],
}


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "structured_state_space_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def split_kernel(N, r, M):
    """Whether the root values run the split-precision kernel with its far form
    (the library's own rule: ranks 2 and 3; rank 1 from 128 states and 4096 roots)."""
    return r in (2, 3) or (r == 1 and N >= 128 and M >= 4096)


def algorithmic(w, M, fused):
    """Per-launch algorithmic work of each kernel (definitions in the design notes).
    fused: the kernel transform runs inside the convolution, which then reads
    the root values instead of the spectra."""
    H, N, r, L, B = w.H, w.N, w.r, w.L, w.Bsz
    roots = M - 1 if M >= 2 else M                      # z = -1 takes its finite formula
    out = {
        # the split-precision kernel (split_kernel) is bound by the vector ALU
        # (forming and splitting the Cauchy entries); the other rank-1 and the
        # rank-4 shapes run the float32 matrix-core kernel.  Both rated on the
        # same per-term flops against 157.3 TFLOP/s (the FP32 vector and FP32
        # dense matrix peaks coincide).
        "cauchy": dict(bound="alu" if split_kernel(N, r, M) else "mfma", unit="TFLOP/s",
                       work=H * roots * N * (8 * (r + 1) ** 2 + 7), scale=1e-12, peak=PEAK_FP32_TFLOPS),
        # the root values read, one spectrum of M complex written per channel
        "spectrum": dict(bound="hbm", unit="GB/s", work=H * M * 8 + H * M * 8, scale=1e-9, peak=PEAK_HBM_GBS),
        "conv": dict(bound="hbm", unit="GB/s", work=8 * B * H * L + 4 * H * L + 4 * H, scale=1e-9,
                     peak=PEAK_HBM_GBS),
    }
    if fused:
        del out["spectrum"]
        out["conv"]["work"] = 8 * B * H * L + 8 * H * M + 4 * H
    return out


def wave_freq(logm, pos):
    """Frequency index held at each output position of the wave-structured
    transforms' scrambled order (M = 2^logm >= 1024; M = P 16384 in slices)."""
    lq = min(logm, 14)
    q = pos & ((1 << lq) - 1)
    logw = lq - 10
    sb = 4 - logw
    wave, e, lane = q >> 10, (q >> 6) & 15, q & 63
    rb = ((lane >> 4) & 3) | (((lane >> 2) & 3) << 2)
    k = ((rb & ((1 << sb) - 1)) | (wave << sb)) + 16 * ((rb >> sb) + (1 << logw) * ((lane & 3) + 4 * e))
    return k if logm <= 14 else (k << (logm - 14)) + (pos >> 14)


def root_value_terms(p, M, scrambled):
    """Terms the rank-2/3 root-value kernel sums per launch, by its own rule: a
    wave of 64 consecutive output positions whose roots s = i a tan(pi k/M) all
    lie at |s - c| >= 2^0.6 R from the channel's pole centre c (R the pole radius)
    sums J = 8 nfb moment terms per root, nfb = 1..5 (the fewest with
    |v|^J <= 2^-24, v = R/(s - c)); any other wave sums the N states.  Returns
    (terms over the M - 1 roots != -1, fraction of those roots in far waves)."""
    pos = np.arange(M)
    k = wave_freq(int(math.log2(M)), pos) if scrambled else pos
    t = np.tan(np.pi * k / M)
    t[2 * k == M] = 0.0
    pos_m1 = 512 if scrambled else M // 2
    counted = np.ones(M, dtype=bool)
    counted[pos_m1] = False
    pad = (-M) % 64
    terms, far_roots = 0, 0
    for h in range(p.H):
        lam = p.Lambda[h].astype(np.complex128)
        c = lam.mean()
        R = float(np.sqrt(np.max((lam.real - c.real) ** 2 + (lam.imag - c.imag) ** 2)))
        if not (1e-30 <= R <= 1e30):
            R = 0.0
        cx, cy, rf = np.float32(c.real), np.float32(c.imag), np.float32(R)
        st = (2.0 / float(np.float32(p.dt[h])) * t).astype(np.float32)
        d = np.hypot(cx, (st - cy).astype(np.float32)).astype(np.float32)
        ratios = np.float32([8.0, 2.8284271, 2.0, 1.6817928, 1.5157166])  # 2^(3/nfb)
        far = (rf > 0) & (d >= ratios[-1] * rf)
        lv = 1 + sum((~(d >= q * rf)).astype(int) for q in ratios[:-1])
        far = np.concatenate([far | ~counted, np.ones(pad, bool)]).reshape(-1, 64).all(1)
        lv = np.concatenate([np.where(counted, lv, 0), np.zeros(pad, int)]).reshape(-1, 64).max(1)
        cnt = np.concatenate([counted, np.zeros(pad, bool)]).reshape(-1, 64).sum(1)
        terms += int(np.sum(np.where(far, 8 * lv, p.N) * cnt))
        far_roots += int(np.sum(cnt[far]))
    return terms, far_roots / (p.H * (M - 1))


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, scaled by
    the copy-kernel calibration; None when absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    def val(key):
        m = re.search(rf"^{key}:\s*([0-9.eE+-]+|[0-9a-f]+)\s*$", text, re.M)
        return m.group(1) if m else None
    if val("source_sha") != source_hash(kernel):
        return None
    try:
        fetch = float(val("fetch_kib_per_dispatch")) * float(val("copy_scale_fetch"))
        write = float(val("write_kib_per_dispatch")) * float(val("copy_scale_write"))
    except (TypeError, ValueError):
        return None
    return (fetch + write) * 1024.0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_workers():
    """Worker processes for the CPU baseline: the cores this process may run
    on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


_CPU_JOB = {}


def _cpu_worker(args):
    """One worker: whole channels of the shard, one BLAS thread, until the time
    budget is spent (at least one channel)."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    chans, seconds = args
    p, u = _CPU_JOB["p"], _CPU_JOB["u"]
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        for h in chans:
            c = p.channel(int(h))
            O.channel_reference(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], c["D"], u[:, int(h), :], p.L)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
    return done, time.perf_counter() - t0


def cpu_baseline(w, p, u, seconds):
    """The oracle as it stands on this host's cores: one worker process per
    core (one BLAS thread each), channels sharded round-robin, each worker
    stopping after about `seconds`.  Runs before the GPU is touched, so the
    workers are plain forks of a process with no device state."""
    import multiprocessing as mp

    nw = host_workers()
    shards = [list(range(i, w.H, nw)) for i in range(nw)]
    shards = [s for s in shards if s]
    _CPU_JOB.update(p=p, u=u)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(shards)) as pool:
        res = pool.map(_cpu_worker, [(s, seconds) for s in shards])
    wall = time.perf_counter() - t0
    _CPU_JOB.clear()
    chans = sum(d for d, _ in res)
    busy = max(t for _, t in res)
    return {"value": chans * w.Bsz * w.L / busy, "unit": UNIT, "cores": len(shards), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{chans} of {w.H} channels x {w.Bsz} rows x {w.L} steps of workload {w.name} on "
                      f"{len(shards)} worker processes (one BLAS thread each, channels sharded round-robin, each "
                      f"worker stopping after ~{seconds:.0f} s): complex128 dense discretisation, kernel by matrix "
                      f"iteration, time-stepped recurrence; rate = channel-steps done / longest worker time "
                      f"({busy:.1f} s; {wall:.1f} s wall with pool start-up)"}


STEP_METRIC = "channel-steps/sec (B·H·T) for the S4 recurrent step mode; % FP32 roofline"


def step_flops(w):
    """Algorithmic flops of one ssm_step call over T = L steps: per (sequence,
    step, state) the r sums Q^* D^{-1} x and C^* x (8 flops per complex
    multiply-add), D^{-1} x (6), the rank-r correction (8 r) and the update
    2 g - x + Bbar u (8)."""
    return w.Bsz * w.H * w.L * w.N * (16 * w.r + 22)


def cpu_baseline_step(w, p, u, seconds):
    """The oracle's recurrence from a state, one thread, on a bounded channel sample."""
    from threadpoolctl import threadpool_limits

    import numpy as np
    import oracle as O
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while done < w.H and time.perf_counter() - t0 < seconds:
            c = p.channel(done)
            Abar, Bbar, _ = O.bilinear(O.dplr_matrix(c["Lambda"], c["P"], c["Q"]), c["B"], float(c["dt"]))
            for b in range(w.Bsz):
                O.recurrence_from(Abar, Bbar, c["C"], float(c["D"]), u[b, done, :], np.zeros(w.N, complex))
            done += 1
    dt = time.perf_counter() - t0
    return {"value": done * w.Bsz * w.L / dt, "unit": UNIT, "cores": 1, "kind": "oracle",
            "sample": f"{done} of {w.H} channels x {w.Bsz} rows x {w.L} steps of workload {w.name}: complex128 "
                      f"dense bilinear matrices, time-stepped recurrence ({dt:.1f} s, one thread)"}


def bench_step(args, w, p, u, dev):
    import torch

    from structured_state_space_amd import ssm
    d = ssm.to_device(p, dev)
    if args.decode == "only":  # short calls alone (a kernel trace of them stays apart from the long calls)
        prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
        print(json.dumps({"metric": "microseconds per streaming-decode call from a HIP graph", "unit": "us",
                          "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
                          "config": {"workload": w.name, "op": "step", "H": w.H, "N": w.N, "r": w.r, "batch": w.Bsz},
                          "decode_us_per_call_graph": decode_us(ssm, d, prep, u, w, dev)}))
        return 0
    ut = torch.from_numpy(u).to(dev)
    x = torch.zeros((w.Bsz, w.H, w.N), dtype=torch.complex64, device=dev)
    y = torch.empty_like(ut)
    status = torch.empty(w.H, dtype=torch.int32, device=dev)

    def call():
        ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], ut, x=x, y=y, status=status)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 100))  # one call covers L steps of every sequence
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_events = start.elapsed_time(end) / steps
    ms = max(ms_events, 1e3 * t_wall / steps)
    if int(status.abs().max()) != 0 or not bool(torch.isfinite(y).all()):
        raise RuntimeError("step mode produced a nonzero status or non-finite output")
    flops = step_flops(w)
    achieved = flops * 1e-12 / (ms_events * 1e-3)
    line = {
        "metric": STEP_METRIC, "value": w.Bsz * w.H * w.L / (ms * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "op": "step", "H": w.H, "N": w.N, "r": w.r, "T": w.L, "batch": w.Bsz},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_TFLOPS, "traffic": None, "kernel": "step"},
        "ms_per_step_events": ms_events,
    }
    # the two-call form: the set-up once, then only the recurrence per call,
    # in the layout the library picks (0) and in each fixed one
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    line["prepared"] = {}
    for lanes in ((0, 16, 64) if w.N <= 64 else (0, 64)):
        def call_prepared():
            ssm.step_prepared(prep, d["D"], ut, x=x, y=y, status=status, lanes=lanes)

        for _ in range(args.warmup):
            call_prepared()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            call_prepared()
        end.record()
        torch.cuda.synchronize()
        if int(status.abs().max()) != 0 or not bool(torch.isfinite(y).all()):
            raise RuntimeError("prepared step mode produced a nonzero status or non-finite output")
        key = "ms_per_call_events" if lanes == 0 else f"ms_per_call_events_lanes{lanes}"
        line["prepared"][key] = start.elapsed_time(end) / steps
    if args.decode == "graph":
        line["prepared"]["decode_us_per_call_graph"] = decode_us(ssm, d, prep, u, w, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_step(w, p, u, args.cpu_seconds)
    print(json.dumps(line))
    return 0


def decode_us(ssm, d, prep, u, w, dev, calls=50):
    """Streaming decode: microseconds per call of T = 1, 8 and 64 steps, for
    ssm_step and ssm_step_prepared, each captured `calls` times in one HIP
    graph and the graph replayed (launch overhead of the graph included)."""
    import torch
    x = torch.zeros((w.Bsz, w.H, w.N), dtype=torch.complex64, device=dev)
    st = torch.empty(w.H, dtype=torch.int32, device=dev)
    out = {}
    for T in (1, 8, 64):
        ut = torch.from_numpy(u[:, :, :T].copy()).to(dev)
        y = torch.empty_like(ut)
        fns = {"step": lambda: ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], ut, x=x, y=y,
                                        status=st),
               "prepared": lambda: ssm.step_prepared(prep, d["D"], ut, x=x, y=y, status=st)}
        for name, f in fns.items():
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                f()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(calls):
                    f()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            out[f"{name}_T{T}"] = e0.elapsed_time(e1) / calls * 1e3
            if int(st.abs().max()) != 0 or not bool(torch.isfinite(y).all()):
                raise RuntimeError(f"decode timing: {name} at T = {T} gave a nonzero status or non-finite output")
    return out


def bench_complex(args, w, p, u, dev):
    """ssm_forward_complex timed like the headline step; its roofline is that of
    the work it adds to ssm_forward, rated as a whole: the root values' flops
    at the FP32 peak plus twice the convolution's algorithmic bytes at the HBM
    peak (the phases are serial), over the measured step."""
    import torch

    from structured_state_space_amd import ssm
    d = ssm.to_device(p, dev)
    ut = torch.from_numpy(u).to(dev)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], w.L, want_bbar=False)["Ctilde"]
    nbytes = ssm.workspace_bytes(ssm.OP_FORWARD_COMPLEX, w.Bsz, w.H, w.N, w.r, w.L)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def call():
        return ssm.forward_complex(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], ut, workspace=ws)

    for _ in range(args.warmup):
        out = call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        out = call()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_events = start.elapsed_time(end) / args.steps
    ms = max(ms_events, 1e3 * t_wall / args.steps)
    if int(out["status"].abs().max()) != 0 or not bool(torch.isfinite(out["y_im"]).all()):
        raise RuntimeError("complex output produced a nonzero status or non-finite values")
    M = ssm.transform_lengths(w.L)[0]
    alg = algorithmic(w, M, False)
    troof_ms = (alg["cauchy"]["work"] / (PEAK_FP32_TFLOPS * 1e12) + 2 * alg["conv"]["work"] / (PEAK_HBM_GBS * 1e9)) * 1e3
    line = {
        "metric": "channel-steps/sec (B·H·L) for the S4 filter path with complex output", "unit": UNIT,
        "value": w.Bsz * w.H * w.L / (ms * 1e-3), "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": w.name, "op": "complex", "H": w.H, "N": w.N, "r": w.r, "L": w.L,
                                        "batch": w.Bsz},
        "composite_roofline_frac": troof_ms / ms, "ms_per_step_events": ms_events,
    }
    print(json.dumps(line))
    return 0


def bench_kernel_gen(args, w, p, dev):
    """ssm_kernel_gen (root values and the kernel K, no roots output) as whole
    calls on the workload's channels.  Rated on the root values' algorithmic
    flops alone (as the forward's root-value stage: the terms summed) over the
    whole call, so the kernel transform's time counts against it."""
    import torch

    from structured_state_space_amd import ssm
    d = ssm.to_device(p, dev)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], w.L, want_bbar=False)["Ctilde"]
    ws = torch.empty(ssm.workspace_bytes(ssm.OP_KERNEL_GEN, 1, w.H, w.N, w.r, w.L), dtype=torch.uint8, device=dev)

    def call():
        return ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], w.L, workspace=ws)

    for _ in range(args.warmup):
        out = call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        out = call()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_events = start.elapsed_time(end) / args.steps
    ms = max(ms_events, 1e3 * t_wall / args.steps)
    if int(out["status"].abs().max()) != 0 or not bool(torch.isfinite(out["K"]).all()):
        raise RuntimeError("kernel generation produced a nonzero status or non-finite values")
    M = ssm.transform_lengths(w.L)[0]
    alg = algorithmic(w, M, False)["cauchy"]
    if split_kernel(w.N, w.r, M):
        alg["work"] = root_value_terms(p, M, False)[0] * (8 * (w.r + 1) ** 2 + 7)
    achieved = alg["work"] * alg["scale"] / (ms * 1e-3)
    one_launch = M == 1024 and w.H >= 256
    line = {
        "metric": "kernel generations/sec (root values and K for every channel)", "unit": "calls/s",
        "value": 1e3 / ms, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "op": "kernel_gen", "H": w.H, "N": w.N, "r": w.r, "L": w.L, "M": M,
                   "launches": 1 if one_launch else 2},
        "roofline": {"bound": alg["bound"], "achieved": achieved, "peak": alg["peak"], "unit": alg["unit"],
                     "frac": achieved / alg["peak"], "traffic": None,
                     "work": "root values' algorithmic flops over the whole call"},
        "ms_per_step_events": ms_events,
    }
    print(json.dumps(line))
    return 0


HIPPO_METRIC = "HiPPO-to-DPLR constructions/sec (generator, eigenvectors, B and per-channel C)"


def hippo_flops(N, rows):
    """Algorithmic float64 flops of one construction: the tridiagonal reduction
    of the skew part (4 N^3 / 3, the symmetric count), applying the N - 2
    reflections to N complex vectors (4 N^3), and projecting `rows` input rows
    onto the eigenvectors (8 N^2 each); the O(N^2) eigenvalue and
    inverse-iteration work is left out."""
    return 4.0 * N ** 3 / 3.0 + 4.0 * N ** 3 + 8.0 * N * N * rows


def cpu_baseline_hippo(kind, N, theta, B, C, seconds):
    """The oracle's construction as it stands, one thread, repeated for about
    `seconds` (at least once)."""
    from threadpoolctl import threadpool_limits

    import oracle.hippo_oracle as HO
    n, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            HO.hippo_dplr(kind, N, theta, B, C)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": n / el, "unit": "constructions/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} oracle constructions ({kind}, N={N}, {C.shape[0]} C rows, complex128, library "
                      f"Hermitian eigensolver) in {el:.1f} s, one thread"}


def bench_hippo(args, w, dev):
    """ssm_hippo_dplr for the workload's state size N, with one B row and one C
    row per channel (H rows)."""
    import numpy as np
    import torch

    from structured_state_space_amd import ssm
    kind, N, H, theta = args.hippo_kind, w.N, w.H, 1.0
    rng = np.random.default_rng(7)
    Bn = ((rng.normal(size=(1, N)) + 1j * rng.normal(size=(1, N))) / np.sqrt(2)).astype(np.complex64)
    Cn = ((rng.normal(size=(H, N)) + 1j * rng.normal(size=(H, N))) / np.sqrt(2)).astype(np.complex64)
    B, C = torch.from_numpy(Bn).to(dev), torch.from_numpy(Cn).to(dev)
    ws = torch.empty(ssm.workspace_bytes(ssm.OP_HIPPO, 0, 0, N, 0, 0), dtype=torch.uint8, device=dev)

    def call():
        return ssm.hippo_dplr(kind, N, theta, B, C, workspace=ws)

    for _ in range(args.warmup):
        out = call()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 200))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(steps):
        out = call()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_events = start.elapsed_time(end) / steps
    ms = max(ms_events, 1e3 * t_wall / steps)
    if not all(bool(torch.isfinite(torch.view_as_real(out[k])).all()) for k in ("Lambda", "P", "Bt", "Ct")):
        raise RuntimeError("HiPPO construction produced non-finite values")
    achieved = hippo_flops(N, 1 + H) * 1e-12 / (ms_events * 1e-3)
    line = {
        "metric": HIPPO_METRIC, "value": 1e3 / ms, "unit": "constructions/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"hippo-{kind}-n{N}-h{H}", "op": "hippo", "N": N, "C_rows": H, "B_rows": 1},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP64_TFLOPS, "traffic": None, "kernel": "hippo (three launches)"},
        "ms_per_step_events": ms_events,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_hippo(kind, N, theta, Bn.astype(np.complex128),
                                                  Cn.astype(np.complex128), min(args.cpu_seconds, 10.0))
    print(json.dumps(line))
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--stage-repeat", type=int, default=10,
                    help="launches of each stage per timing bracket in the per-kernel measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", choices=("graph", "none", "only"), default="graph",
                    help="--op step: also time short decode calls from a HIP graph (graph), skip them (none), "
                         "or time only them (only)")
    ap.add_argument("--hippo-kind", choices=("legs", "legt", "lagt"), default="legs",
                    help="generator for --op hippo")
    ap.add_argument("--op", choices=("forward", "step", "complex", "hippo", "kernel_gen"), default="forward",
                    help="forward: the filter path (the headline); step: the recurrent step mode, "
                         "T = L steps of every sequence per call, the state carried between calls; "
                         "complex: the filter path with the imaginary output as well; "
                         "hippo: DPLR parameters of a HiPPO generator at the workload's N, one C row per channel; "
                         "kernel_gen: the kernel generator alone (root values and K)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the S4 filter path shards over channels with no exchange, "
              "and the benchmark measures the one-GPU share (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    cpu_line = None
    if args.op == "forward" and not args.no_cpu_baseline and not args.calibrate_copy:
        # the oracle on the host cores first: forked workers of a process that
        # has not touched the GPU yet
        from structured_state_space_amd import inputs as I
        w0, p0, u0 = I.workload(args.workload)
        cpu_line = cpu_baseline(w0, p0, u0, args.cpu_seconds)
        del w0, p0, u0

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 5}))
        return 0

    from structured_state_space_amd import inputs as I
    from structured_state_space_amd import ssm

    w, p, u = I.workload(args.workload)
    if args.op == "step":
        return bench_step(args, w, p, u, dev)
    if args.op == "complex":
        return bench_complex(args, w, p, u, dev)
    if args.op == "hippo":
        return bench_hippo(args, w, dev)
    if args.op == "kernel_gen":
        return bench_kernel_gen(args, w, p, dev)
    M, n_fft = ssm.transform_lengths(w.L)
    form = ssm.forward_form(w.Bsz, w.H, w.L)
    fused = form == 2
    d = ssm.to_device(p, dev)
    ut = torch.from_numpy(u).to(dev)

    # C~ once, off the timer
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], w.L, want_bbar=False)
    e1.record()
    torch.cuda.synchronize()
    discretize_ms = e0.elapsed_time(e1)
    if int(disc["status"].abs().max()) != 0:
        raise RuntimeError("discretisation reported a nonzero status")
    Ct = disc["Ctilde"]

    y = torch.empty_like(ut)
    status = torch.empty(w.H, dtype=torch.int32, device=dev)
    ws = torch.empty(ssm.workspace_bytes(ssm.OP_FORWARD, w.Bsz, w.H, w.N, w.r, w.L), dtype=torch.uint8,
                     device=dev)

    def step(events=None):
        ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], ut, y=y, status=status,
                    workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_events = start.elapsed_time(end) / args.steps
    ms_per_step = max(ms_events, 1e3 * t_wall / args.steps)
    if int(status.abs().max()) != 0 or not bool(torch.isfinite(y).all()):
        raise RuntimeError("forward produced a nonzero status or non-finite output")

    # per-kernel durations, live, on the launch stream: each stage launched
    # `repeat` times back to back between events (dispatch gaps amortised)
    stages = ("cauchy", "spectrum", "conv")
    acc = {k: 0.0 for k in stages}
    reps = max(1, args.stage_repeat)
    nprof = min(args.steps, 20)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nprof)]
    for i in range(nprof):
        ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], ut, y=y, status=status,
                    workspace=ws, events=evs[i], repeat=reps)
    torch.cuda.synchronize()
    for i in range(nprof):
        for j, k in enumerate(stages):
            acc[k] += evs[i][j].elapsed_time(evs[i][j + 1]) / reps
    phase_ms = {k: acc[k] / nprof for k in stages}
    # form 2: stage 2 launches nothing and the convolution kernel includes it;
    # form 1: one kernel does everything (timed as stage 1)
    names = ("filter",) if form == 1 else ("cauchy", "conv") if fused else stages
    if form == 1:
        phase_ms["filter"] = phase_ms["cauchy"]
    if M > 16384:
        # the repeated multi-pass kernel transform regenerates the root values each time
        phase_ms["spectrum"] -= phase_ms["cauchy"] * (reps - 1) / reps

    alg = algorithmic(w, M, fused)
    far_info = None
    if form != 1 and split_kernel(w.N, w.r, M):
        # the rank-2/3 kernel sums moment expansions for far waves: its
        # algorithmic flops are the same per-term figure over the terms it sums
        scrambled = M > 16384 or (not fused and M >= 1024)
        terms, far_frac = root_value_terms(p, M, scrambled)
        direct = alg["cauchy"]["work"]
        alg["cauchy"]["work"] = terms * (8 * (w.r + 1) ** 2 + 7)
        far_info = {"work_direct_sum": direct, "terms_per_root": terms / (w.H * (M - 1)),
                    "far_root_fraction": far_frac}
    if form == 1:
        # the single launch is compute-bound (root-value sums on the matrix cores,
        # transforms on the vector ALU): rated on the root values' flops plus the
        # convolution's transform flops, Bsz*H*(5 n log2 n + 6 (n/2 + 1)), n = n_fft
        conv_flops = w.Bsz * w.H * (5 * n_fft * int(math.log2(n_fft)) + 6 * (n_fft // 2 + 1))
        alg["filter"] = dict(alg["cauchy"], work=alg["cauchy"]["work"] + conv_flops)
    phases = {}
    for k in names:
        a = alg[k]
        achieved = a["work"] * a["scale"] / (phase_ms[k] * 1e-3)
        phases[k] = {"bound": a["bound"], "achieved": achieved, "peak": a["peak"], "unit": a["unit"],
                     "frac": achieved / a["peak"], "ms": phase_ms[k], "work_per_launch": a["work"]}
    if "conv" in phases:
        # the convolution sits near the ridge: its transform flops (FFTW
        # convention, n = n_fft) against the FP32 peak, beside its HBM rating
        conv_flops = w.Bsz * w.H * (5 * n_fft * int(math.log2(max(n_fft, 2))) + 6 * (n_fft // 2 + 1))
        tf = conv_flops * 1e-12 / (phase_ms["conv"] * 1e-3)
        phases["conv"]["transform_flops_per_launch"] = conv_flops
        phases["conv"]["transform_tflops"] = tf
        phases["conv"]["transform_frac_fp32"] = tf / PEAK_FP32_TFLOPS
    if far_info is not None and "cauchy" in phases:
        phases["cauchy"].update(far_info)
        phases["cauchy"]["direct_sum_equivalent_tflops"] = far_info["work_direct_sum"] * 1e-12 / (
            phase_ms["cauchy"] * 1e-3)
    if "cauchy" in phases and split_kernel(w.N, w.r, M):
        # the split-precision kernel's matrix-core side: three float16 products
        # of 32 x 32 x 16 per block of 8 states (or moment terms) and 32 roots
        # (32 columns, of which 2 (r+1)^2 are used), against the dense float16 peak
        blocks = far_info["terms_per_root"] / 8 if far_info is not None else (w.N + 7) // 8
        mf = 3 * 2 * 32 * 32 * 16 * w.H * M * blocks / 32
        phases["cauchy"]["matrix_core_flops_per_launch"] = mf
        phases["cauchy"]["matrix_core_frac_fp16"] = mf * 1e-12 / (phase_ms["cauchy"] * 1e-3) / PEAK_FP16_TFLOPS
    dom = max(names, key=lambda k: phase_ms[k])
    traffic = read_traffic(dom, w.name)
    roofline = {"bound": phases[dom]["bound"], "achieved": phases[dom]["achieved"], "peak": phases[dom]["peak"],
                "unit": phases[dom]["unit"], "frac": phases[dom]["frac"], "traffic": traffic, "kernel": dom}
    troof_ms = (alg["cauchy"]["work"] / (PEAK_FP32_TFLOPS * 1e12) + alg["conv"]["work"] / (PEAK_HBM_GBS * 1e9)) * 1e3
    # the whole step against its composite roofline: the root values' flops at
    # the FP32 peak plus the convolution's bytes at the HBM peak (serial phases)
    phases["composite"] = {"t_roof_ms": troof_ms, "ms": ms_per_step, "frac": troof_ms / ms_per_step}

    # the other entry points of the path as whole calls: the kernel alone
    # (root values and its transform) and the convolution with a given kernel
    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ws_kg = torch.empty(ssm.workspace_bytes(ssm.OP_KERNEL_GEN, 1, w.H, w.N, w.r, w.L), dtype=torch.uint8,
                        device=dev)
    ws_fc = torch.empty(ssm.workspace_bytes(ssm.OP_FFTCONV, w.Bsz, w.H, w.N, w.r, w.L), dtype=torch.uint8,
                        device=dev)
    Kbuf = torch.empty((w.H, w.L), dtype=torch.complex64, device=dev)
    y2 = torch.empty_like(ut)
    kg = lambda: ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], w.L, workspace=ws_kg)
    calls_ms = {"kernel_gen": timed(kg)}
    Kbuf.copy_(kg()["K"])
    calls_ms["fftconv"] = timed(lambda: ssm.fftconv(Kbuf, ut, d["D"], y=y2, workspace=ws_fc))

    value = w.Bsz * w.H * w.L / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "N": w.N, "r": w.r, "L": w.L, "M": M, "n_fft": n_fft,
                   "batch": w.Bsz, "launch_form": form},
        "roofline": roofline,
        "phases": phases,
        "composite_roofline_frac": troof_ms / ms_per_step,
        "ms_per_step_events": ms_events,
        "discretize_ms_off_timer": discretize_ms,
        "calls_ms_off_timer": calls_ms,
    }
    if cpu_line is not None:
        out["cpu_baseline"] = cpu_line
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
