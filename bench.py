#!/usr/bin/env python3
"""Benchmark of the weighted SiTU-GLU hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dense_ffn]

One step is one pass of the whole path over one batch: the forward kernel and
the backward kernel (with d_routing_weights where the workload asks for it),
inputs already resident in HBM.  The default workload is the largest bf16
forward + backward one, dense_ffn ([16384, 2 x 18432]); the routed and stress
workloads are timed in the same run and summarised under other_workloads.  The routed_top8_mxfp8 workload times the
forward with MXFP8 output instead (forward only); attn_res_mix times the
attention-residual mixing kernel; grouped_fc1_top8 (bf16 operands) and
grouped_fc1_top8_mxfp8 (MXFP8 operands) time the fused FC1 grouped GEMM +
SiTU-GLU (value and roofline in TFLOP/s against the matrix-core peak of the
operand type).  The step first runs for --settle-ms (the GPU's clocks ramp
up from idle), then W untimed steps, then K timed steps between two device
synchronisations.  Prints ONE JSON line:

  value        whole-step algorithmic HBM throughput, GB/s (10^9 B/s): the bytes
               the method must move (every input read once, every output
               written once) / wall time per step
  roofline     the dominant kernel (the backward) against the MI355X HBM peak
               (8 TB/s): algorithmic bytes per launch / its mean launch time,
               timed with HIP events on the stream it runs on around K
               back-to-back launches of that kernel
  parity       the parity gate: the oracle on evenly spaced rows of the very
               bytes the GPU read (copied back from HBM), against the timed
               outputs at the parity bar; value is null when it fails
  cpu_baseline the fp64 CPU oracle on those rows (a reported baseline, not
               the target), and single-thread times of the two small
               workloads
  cold_cache_and_ceilings
               (elementwise workloads) the median of each kernel's launches
               with a 512 MiB read before each one (nothing left in L2 or the
               Infinity Cache), the same after a 512 MiB write instead
               (*_cold_after_write: its dirty lines are written back during
               the launch), and a plain copy and bf16 add of the same sizes,
               warm and cold, as measured ceilings of their read:write mixes

Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SiTU-GLU fwd+bwd achieved HBM GB/s (% of MI355X peak) and rows/s, bf16"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 10**6       # MI355X Infinity Cache (AMD public spec)
CSRC = os.path.join(ROOT, "ffn_gated_activation_amd", "csrc")
KERNEL_SOURCE = os.path.join(CSRC, "situ_glu_kernels.hip")
MX_KERNEL_SOURCE = os.path.join(CSRC, "situ_glu_mx.hip")
ARES_KERNEL_SOURCE = os.path.join(CSRC, "situ_glu_attn_res.hip")
GEMM_KERNEL_SOURCE = os.path.join(CSRC, "situ_glu_gemm.hip")
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")


def _kernel_source_hash(path: str = KERNEL_SOURCE) -> str:
    """sha256 of a kernel source and the device header it includes."""
    h = hashlib.sha256()
    for p in (path, os.path.join(CSRC, "situ_glu_device.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic(workload: str, kernel: str, source: str = KERNEL_SOURCE):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != _kernel_source_hash(source):
        return None
    return rec.get("hbm_bytes_per_launch")


def _cores() -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(cores, 16))


def _host_info() -> dict:
    """The host and software the numbers were taken on."""
    import platform

    import torch
    info = {"cpu_model": None, "host_threads": _cores(), "python": platform.python_version(),
            "torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None),
            "rocm": None, "amdgpu_driver": None,
            "gpu": torch.cuda.get_device_name(0) if torch.cuda.is_available() else None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    for key, path in (("rocm", "/opt/rocm/.info/version"), ("amdgpu_driver", "/sys/module/amdgpu/version")):
        try:
            with open(path) as f:
                info[key] = f.read().strip()
        except OSError:
            pass
    return info


def _ordinal_bf16(bits):
    import numpy as np
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def _max_bf16_ulp(gpu, ref64) -> int:
    """Largest ordinal distance between the GPU's bf16 values and the
    oracle's fp64 values rounded once to bf16 (+0 and -0 the same point)."""
    import numpy as np

    import oracle
    import torch
    g = gpu.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(ref64.shape)
    d = np.abs(_ordinal_bf16(g) - _ordinal_bf16(oracle.round_bf16_bits(ref64)))
    return int(d.max()) if d.size else 0


def _oracle_leg(name: str, x: dict, outs: dict, sample_elems: int, timed: bool) -> tuple:
    """The oracle on rows of the very inputs the GPU ran on (copied back from
    HBM): the parity gate (every output of those rows against the oracle at
    the parity bar: 1 bf16 ulp; dr within 1e-4 of its row sum's condition
    scale plus one ulp) and, when `timed`, the CPU baseline (the fp64 oracle's
    forward and backward on those rows, on the host's cores)."""
    import numpy as np

    import oracle
    import torch

    from ffn_gated_activation_amd.workloads import algorithmic_bytes
    gu, rw, go = x["gate_up"], x["routing_weights"], x["grad_out"]
    rows, inter = gu.shape[0], gu.shape[1] // 2
    n = max(1, min(rows, sample_elems // inter))
    idx = torch.unique(torch.linspace(0, rows - 1, n, device=gu.device).round().long())
    n = int(idx.numel())
    broadcast = rw.numel() == 1 and rows != 1
    want = x["want_drw"] and not broadcast
    gu64 = gu.index_select(0, idx).double().cpu().numpy()
    rw64 = (rw if broadcast else rw.index_select(0, idx)).double().cpu().numpy().reshape(-1)
    go64 = None if go is None else go.index_select(0, idx).double().cpu().numpy()
    cores = _cores()
    t0 = time.perf_counter()
    y = oracle.forward(gu64, rw64, x["beta"], x["linear_beta"], threads=cores)
    b = None
    if go64 is not None:
        b = oracle.backward(gu64, rw64, go64, x["beta"], x["linear_beta"], want_dr=want,
                            want_scales=want or gu.dtype != torch.bfloat16, threads=cores)
    dt = time.perf_counter() - t0
    if "y" not in outs:
        parity = None        # MXFP8 outputs: the GPU tests check those against the oracle's windows
    elif gu.dtype != torch.bfloat16:
        parity = _parity_f32(outs, idx, inter, y, b, want, n, rows)
    else:
        parity = _parity(outs, idx, inter, y, b, want, n, rows)
    base = None
    if timed:
        nbytes = algorithmic_bytes(name, rows=n)["total"]
        what = "fp64 forward+backward" if go is not None else "fp64 forward"
        base = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{name}: {n} of its {rows} rows, evenly spaced, the same bytes the GPU read "
                          f"(copied back from HBM), {what}, {dt:.2f} s wall",
                "rows_per_s": round(n / dt, 1)}
    return base, parity


def _parity(outs: dict, idx, inter: int, y, b, want: bool, n: int, rows: int) -> dict:
    """bf16 outputs of the sampled rows against the oracle: at most 1 ulp;
    dr within 1e-4 of its row sum's condition scale plus one fp32 ulp."""
    import numpy as np
    parity = {"rows_checked": n, "of_rows": rows, "values_checked": n * inter * (1 if b is None else 3),
              "max_bf16_ulp": {"y": _max_bf16_ulp(outs["y"].index_select(0, idx), y)}}
    if b is not None:
        d = outs["dgu"].index_select(0, idx)
        parity["max_bf16_ulp"]["dG"] = _max_bf16_ulp(d[:, :inter], b["d_gate_up"][:, :inter])
        parity["max_bf16_ulp"]["dU"] = _max_bf16_ulp(d[:, inter:], b["d_gate_up"][:, inter:])
        if want:
            g = outs["drw"].index_select(0, idx).double().cpu().numpy().reshape(-1)
            err = np.abs(g - b["dr"])
            tol = 1e-4 * np.maximum(b["dr_abs"], 2.0 ** -126) + 2.0 ** -24 * np.abs(b["dr"])
            parity["dr_max_err_over_scale"] = float(np.max(err / np.maximum(b["dr_abs"], 1e-300)))
            parity["dr_within_bar"] = bool(np.all(err <= tol))
    parity["pass"] = max(parity["max_bf16_ulp"].values()) <= 1 and parity.get("dr_within_bar", True)
    return parity


def _parity_f32(outs: dict, idx, inter: int, y, b, want: bool, n: int, rows: int) -> dict:
    """fp32 outputs of the sampled rows against the oracle: |gpu - ref| at most
    1e-5 of |ref| (floored at fp32's smallest normal number) for Y, dG and dU,
    dG's scale being the sum of its two terms' magnitudes where they cancel by
    100x or more; dr as for bf16.  No subnormal allowance: the fp32 workload's
    inputs keep every intermediate normal."""
    import numpy as np

    def rel_err(t, ref, scale=None):
        g = t.index_select(0, idx).double().cpu().numpy().reshape(ref.shape)
        s = np.maximum(np.abs(ref), 2.0 ** -126)
        if scale is not None:
            s = np.where(scale >= 100.0 * np.abs(ref), np.maximum(s, scale), s)
        return float(np.max(np.abs(g - ref) / s)) if ref.size else 0.0

    parity = {"rows_checked": n, "of_rows": rows, "values_checked": n * inter * (1 if b is None else 3),
              "max_rel_err": {"y": rel_err(outs["y"], y)}}
    if b is not None:
        d = outs["dgu"]
        parity["max_rel_err"]["dG"] = rel_err(d[:, :inter], b["d_gate_up"][:, :inter], b["dg_scale"])
        parity["max_rel_err"]["dU"] = rel_err(d[:, inter:], b["d_gate_up"][:, inter:])
        if want:
            g = outs["drw"].index_select(0, idx).double().cpu().numpy().reshape(-1)
            err = np.abs(g - b["dr"])
            tol = 1e-4 * np.maximum(b["dr_abs"], 2.0 ** -126) + 2.0 ** -24 * np.abs(b["dr"])
            parity["dr_max_err_over_scale"] = float(np.max(err / np.maximum(b["dr_abs"], 1e-300)))
            parity["dr_within_bar"] = bool(np.all(err <= tol))
    parity["pass"] = max(parity["max_rel_err"].values()) <= 1e-5 and parity.get("dr_within_bar", True)
    return parity


def _single_thread_oracle() -> dict:
    """The oracle on one host thread at the two small workloads: all of
    fp32_small (forward + backward + dr) and all of top1_fwd (forward)."""
    import oracle

    from ffn_gated_activation_amd.workloads import algorithmic_bytes, make_inputs
    out = {}
    for name in ("fp32_small", "top1_fwd"):
        x = make_inputs(name, device="cpu", seed=0)
        gu = x["gate_up"].double().numpy()
        rw = x["routing_weights"].double().numpy().reshape(-1)
        go = None if x["grad_out"] is None else x["grad_out"].double().numpy()
        t0 = time.perf_counter()
        oracle.forward(gu, rw, x["beta"], x["linear_beta"], threads=1)
        if go is not None:
            oracle.backward(gu, rw, go, x["beta"], x["linear_beta"], want_dr=x["want_drw"], want_scales=False,
                            threads=1)
        dt = time.perf_counter() - t0
        rows = gu.shape[0]
        out[name] = {"rows": rows, "seconds": round(dt, 4), "rows_per_s": round(rows / dt, 1),
                     "GB/s": round(algorithmic_bytes(name)["total"] / dt / 1e9, 4),
                     "passes": "fwd+bwd+dr" if go is not None else "fwd", "threads": 1,
                     "inputs": "drawn on the host (seed 0)"}
    return out


def _copy_calibration(args, dev):
    """A plain device copy of known size, for the HBM counter calibration runs."""
    if not args.copy_calibration_mib:
        return
    import torch
    n = args.copy_calibration_mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def _cpu_baseline_attn_res(name: str) -> dict:
    import oracle
    from ffn_gated_activation_amd.workloads import ATTN_RES, attn_res_bytes, make_attn_res_inputs
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    w = ATTN_RES[name]
    x = make_attn_res_inputs(w.tokens, w.stored, w.hidden, True, dtype=w.dtype, device="cpu", seed=0, eps=w.eps)
    args = [t.double().numpy() for t in (x["blocks"], x["prefix"], x["norm_weight"], x["proj_weight"])]
    t0 = time.perf_counter()
    oracle.attn_res_forward(*args, w.eps, threads=cores)
    dt = time.perf_counter() - t0
    return {"value": round(attn_res_bytes(name) / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{name} recipe, all {w.tokens} tokens (seed 0, drawn on the host), fp64, {dt:.2f} s wall",
            "tokens_per_s": round(w.tokens / dt, 1)}


def bench_attn_res(args) -> int:
    import torch

    from ffn_gated_activation_amd import situ_glu_attn_res_fwd
    from ffn_gated_activation_amd.workloads import ATTN_RES, attn_res_bytes, make_attn_res_inputs
    w = ATTN_RES[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_attn_res_inputs(w.tokens, w.stored, w.hidden, True, dtype=w.dtype, device=dev, seed=0, eps=w.eps)
    out = torch.empty(w.tokens, w.hidden, dtype=w.dtype, device=dev)

    def step():
        situ_glu_attn_res_fwd(x["blocks"], x["prefix"], x["norm_weight"], x["proj_weight"], w.eps, out=out)

    settle_ms = _settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(args.steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    k_ms = ev[0].elapsed_time(ev[1]) / args.steps
    _copy_calibration(args, dev)
    nbytes = attn_res_bytes(args.workload)
    ms = wall / args.steps * 1e3
    value = nbytes / (ms / 1e3) / 1e9
    achieved = nbytes / (k_ms / 1e3) / 1e9
    rec = {
        "metric": "attention-residual mixing achieved HBM GB/s (% of MI355X peak) and tokens/s, bf16",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "tokens": w.tokens, "blocks": w.stored + 1,
                   "hidden": w.hidden, "eps": w.eps, "algorithmic_bytes_per_step": nbytes},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.tokens / (ms / 1e3), 1),
        "clock_settle_ms": round(settle_ms, 1),
        "host": _host_info(),
        "kernels": {"attn_res": {"ms": round(k_ms, 5), "bytes": nbytes, "GB/s": round(achieved, 2)}},
        "roofline": {"bound": "hbm", "kernel": "situ_glu_attn_res_stream_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic(args.workload, "attn_res", ARES_KERNEL_SOURCE)},
        "cpu_baseline": None if args.no_cpu_baseline else _cpu_baseline_attn_res(args.workload),
    }
    print(json.dumps(rec), flush=True)
    return 0


def _median_ms(fn, n, flush=None, write: bool = False) -> float:
    """Median duration of n launches of fn, each between two HIP events on
    the launch stream; with `flush`, a read of 512 MiB (not timed) runs
    before every launch so that nothing the launch reads is left in L2 or the
    Infinity Cache.  A read, not a fill: a fill leaves up to the Infinity
    Cache's 256 MB of dirty lines, whose write-back the timed launch would
    then pay for.  `write` takes the fill instead (the literal flush-write of
    the timing protocol, reported beside the read)."""
    import torch
    ts = []
    for _ in range(n):
        if flush is not None:
            if write:
                flush.fill_(1.0)
            else:
                flush.amax()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return statistics.median(ts)


def _under_rocprof() -> bool:
    """True when rocprofv3 has preloaded its tool library into this process."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ)


def _kernel_only_cold_ms(fn, n, flush):
    """Median kernel-only duration (ms) of n cold launches of fn: the same
    protocol as _median_ms with a flush, the durations taken from the
    device's own kernel timestamps (torch.profiler over the ROCm tracer)
    instead of HIP events, which also count the launch's dispatch latency.
    The library's kernels of one call are added.  None if the profiler gives
    no device events here."""
    import torch
    if _under_rocprof():
        return None      # one tracer at a time: rocprofv3 already records these kernels
    try:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(n):
                flush.amax()
                fn()
                torch.cuda.synchronize()
        d = [e.device_time for e in prof.events()
             if e.device_type == torch.autograd.DeviceType.CUDA and "situ" in e.name]
    except Exception:    # no tracer on this host: the HIP-event medians stand alone
        return None
    if not d or len(d) % n:
        return None
    k = len(d) // n
    per_call = [sum(d[i * k:(i + 1) * k]) for i in range(n)]
    return statistics.median(per_call) / 1e3


def _cold_entry(ms, nbytes):
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"ms": round(ms, 5), "GB/s": round(gbs, 2), "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}


def _graph_replay_ms(kernels: dict, nbytes: dict, n: int) -> dict:
    """Launches too short for the host to keep the queue full (a few tens of
    microseconds, against a few microseconds of Python and ctypes per call):
    n back-to-back launches of each kernel recorded once in a HIP graph, the
    graph replayed between two HIP events.  The kernels are the same; only
    the host's launch cost leaves the measurement."""
    import torch
    out = {"launches_per_replay": n}
    side = torch.cuda.Stream()
    for name, fn in kernels.items():
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        ms = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b) / n)
        m = statistics.median(ms)
        out[name] = {"ms": round(m, 5), "GB/s": round(nbytes[name] / (m / 1e3) / 1e9, 2),
                     "pct_of_hbm_peak": round(100.0 * nbytes[name] / (m / 1e3) / 1e9 / HBM_PEAK_GBS, 2)}
        del g
    return out


def _cold_kernels(kernels: dict, nbytes: dict, n: int, dev) -> dict:
    """Cold-cache medians (a 512 MiB read before each launch) of the path's
    kernels alone: between HIP events on the launch stream, and kernel-only
    from the device's timestamps."""
    import torch
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    out = {"flush_bytes_read": 512 << 20, "launches": n}
    for name, fn in kernels.items():
        out[f"{name}_cold"] = _cold_entry(_median_ms(fn, n, flush), nbytes[name])
        ko = _kernel_only_cold_ms(fn, n, flush)
        out[f"{name}_cold_kernel_only"] = None if ko is None else _cold_entry(ko, nbytes[name])
    del flush
    return out


def _cold_and_ceilings(kernels: dict, nbytes: dict, rows: int, inter: int, n: int, dev) -> dict:
    """Cold-cache medians of the path's kernels, and plain elementwise kernels
    of the same byte counts for scale: a copy (1 read : 1 write), a bf16 add
    (2 : 1, the forward's mix) and the stream probe at the forward's and the
    backward's mixes, timed warm (back to back) and cold."""
    import torch
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    out = {"flush_bytes_read": 512 << 20, "launches": n}
    for name, fn in kernels.items():
        ms = _median_ms(fn, n, flush)
        out[f"{name}_cold"] = {"ms": round(ms, 5), "GB/s": round(nbytes[name] / (ms / 1e3) / 1e9, 2)}
        ko = _kernel_only_cold_ms(fn, n, flush)
        out[f"{name}_cold_kernel_only"] = None if ko is None else _cold_entry(ko, nbytes[name])
    for name, fn in kernels.items():
        ms = _median_ms(fn, n, flush, write=True)
        out[f"{name}_cold_after_write"] = {"ms": round(ms, 5), "GB/s": round(nbytes[name] / (ms / 1e3) / 1e9, 2)}
    a = torch.empty(rows, inter, dtype=torch.bfloat16, device=dev).normal_()
    b = torch.empty_like(a).normal_()
    c = torch.empty_like(a)
    e = a.numel() * 2
    for name, fn, nb in (("copy_1to1", lambda: c.copy_(a), 2 * e), ("add_2to1", lambda: torch.add(a, b, out=c), 3 * e)):
        warm = _median_ms(fn, n)
        cold = _median_ms(fn, n, flush)
        out[name] = {"bytes": nb, "warm_GB/s": round(nb / (warm / 1e3) / 1e9, 2),
                     "cold_GB/s": round(nb / (cold / 1e3) / 1e9, 2)}
    del b, c
    out["stream_probe"] = _probe_ceilings(a, n, flush)
    del flush
    return out


def _probe_ceilings(a, n: int, flush) -> dict:
    """The SiTU kernels' access pattern with no arithmetic
    (libsitu_stream_probe.so, built next to the library): 16-byte
    non-temporal loads and stores, one wavefront per 1 KiB chunk of every
    stream, at the forward's mix (2 read streams : 1 written) and the
    backward's (3 : 2, the routing weights aside), streams of the workload's
    [rows, I] bf16 size.  The memory ceiling of each mix."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "ffn_gated_activation_amd", "libsitu_stream_probe.so")
    if not os.path.exists(path):
        return {"error": "libsitu_stream_probe.so is not built (run __graft_entry__.build())"}
    lib = ctypes.CDLL(path)
    lib.situ_stream_probe.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    lib.situ_stream_probe.restype = ctypes.c_int
    e = a.numel() * a.element_size()
    ins = [a] + [torch.empty_like(a).normal_() for _ in range(2)]
    outs = [torch.empty_like(a) for _ in range(2)]
    res = {"stream_bytes": e}
    for name, ni, no in (("probe_2to1", 2, 1), ("probe_3to2", 3, 2)):
        pin = (ctypes.c_void_p * ni)(*[t.data_ptr() for t in ins[:ni]])
        pout = (ctypes.c_void_p * no)(*[t.data_ptr() for t in outs[:no]])

        def fn():
            rc = lib.situ_stream_probe(pin, ni, pout, no, e, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"situ_stream_probe returned {rc}")
        nb = (ni + no) * e
        warm = _median_ms(fn, n)
        cold = _median_ms(fn, n, flush)
        res[name] = {"bytes": nb, "warm_GB/s": round(nb / (warm / 1e3) / 1e9, 2),
                     "cold_GB/s": round(nb / (cold / 1e3) / 1e9, 2)}
    del ins, outs
    return res


def _cpu_baseline_grouped(name: str, sample_rows: int) -> dict:
    import oracle
    from threadpoolctl import threadpool_limits

    from ffn_gated_activation_amd.workloads import GROUPED, GROUPED_MX, make_grouped_inputs, make_grouped_mx_inputs
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    mx = name in GROUPED_MX
    w = GROUPED_MX[name] if mx else GROUPED[name]
    if mx:
        x = make_grouped_mx_inputs(w.rows, w.experts, w.hidden, w.inter, "e4m3", device="cpu", seed=0)
    else:
        x = make_grouped_inputs(w.rows, w.experts, w.hidden, w.inter, device="cpu", seed=0)
    # the first sample_rows rows with their experts' weights (rows are grouped by expert)
    off = x["offsets"]
    n = min(sample_rows, w.rows)
    last = max(e for e in range(w.experts) if off[e] < n)
    sub_off = [min(o, n) for o in off[:last + 2]]
    rs = x["routing_weights"][:n].double().numpy()
    if mx:
        args = (x["x_codes"][:n].numpy(), x["x_scales"][:n].numpy(), x["weight_codes"][:last + 1].numpy(),
                x["weight_scales"][:last + 1].numpy())
    else:
        args = (x["x"][:n].double().numpy(), x["weight"][:last + 1].double().numpy())
    del x
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        if mx:
            oracle.grouped_glu_forward_mx(*args, sub_off, rs, "e4m3", w.beta, w.linear_beta, threads=cores,
                                          want_terms=False)
        else:
            oracle.grouped_glu_forward(*args, sub_off, rs, w.beta, w.linear_beta, threads=cores, want_terms=False)
        dt = time.perf_counter() - t0
    flops = 2 * n * w.hidden * 2 * w.inter
    what = "MX decoding + " if mx else ""
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{name} recipe, first {n} rows ({last + 1} expert(s); seed 0, drawn on the host), "
                      f"{what}fp64 matrix products per expert + fp64 activation, {dt:.2f} s wall",
            "rows_per_s": round(n / dt, 1)}


def bench_grouped(args) -> int:
    import torch

    from ffn_gated_activation_amd import situ_glu_grouped_fwd, situ_glu_grouped_fwd_mxfp8
    from ffn_gated_activation_amd.workloads import GROUPED, GROUPED_MX, make_grouped_inputs, make_grouped_mx_inputs
    mx = args.workload in GROUPED_MX
    w = GROUPED_MX[args.workload] if mx else GROUPED[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if mx:
        x = make_grouped_mx_inputs(w.rows, w.experts, w.hidden, w.inter, "e4m3", device=dev, seed=0)
    else:
        x = make_grouped_inputs(w.rows, w.experts, w.hidden, w.inter, device=dev, seed=0)
    off = torch.tensor(x["offsets"], dtype=torch.int32, device=dev)
    out = torch.empty(w.rows, w.inter, dtype=torch.bfloat16, device=dev)
    gu = torch.empty(w.rows, 2 * w.inter, dtype=torch.bfloat16, device=dev)

    if mx:
        from ffn_gated_activation_amd import situ_glu_grouped_fwd_mxfp8_workspace_bytes
        wk = torch.empty(situ_glu_grouped_fwd_mxfp8_workspace_bytes(w.rows, w.hidden, w.experts, w.inter),
                         dtype=torch.uint8, device=dev)

    def step(with_gu=False):
        if mx:
            situ_glu_grouped_fwd_mxfp8(x["x_codes"], x["x_scales"], x["weight_codes"], x["weight_scales"], off,
                                       x["routing_weights"], "e4m3", w.beta, w.linear_beta, out=out,
                                       gate_up_out=gu if with_gu else None, workspace=wk)
        else:
            situ_glu_grouped_fwd(x["x"], x["weight"], off, x["routing_weights"], w.beta, w.linear_beta, out=out,
                                 gate_up_out=gu if with_gu else None)

    def events(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(n):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    settle_ms = _settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = events(step, args.steps)
    gu_ms = events(lambda: step(True), max(1, args.steps // 4))
    kernels = {"grouped_fwd": {"ms": round(k_ms, 5)}, "grouped_fwd_with_gate_up": {"ms": round(gu_ms, 5)}}
    if args.compare_unfused and mx:
        # context only: the library's block-scaled fp8 GEMM (torch._scaled_mm with E8M0 scales per 32
        # values) on one dense product of the same FLOPs, [M, K] x [K, 2I] with expert 0's weight, the
        # workload's own codes and scales; then the stand-alone activation kernel on its [M, 2I] output
        from ffn_gated_activation_amd import situ_glu_fwd
        e8 = torch.float8_e8m0fnu
        xa = x["x_codes"].view(torch.float8_e4m3fn)
        wb = x["weight_codes"][0].view(torch.float8_e4m3fn)
        sa, sb = x["x_scales"].view(e8), x["weight_scales"][0].contiguous().view(e8)
        rw2 = x["routing_weights"].reshape(-1, 1)

        def lib_mx():
            return torch._scaled_mm(xa, wb.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)

        def unfused():
            situ_glu_fwd(lib_mx(), rw2, w.beta, w.linear_beta, out=out)
        try:
            for _ in range(5):
                unfused()
            kernels["library_mx_gemm_same_flops"] = {"ms": round(events(lib_mx, 20), 5)}
            kernels["library_mx_gemm_then_activation"] = {"ms": round(events(unfused, 20), 5)}
        except (RuntimeError, TypeError, AttributeError) as ex:
            kernels["library_mx_gemm_same_flops"] = {"unavailable": f"{type(ex).__name__}: {str(ex)[:120]}"}
    if args.compare_unfused and not mx:
        # context only: the library grouped GEMM (torch._grouped_mm) writing gate_up, then the
        # stand-alone activation kernel on it
        from ffn_gated_activation_amd import situ_glu_fwd
        wt = x["weight"].transpose(1, 2)
        ends = off[1:].contiguous()
        rw2 = x["routing_weights"].reshape(-1, 1)

        def unfused():
            g = torch._grouped_mm(x["x"], wt, offs=ends)
            situ_glu_fwd(g, rw2, w.beta, w.linear_beta, out=out)
        for _ in range(20):
            unfused()
        kernels["unfused_grouped_mm_then_activation"] = {"ms": round(events(unfused, 20), 5)}
    _copy_calibration(args, dev)
    flops = 2 * w.rows * w.hidden * 2 * w.inter
    peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
    ms = wall / args.steps * 1e3
    value = flops / (ms / 1e3) / 1e12
    achieved = flops / (k_ms / 1e3) / 1e12
    for k in kernels.values():
        if "ms" in k:
            k["TFLOP/s"] = round(flops / (k["ms"] / 1e3) / 1e12, 2)
    prec = "MXFP8 (E4M3)" if mx else "bf16"
    rec = {
        "metric": f"fused FC1 grouped GEMM + SiTU-GLU achieved TFLOP/s (% of MI355X {prec} dense peak) and rows/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3-mx" if mx else "bf16", "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "rows": w.rows, "experts": w.experts,
                   "hidden": w.hidden, "intermediate": w.inter, "rows_per_expert": x["counts"],
                   "flops_per_step": flops},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "rows_per_s": round(w.rows / (ms / 1e3), 1),
        "clock_settle_ms": round(settle_ms, 1),
        "host": _host_info(),
        "kernels": kernels,
        "roofline": {"bound": "mfma",
                     "kernel": ("situ_glu_grouped_fwd_kernel, with the two situ_mx_scales_stage_major_kernel "
                                "launches of the same call" if mx else "situ_glu_grouped_fwd_kernel"),
                     "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": _traffic(args.workload, "grouped", GEMM_KERNEL_SOURCE)},
        "cpu_baseline": None if args.no_cpu_baseline else _cpu_baseline_grouped(args.workload,
                                                                               args.cpu_sample_rows_gemm),
    }
    print(json.dumps(rec), flush=True)
    return 0


def _settle(fn, ms: float) -> float:
    """Run fn back to back for at least `ms` milliseconds of wall time (the
    GPU's clocks ramp up from idle over the first ~25 ms of load); returns
    the milliseconds spent."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def _elementwise(name: str, args, dev, full: bool) -> tuple:
    """Time one elementwise workload: clock settle, W warm-up steps, K timed
    steps between synchronisations (wall clock), then each kernel alone, K
    back-to-back launches between two HIP events on its stream.  With
    `full`, also the cold-cache medians and plain-kernel ceilings.  Returns
    (record, inputs, outputs)."""
    import torch

    from ffn_gated_activation_amd import situ_glu_bwd, situ_glu_bwd_mxfp8, situ_glu_fwd, situ_glu_fwd_mxfp8
    from ffn_gated_activation_amd.workloads import WORKLOADS, algorithmic_bytes, make_inputs
    w = WORKLOADS[name]
    x = make_inputs(name, device=dev, seed=0)
    gu, rw, go = x["gate_up"], x["routing_weights"], x["grad_out"]
    beta, lb, want = x["beta"], x["linear_beta"], x["want_drw"]
    outs = {}
    if w.mx:
        codes = torch.empty(w.rows, w.inter, dtype=torch.uint8, device=dev)
        scales = torch.empty(w.rows, -(-w.inter // 32), dtype=torch.uint8, device=dev)
    else:
        outs["y"] = torch.empty(w.rows, w.inter, dtype=w.dtype, device=dev)
    if w.backward and not w.mx:
        outs["dgu"] = torch.empty_like(gu)
    if w.backward and w.mx:
        dcodes = torch.empty(w.rows, 2 * w.inter, dtype=torch.uint8, device=dev)
        dscales = torch.empty(w.rows, 2 * -(-w.inter // 32), dtype=torch.uint8, device=dev)
    if want:
        outs["drw"] = torch.empty_like(rw)
    torch.cuda.synchronize()

    def fwd():
        if w.mx:
            situ_glu_fwd_mxfp8(gu, rw, beta, lb, w.mx, "floor", codes=codes, scales=scales)
        else:
            situ_glu_fwd(gu, rw, beta, lb, out=outs["y"])

    def bwd():
        if w.mx:
            situ_glu_bwd_mxfp8(gu, rw, go, beta, lb, want, w.mx, "floor", d_codes=dcodes, d_scales=dscales,
                               d_routing_weights=outs.get("drw"))
        else:
            situ_glu_bwd(gu, rw, go, beta, lb, want_drw=want, d_gate_up=outs["dgu"],
                         d_routing_weights=outs.get("drw"))

    def step():
        fwd()
        if w.backward:
            bwd()

    settle_ms = _settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps between synchronisations (wall clock) ...
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # ... then each kernel on its own: K back-to-back launches between two HIP
    # events on the launch stream (the launches are independent of each other)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(args.steps):
        fwd()
    ev[1].record()
    if w.backward:
        for _ in range(args.steps):
            bwd()
    ev[2].record()
    torch.cuda.synchronize()
    fwd_ms = ev[0].elapsed_time(ev[1]) / args.steps
    bwd_ms = ev[1].elapsed_time(ev[2]) / args.steps if w.backward else 0.0

    unfused = {}
    if w.mx and full:
        # context: the bf16 kernels followed by the stand-alone MXFP8 quantiser (same blocks and rounding;
        # with I a multiple of 32 one quantiser call over [rows, 2I] gives d_gate_up's layout)
        from ffn_gated_activation_amd import situ_glu_mx_quantize
        yb = torch.empty(w.rows, w.inter, dtype=w.dtype, device=dev)
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

        def fwd_unfused():
            situ_glu_fwd(gu, rw, beta, lb, out=yb)
            situ_glu_mx_quantize(yb, w.mx, "floor", codes=codes, scales=scales)
        fns = {"unfused_fwd_then_quantize": fwd_unfused}
        if w.backward and w.inter % 32 == 0:
            dgb = torch.empty_like(gu)

            def bwd_unfused():
                situ_glu_bwd(gu, rw, go, beta, lb, want_drw=want, d_gate_up=dgb, d_routing_weights=outs.get("drw"))
                situ_glu_mx_quantize(dgb, w.mx, "floor", codes=dcodes, scales=dscales)
            fns["unfused_bwd_then_quantize"] = bwd_unfused
        for uname, fn in fns.items():
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            ev2[0].record()
            for _ in range(args.steps):
                fn()
            ev2[1].record()
            torch.cuda.synchronize()
            unfused[uname] = {"ms": round(ev2[0].elapsed_time(ev2[1]) / args.steps, 5)}

    if full:
        _copy_calibration(args, dev)
    ab = algorithmic_bytes(name)
    cold = None
    if not args.no_cold:
        ks = {"fwd": fwd, "bwd": bwd} if w.backward else {"fwd": fwd}
        if full:
            cold = _cold_and_ceilings(ks, ab, w.rows, w.inter, min(args.steps, 20), dev)
        elif ab["total"] < MALL_BYTES:
            # every byte of such a launch fits in the Infinity Cache, so back-to-back
            # launches would read it from there: the cold medians are its number
            cold = _cold_kernels(ks, ab, min(args.steps, 20), dev)
    graph = None
    if not full and fwd_ms < 0.05:
        graph = _graph_replay_ms({"fwd": fwd, "bwd": bwd} if w.backward else {"fwd": fwd}, ab, args.steps)
    ms_per_step = wall / args.steps * 1e3
    value = ab["total"] / (ms_per_step / 1e3) / 1e9
    dom = "bwd" if w.backward else "fwd"
    dom_ms = bwd_ms if w.backward else fwd_ms
    achieved = ab[dom] / (dom_ms / 1e3) / 1e9
    kname = ("situ_glu_bwd_mx_vec_kernel" if w.backward and w.mx else
             ("situ_glu_bwd_dr_kernel" if want else "situ_glu_bwd_kernel") if w.backward else
             "situ_glu_fwd_mx_kernel" if w.mx else "situ_glu_fwd_kernel")
    src = MX_KERNEL_SOURCE if w.mx else KERNEL_SOURCE
    rec = {
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 5),
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "config": {"workload": w.name, "description": w.description, "rows": w.rows,
                   "intermediate": w.inter, "beta": w.beta, "linear_beta": w.linear_beta,
                   "passes": ("fwd+bwd" + ("+d_routing_weights" if want else "") +
                              (f" (MXFP8 {w.mx} Y and d_gate_up)" if w.mx else "") if w.backward else
                              f"fwd (MXFP8 {w.mx} output)" if w.mx else "fwd"),
                   "algorithmic_bytes_per_step": ab["total"]},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "rows_per_s": round(w.rows / (ms_per_step / 1e3), 1),
        "clock_settle_ms": round(settle_ms, 1),
        "kernels": {
            "fwd": {"ms": round(fwd_ms, 5), "bytes": ab["fwd"],
                    "GB/s": round(ab["fwd"] / (fwd_ms / 1e3) / 1e9, 2)},
            "bwd": ({"ms": round(bwd_ms, 5), "bytes": ab["bwd"],
                     "GB/s": round(ab["bwd"] / (bwd_ms / 1e3) / 1e9, 2)} if w.backward else None),
            **unfused,
        },
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic(name, dom, src)},
        "cold_cache_and_ceilings": cold,
    }
    if graph is not None:
        rec["kernels_graph_replay"] = graph
    return rec, x, outs


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    # the GPU's clocks take ~25 ms of load to ramp up from idle: the step runs
    # for this long before the warm-up steps, whatever --warmup is
    ap.add_argument("--settle-ms", type=float, default=100.0)
    ap.add_argument("--workload", default="dense_ffn")
    ap.add_argument("--also", default=None,
                    help="comma-separated elementwise workloads also timed in the same run and summarised under "
                         "'other_workloads' (default for dense_ffn: routed_top8,stress_sat,top1_fwd,fp32_small; "
                         "'' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg: the CPU baseline and the parity gate on the same bytes")
    ap.add_argument("--cpu-sample-elems", type=int, default=3 << 26,
                    help="values per half row times rows of the oracle sample (rows evenly spaced)")
    ap.add_argument("--cpu-sample-rows", type=int, default=65536,
                    help="attention-residual and grouped GEMM workloads: rows of the CPU-oracle sample")
    ap.add_argument("--cpu-sample-rows-gemm", type=int, default=65536,
                    help="rows of the CPU-oracle sample of the grouped GEMM workload")
    ap.add_argument("--compare-unfused", action="store_true",
                    help="grouped GEMM workloads: also time the library GEMM (torch._grouped_mm for bf16, "
                         "torch._scaled_mm with MX scales on the same FLOPs for MXFP8) + the activation kernel "
                         "(context)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache medians and the plain-kernel ceilings")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration runs)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the weighted SiTU-GLU path is row parallel and is measured "
              "on a single MI355X; --gpus above 1 is not supported.", file=sys.stderr)
        return 2

    import torch

    from ffn_gated_activation_amd.workloads import ATTN_RES, GROUPED, GROUPED_MX, WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.workload in ATTN_RES or args.workload in GROUPED or args.workload in GROUPED_MX:
        return bench_attn_res(args) if args.workload in ATTN_RES else bench_grouped(args)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    rec, x, outs = _elementwise(args.workload, args, dev, full=True)
    parity = cpu = None
    if not args.no_cpu_baseline:
        cpu, parity = _oracle_leg(args.workload, x, outs, args.cpu_sample_elems, timed=True)
        cpu["single_thread"] = _single_thread_oracle()
    del x, outs
    torch.cuda.empty_cache()
    also = args.also
    if also is None:
        also = "routed_top8,stress_sat,top1_fwd,fp32_small" if args.workload == "dense_ffn" else ""
    others = {}
    for name in [n for n in also.split(",") if n]:
        r, xo, oo = _elementwise(name, args, dev, full=False)
        par = None if args.no_cpu_baseline else _oracle_leg(name, xo, oo, 1 << 22, timed=False)[1]
        others[name] = {"GB/s": r["value"], "pct_of_hbm_peak": r["pct_of_hbm_peak"],
                        "ms_per_step": r["ms_per_step"], "rows_per_s": r["rows_per_s"],
                        "kernels": r["kernels"], "roofline_frac": r["roofline"]["frac"],
                        "roofline_kernel": r["roofline"]["kernel"], "parity": par}
        if r["cold_cache_and_ceilings"] is not None:
            others[name]["cold"] = r["cold_cache_and_ceilings"]
        if r.get("kernels_graph_replay") is not None:
            others[name]["kernels_graph_replay"] = r["kernels_graph_replay"]
        if par is not None and not par["pass"]:
            others[name]["GB/s"] = None
        del xo, oo
        torch.cuda.empty_cache()
    value = rec["value"]
    if parity is not None and parity.get("pass") is False:
        value = None    # a step whose outputs disagree with the oracle reports no throughput
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic",
        "config": rec["config"],
        "pct_of_hbm_peak": rec["pct_of_hbm_peak"],
        "rows_per_s": rec["rows_per_s"],
        "clock_settle_ms": rec["clock_settle_ms"],
        "parity": parity,
        "kernels": rec["kernels"],
        "roofline": rec["roofline"],
        "cold_cache_and_ceilings": rec["cold_cache_and_ceilings"],
        "other_workloads": others or None,
        "host": _host_info(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
