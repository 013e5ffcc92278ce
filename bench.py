"""Bench: exact attention fwd and fwd+bwd on one MI355X, through libfa's C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole hot path once: fa_fwd_ex (O, LSE) then fa_bwd_ex (D, dQ, dK, dV),
on seeded synthetic bf16 inputs already resident in HBM. Default workload: the long
causal head set (B=1, H=16, N=16384, d=128), the configuration the headline metric is
stated for. Prints one JSON line. Each timed call (step, forward, backward, preprocess) is
launched directly, back to back, with HIP events between the calls. --graph captures each
call once into a HIP graph and times the replays instead: the same kernels, but each
replay adds about 6 us of GPU time, which shows on the smallest workloads (--eager, the
default, is accepted for the recorded profiling commands).

FLOP convention (2 per multiply-add, allowed (query, key) pairs only):
  fwd = 4 * pairs * d (Q K^T and P V); bwd = 10 * pairs * d (recomputed Q K^T, dO V^T,
  P^T dO, dS K, dS^T Q); fwd+bwd = 14 * pairs * d.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA

# The pages' own figures, each on its own (NVIDIA) hardware: context, not targets.
PAGE_CONTEXT = [
    {"figure": "2-3x speed-up and 10x memory saving over standard attention",
     "hardware": "A100", "system": "FlashAttention"},
    {"figure": "175 TFLOP/s at 16K sequence length", "hardware": "A100",
     "system": "FlashAttention-2"},
    {"figure": "550 TFLOP/s forward, fp16, head dim 256", "hardware": "H100",
     "system": "FlashAttention-3"},
    {"figure": "700 TFLOP/s forward, FP8", "hardware": "H100", "system": "FlashAttention-3"},
]
HBM_PEAK_GBS = 8000.0
METRIC = "attention TFLOP/s fwd and fwd+bwd (bf16) at 1 GPU + % MFMA peak"


def allowed_pairs(N, causal, blockmask, kv_len_b, window=None):
    """Number of allowed (query, key) pairs of one head, from the mask definitions: row i
    may see keys lo_i <= j < hi_i (causal, padding, sliding window), thinned by the block
    table."""
    rows = np.arange(N, dtype=np.int64)
    hi = np.full(N, N, dtype=np.int64)
    lo = np.zeros(N, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, rows + 1)
    if kv_len_b is not None:
        hi = np.minimum(hi, int(kv_len_b))
    if window is not None:
        if window[0] >= 0:
            lo = np.maximum(lo, rows - window[0])
        if window[1] >= 0:
            hi = np.minimum(hi, rows + window[1] + 1)
    if blockmask is None:
        return int(np.clip(hi - lo, 0, None).sum())
    nb = blockmask.shape[0]
    total = 0
    for kb in range(nb):
        b0 = kb * 128
        cover = np.clip(np.minimum(hi, b0 + 128) - np.maximum(lo, b0), 0, 128)
        kept = blockmask[rows // 128, kb] != 0
        total += int(cover[kept].sum())
    return total


def workload_pairs(x):
    wl = x.wl
    total = 0
    for b in range(wl.B):
        kv = None if x.kv_len is None else int(x.kv_len[b])
        total += wl.H * allowed_pairs(wl.N, wl.causal, x.blockmask, kv, wl.window)
    return total


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_causal_16k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-footprint", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="with the default workload, skip timing the four other workloads")
    ap.add_argument("--no-device-sample", action="store_true",
                    help="skip the amd-smi clock/power sample (profiling runs)")
    ap.add_argument("--eager", action="store_true",
                    help="time direct calls (the default)")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP graph replays of each call instead of direct calls")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (a kernel of known "
                         "traffic, used to scale hardware byte counters)")
    args = ap.parse_args()
    args.eager = args.eager or not args.graph
    return args


class Buffers:
    def __init__(self, x, torch):
        import exact_io_aware_46_amd as fa
        wl = x.wl

        def dev(x):
            dt = torch.float16 if x.dtype == np.float16 else torch.bfloat16
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(dt)

        self.wl = wl
        self.q, self.k, self.v, self.do = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
        self.o = torch.empty_like(self.q)
        self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
        self.lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device="cuda")
        self.delta = torch.empty_like(self.lse)
        self.ws = torch.empty(fa.fa_bwd_workspace_bytes(wl.B, wl.H, wl.N, wl.d),
                              dtype=torch.uint8, device="cuda")
        self.bm = None if x.blockmask is None else torch.from_numpy(x.blockmask).cuda()
        self.kv = None if x.kv_len is None else torch.from_numpy(x.kv_len).cuda()
        self.fa = fa
        self.dtype_code = fa.DTYPE_F16 if wl.dtype == "f16" else fa.DTYPE_BF16

    def fwd(self):
        w = self.wl
        wl, wr = (-1, -1) if w.window is None else w.window
        if w.dropout is not None:
            self.fa.fa_fwd_dropout(self.dtype_code, self.q, self.k, self.v, self.o, self.lse,
                                   w.B, w.H, w.N, w.d, w.scale, w.causal, self.bm, self.kv,
                                   wl, wr, *w.dropout)
            return
        fn = self.fa.fa_fwd_f16 if w.dtype == "f16" else self.fa.fa_fwd_window
        fn(self.q, self.k, self.v, self.o, self.lse, w.B, w.H, w.N, w.d, w.scale, w.causal,
           self.bm, self.kv, wl, wr)

    def bwd(self):
        w = self.wl
        wl, wr = (-1, -1) if w.window is None else w.window
        if w.dropout is not None:
            self.fa.fa_bwd_dropout(self.dtype_code, self.q, self.k, self.v, self.o, self.lse,
                                   self.do, self.dq, self.dk, self.dv, w.B, w.H, w.N, w.d,
                                   w.scale, w.causal, self.bm, self.kv, wl, wr, *w.dropout,
                                   workspace=self.ws)
            return
        fn = self.fa.fa_bwd_f16 if w.dtype == "f16" else self.fa.fa_bwd_window
        fn(self.q, self.k, self.v, self.o, self.lse, self.do, self.dq, self.dk, self.dv, w.B,
           w.H, w.N, w.d, w.scale, w.causal, self.bm, self.kv, wl, wr, self.ws)

    def pre(self):
        w = self.wl
        fn = self.fa.fa_bwd_preprocess_f16 if w.dtype == "f16" else self.fa.fa_bwd_preprocess
        fn(self.o, self.do, self.delta, w.B, w.H, w.N, w.d)

    def step(self):
        self.fwd()
        self.bwd()


class Fp8Buffers:
    """Device buffers of the FP8 forward (E4M3 Q, K, V; bf16 O; V^T workspace)."""

    def __init__(self, x, torch):
        import exact_io_aware_46_amd as fa
        wl = x.wl
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.wl, self.fa, self.descale = wl, fa, x.descale
        self.q, self.k, self.v = dev(x.q), dev(x.k), dev(x.v)
        self.o = torch.empty((wl.B, wl.H, wl.N, wl.d), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(fa.fa_fwd_fp8_workspace_bytes(wl.B, wl.H, wl.N, wl.d),
                              dtype=torch.uint8, device="cuda")
        self.bm = None if x.blockmask is None else torch.from_numpy(x.blockmask).cuda()
        self.kv = None if x.kv_len is None else torch.from_numpy(x.kv_len).cuda()

    def fwd(self):
        w = self.wl
        wl, wr = (-1, -1) if w.window is None else w.window
        self.fa.fa_fwd_fp8(self.q, self.k, self.v, self.o, self.lse, w.B, w.H, w.N, w.d,
                           w.scale, *self.descale, w.causal, self.bm, self.kv, wl, wr, self.ws)


def fp8_cpu_baseline(x, heads=2):
    """The FP8 oracle forward (as it stands) on the first ``heads`` heads; rate =
    4 * pairs * d FLOP / wall time."""
    import threadpoolctl
    from oracle import attention as orc
    wl = x.wl
    sel = [(b, h) for b in range(wl.B) for h in range(wl.H)][:heads]
    flop = 0.0
    t0 = time.perf_counter()
    for b, h in sel:
        kv = None if x.kv_len is None else int(x.kv_len[b])
        orc.head_forward_fp8(x.q[b, h], x.k[b, h], x.v[b, h], x.descale, wl.scale, wl.causal,
                             x.blockmask, kv, window=wl.window)
        flop += 4.0 * allowed_pairs(wl.N, wl.causal, x.blockmask, kv, wl.window) * wl.d
    dt = time.perf_counter() - t0
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{len(sel)} of {wl.B * wl.H} heads of {wl.name} (N={wl.N}, d={wl.d}): "
                      f"fp64 FP8-quantised forward with S and P materialised, numpy/OpenBLAS, "
                      f"{dt:.1f} s wall"}


def fp8_main(args, torch, wl, x):
    """FP8 workloads are forward only: a step is one forward (the V transpose pass
    included)."""
    pairs = workload_pairs(x)
    fl_fwd = 4.0 * pairs * wl.d
    buf = Fp8Buffers(x, torch)
    ms_fwd = time_loop(torch, buf.fwd if args.eager else graphed(torch, buf.fwd), args.steps,
                       args.warmup)
    tf_fwd = fl_fwd / (ms_fwd * 1e-3) / 1e12
    k_fwd = f"fwd_fp8_kernel<{wl.d}>"
    rec = {
        "metric": "attention TFLOP/s fwd (fp8 e4m3 inputs) at 1 GPU + % MFMA peak",
        "value": round(tf_fwd, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_fwd, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "causal": wl.causal, "mask": wl.mask, "window": wl.window,
                   "scale": wl.scale, "descale": list(x.descale), "allowed_pairs": pairs},
        "fwd_tflops": round(tf_fwd, 2), "fwd_ms": round(ms_fwd, 4),
        "timing_mode": "direct calls" if args.eager else "HIP graph replay of each call",
        "timing_ms": {"fwd": timing_record(ms_fwd)},
        "fwd_pct_mfma_peak": round(100 * tf_fwd / MFMA_FP8_PEAK_TFLOPS, 2),
        "roofline": {"kernel": f"{k_fwd} + vt_fp8_kernel<{wl.d}> (whole forward)",
                     "bound": "mfma", "achieved": round(tf_fwd, 2),
                     "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_fwd / MFMA_FP8_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name, "fp8_kernel", [k_fwd])},
    }
    peak = mfma_peak_record("fp8")
    rec["mfma_peak"] = peak
    if "tflops" in peak:
        rec["fwd_pct_measured_mfma_peak"] = round(100 * tf_fwd / peak["tflops"], 2)
        rec["roofline"]["frac_of_measured_peak"] = round(tf_fwd / peak["tflops"], 4)
    rec["device"] = None if args.no_device_sample else device_sample(torch, buf.fwd)
    rec["context"] = {"note": "the pages' figures on their own hardware; context only",
                      "items": PAGE_CONTEXT}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = fp8_cpu_baseline(x)
        rec["cpu_baseline"]["gpu_over_cpu"] = round(rec["value"] / rec["cpu_baseline"]["value"], 1)
    print(json.dumps(rec), flush=True)


def device_sample(torch, fn, seconds=5.0):
    """Clock and power while the GPU runs ``fn`` back to back: about 1 s of steps runs
    first (so the clocks have ramped), then one ``amd-smi metric`` query runs in a child
    process while steps keep the queue full (synchronising every ~100 ms of work). A
    reading below 1 GHz means the query caught the GPU idle and is labelled as such.
    Returns None if amd-smi is missing or fails."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    chunk = max(20, int(0.1 / max(time.perf_counter() - t0, 1e-5)))  # steps per ~100 ms
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        fn()
        n += 1
        if n % chunk == 0:
            torch.cuda.synchronize()
    try:
        proc = subprocess.Popen([exe, "metric", "-c", "-p", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        torch.cuda.synchronize()
        return None
    t1 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t1 < seconds:
        fn()
        n += 1
        if n % chunk == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    try:
        out, _ = proc.communicate(timeout=max(1.0, seconds - (time.perf_counter() - t1)))
        gpu = json.loads(out)["gpu_data"][0]
        clks = [v["clk"]["value"] for k, v in gpu["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and "clk" in v]
        rec = {"gfx_clk_mhz_mean": round(sum(clks) / len(clks), 1), "gfx_clk_mhz": clks,
               "socket_power_w": gpu["power"]["socket_power"]["value"],
               "source": "amd-smi metric -c -p, sampled while steps ran"}
        if rec["gfx_clk_mhz_mean"] < 1000:
            rec["note"] = "below 1 GHz: the query caught the GPU idle; not the clock under load"
        return rec
    except Exception:  # noqa: BLE001 -- the sample is optional context
        proc.kill()
        return None


class Timing(float):
    """Mean milliseconds per call (the float value), with the median and minimum of the
    per-call times as attributes."""

    def __new__(cls, mean, median, minimum):
        t = super().__new__(cls, mean)
        t.median, t.min = median, minimum
        return t


def time_loop(torch, fn, steps, warmup):
    """Milliseconds per call, HIP events on the stream the kernels run on: ``steps`` calls
    back to back with an event between each two, no synchronisation inside the timed
    region. The mean is first-to-last event over ``steps``."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(s)
    for i in range(steps):
        fn()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return Timing(ev[0].elapsed_time(ev[steps]) / steps, per[len(per) // 2], per[0])


def graphed(torch, fn):
    """``fn`` captured once into a HIP graph (through torch's graph API: the library's
    launches go to the capturing stream, and it allocates and clears nothing, so the whole
    call is capturable); returns the graph's replay. A replay takes the host less time
    than the calls it holds, and the GPU about 6 us more than a direct launch."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g.replay


def timing_record(t):
    return {"mean": round(float(t), 4), "median": round(t.median, 4), "min": round(t.min, 4)}


def mfma_peak_record(dtype):
    """The matrix-core probe's sustained rate (bf16 or fp8), or None if it cannot run."""
    try:
        from exact_io_aware_46_amd import mfma_peak
        return mfma_peak.measure(dtype)
    except Exception as e:  # noqa: BLE001 -- a missing probe leaves only the spec fraction
        return {"error": str(e)}


def footprint_sweep(torch, base, steps=10, warmup=3):
    """Peak device bytes of fwd+bwd buffers + workspace + calls at several N (same B, H, d),
    and the fwd and fwd+bwd TFLOP/s at each N (timed like the main loop)."""
    from exact_io_aware_46_amd import inputs as inp
    out = {}
    for n in (2048, 4096, 8192, 16384):
        wl = base.with_n(n)
        x = inp.make_inputs(wl)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        before = torch.cuda.memory_allocated()
        free0, _ = torch.cuda.mem_get_info()
        buf = Buffers(x, torch)
        buf.step()
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        out[str(n)] = {"peak_bytes": int(torch.cuda.max_memory_allocated() - before),
                       "hip_free_delta_bytes": int(free0 - free1),
                       "materialised_SP_bf16_bytes": 2 * wl.B * wl.H * n * n * 2}
        pairs = workload_pairs(x)
        ms_f = time_loop(torch, buf.fwd, steps, warmup)
        ms_s = time_loop(torch, buf.step, steps, warmup)
        out[str(n)]["fwd_tflops"] = round(4.0 * pairs * wl.d / (ms_f * 1e-3) / 1e12, 2)
        out[str(n)]["fwd_bwd_tflops"] = round(14.0 * pairs * wl.d / (ms_s * 1e-3) / 1e12, 2)
        del buf
    ns = np.array([int(n) for n in out])
    pk = np.array([out[str(n)]["peak_bytes"] for n in ns], dtype=np.float64)
    slope, icpt = np.polyfit(ns, pk, 1)
    resid = float(np.max(np.abs(pk - (slope * ns + icpt)) / pk))
    return {"per_N": out, "linear_fit_bytes_per_token": float(slope),
            "linear_fit_max_rel_residual": resid}


KERNEL_SOURCES = {"fwd_kernel": ["fa_fwd.hip", "fa_device.hpp", "fa_internal.h"],
                  "bwd_kernel": ["fa_bwd.hip", "fa_bwd_rk.hip", "fa_bwd_rk_drop.hip", "fa_device.hpp",
                                 "fa_internal.h"],
                  "fp8_kernel": ["fa_fwd_fp8.hip", "fa_device.hpp", "fa_internal.h"]}


def source_hash(kind):
    """Hash of a kernel's sources with // comments, trailing blanks and empty lines left
    out, so an edit of comments alone keeps the recorded counters; a source built with
    options of its own adds them."""
    import hashlib
    from exact_io_aware_46_amd import build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "exact_io_aware_46_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
        if f in build.SOURCE_FLAGS:
            h.update(" ".join(build.SOURCE_FLAGS[f]).encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload, kind, kernels):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (profiles/traffic_<workload>.md, copy-calibrated), or None when there is no summary
    or the kernel's sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- traffic-json: (.*) -->", open(path).read())
    if not m:
        return None
    blob = json.loads(m.group(1))
    if blob.get("source_sha256", {}).get(kind) != source_hash(kind):
        return None
    try:
        return int(sum(blob["kernels"][k]["read_bytes"] + blob["kernels"][k]["write_bytes"]
                       for k in kernels))
    except KeyError:
        return None


OTHER_CONFIGS = ("single_head_256", "gpt2s_causal_1k", "bertl_kpad_512", "blocksparse_8k")


def other_configs(torch, inp, steps, warmup):
    """The other four workloads the headline metric is stated beside (one head of 256,
    GPT-2-small causal 1K, BERT-large with key padding, block-sparse 8K), timed like the
    main one with direct calls. Per workload: fwd, bwd and fwd+bwd times and TFLOP/s, and
    the HBM rate of the forward and backward: the compulsory bytes (forward 8Nd + 4N and
    backward 18Nd + 16N per head, bf16), and the copy-calibrated bytes that rocprofv3
    measured for these kernels when that summary is present and current, over the time."""
    out = {}
    for name in OTHER_CONFIGS:
        wl = inp.WORKLOADS[name]
        x = inp.make_inputs(wl)
        pairs = workload_pairs(x)
        fl_fwd, fl_bwd = 4.0 * pairs * wl.d, 10.0 * pairs * wl.d
        buf = Buffers(x, torch)
        t_fwd = time_loop(torch, buf.fwd, steps, warmup)
        t_bwd = time_loop(torch, buf.bwd, steps, warmup)
        t_step = time_loop(torch, buf.step, steps, warmup)
        heads = wl.B * wl.H
        comp_fwd = heads * (8 * wl.N * wl.d + 4 * wl.N)
        comp_bwd = heads * (18 * wl.N * wl.d + 16 * wl.N)
        rec = {"fwd_ms": round(float(t_fwd), 4), "bwd_ms": round(float(t_bwd), 4),
               "step_ms": round(float(t_step), 4),
               "fwd_median_ms": round(t_fwd.median, 4), "step_median_ms": round(t_step.median, 4),
               "fwd_tflops": round(fl_fwd / (t_fwd * 1e-3) / 1e12, 2),
               "bwd_tflops": round(fl_bwd / (t_bwd * 1e-3) / 1e12, 2),
               "fwd_bwd_tflops": round((fl_fwd + fl_bwd) / (t_step * 1e-3) / 1e12, 2),
               "fwd_bwd_frac_of_peak": round((fl_fwd + fl_bwd) / (t_step * 1e-3) / 1e12
                                             / MFMA_BF16_PEAK_TFLOPS, 4),
               "fwd_compulsory_gbs": round(comp_fwd / (t_fwd * 1e-3) / 1e9, 1),
               "bwd_compulsory_gbs": round(comp_bwd / (t_bwd * 1e-3) / 1e9, 1)}
        m = re.search(r"<!-- traffic-json: (.*) -->", _read(os.path.join(
            ROOT, "profiles", f"traffic_{name}.md")))
        if m:
            blob = json.loads(m.group(1))
            cur = all(blob.get("source_sha256", {}).get(k) == source_hash(k)
                      for k in ("fwd_kernel", "bwd_kernel"))
            if cur:
                kern = blob["kernels"]
                fw = sum(v["read_bytes"] + v["write_bytes"] for k, v in kern.items()
                         if k.startswith("fwd_kernel"))
                bw = sum(v["read_bytes"] + v["write_bytes"] for k, v in kern.items()
                         if k.startswith("bwd_dkdv") or k.startswith("bwd_dq"))
                rec["fwd_measured_gbs"] = round(fw / (t_fwd * 1e-3) / 1e9, 1)
                rec["bwd_measured_gbs"] = round(bw / (t_bwd * 1e-3) / 1e9, 1)
        out[name] = rec
        del buf, x
    return out


def _read(path):
    try:
        with open(path) as fh:
            return fh.read()
    except OSError:
        return ""


def cpu_baseline(x, heads=4):
    """The fp64 oracle (as it stands), timed on the host on the first ``heads`` (b, h)
    heads of the same workload; rate = their allowed-pair FLOP / wall time."""
    import threadpoolctl
    from oracle import attention as orc
    wl = x.wl
    sel = [(b, h) for b in range(wl.B) for h in range(wl.H)][:heads]
    flop = 0.0
    t0 = time.perf_counter()
    for b, h in sel:
        kv = None if x.kv_len is None else int(x.kv_len[b])
        args = [orc.as_f64(t[b, h]) for t in (x.q, x.k, x.v, x.do)]
        drop = None if wl.dropout is None else (*wl.dropout, b * wl.H + h)
        orc.head_backward(*args, wl.scale, wl.causal, x.blockmask, kv, window=wl.window,
                          dropout=drop)
        flop += 14.0 * allowed_pairs(wl.N, wl.causal, x.blockmask, kv, wl.window) * wl.d
    dt = time.perf_counter() - t0
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{len(sel)} of {wl.B * wl.H} heads of {wl.name} (N={wl.N}, d={wl.d}): "
                      f"fp64 forward+backward with S and P materialised, numpy/OpenBLAS, "
                      f"{dt:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: libfa is measured on one GPU only (asked for --gpus {args.gpus}); "
              "how the path would shard over several GPUs is described in the design notes, "
              "not implemented.", file=sys.stderr)
        sys.exit(2)
    import torch
    from exact_io_aware_46_amd import inputs as inp

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = inp.WORKLOADS[args.workload]
    x = inp.make_inputs(wl)
    if wl.dtype == "fp8":
        fp8_main(args, torch, wl, x)
        return
    pairs = workload_pairs(x)
    fl_fwd, fl_bwd = 4.0 * pairs * wl.d, 10.0 * pairs * wl.d
    buf = Buffers(x, torch)

    if args.eager:
        f_step, f_fwd, f_bwd, f_pre = buf.step, buf.fwd, buf.bwd, buf.pre
    else:
        f_step, f_fwd, f_bwd, f_pre = (graphed(torch, f)
                                       for f in (buf.step, buf.fwd, buf.bwd, buf.pre))
    ms_step = time_loop(torch, f_step, args.steps, args.warmup)
    ms_fwd = time_loop(torch, f_fwd, args.steps, args.warmup)
    ms_bwd = time_loop(torch, f_bwd, args.steps, args.warmup)
    ms_pre = time_loop(torch, f_pre, args.steps, args.warmup)
    # The backward's row statistics (D, LSE * log2(e)) are formed at the start of its dQ
    # kernel; the standalone preprocess entry point is timed apart and not subtracted.
    ms_bwd_main = ms_bwd

    tf_step = (fl_fwd + fl_bwd) / (ms_step * 1e-3) / 1e12
    tf_fwd = fl_fwd / (ms_fwd * 1e-3) / 1e12
    tf_bwd_main = fl_bwd / (ms_bwd_main * 1e-3) / 1e12
    # Kernel template names as the profiler prints them.
    tn = "fa::F16" if wl.dtype == "f16" else "fa::Bf16"
    dr = "true" if wl.dropout is not None and wl.dropout[0] > 0 else "false"
    kd = 256 if wl.d > 128 else 128 if wl.d > 64 else 64      # kernel (LDS layout) head dim
    pad = "false" if wl.d == kd else "true"                    # rows narrower than kd
    dc = wl.d if wl.d in (32, 96) else kd                      # head dim computed on
    nw = 4 if kd == 256 else 8                                 # waves per workgroup
    # the 64-wide forward and dQ kernels run four-wave workgroups under a block table; the
    # forward also when its eight-wave grid is under two workgroups per CU
    nwq = 4 if kd == 64 and wl.mask == "block" and dr == "false" else nw
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    small = math.ceil(wl.N / 256) * wl.B * wl.H < 2 * cus
    nwf = 4 if kd == 64 and dr == "false" and (wl.mask == "block" or small) else nw
    rk = kd == 128 or (kd == 64 and dr == "false")             # one-wave dK/dV kernel
    k_dkdv = (f"bwd_dkdv_rk_kernel<{tn}, {kd}, {dr}, {pad}, {dc}>" if rk
              else f"bwd_dkdv_kernel<{tn}, {kd}, {dr}, {pad}, {dc}, {nw}>")
    bc = 128 if kd == 128 else 64                              # forward key tile
    bcq = 128 if kd <= 128 else 64                             # dQ key tile
    k_dq = f"bwd_dq_kernel<{tn}, {kd}, {bcq}, {dr}, {pad}, {dc}, {nwq}>"
    k_fwd = f"fwd_kernel<{tn}, {kd}, {bc}, {dr}, {pad}, {dc}, {nwf}>"
    rec = {
        "metric": METRIC, "value": round(tf_step, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "causal": wl.causal, "mask": wl.mask, "window": wl.window,
                   "dropout": None if wl.dropout is None else wl.dropout[0],
                   "scale": wl.scale,
                   "allowed_pairs": pairs},
        "fwd_tflops": round(tf_fwd, 2), "fwd_ms": round(ms_fwd, 4),
        "fwd_bwd_tflops": round(tf_step, 2),
        "fwd_pct_mfma_peak": round(100 * tf_fwd / MFMA_BF16_PEAK_TFLOPS, 2),
        "fwd_bwd_pct_mfma_peak": round(100 * tf_step / MFMA_BF16_PEAK_TFLOPS, 2),
        "bwd_ms": round(ms_bwd, 4), "bwd_preprocess_ms": round(ms_pre, 4),
        "timing_mode": "direct calls" if args.eager else "HIP graph replay of each call",
        "timing_ms": {"step": timing_record(ms_step), "fwd": timing_record(ms_fwd),
                      "bwd": timing_record(ms_bwd), "bwd_preprocess": timing_record(ms_pre)},
        "fwd_bwd_tflops_at_median": round((fl_fwd + fl_bwd) / (ms_step.median * 1e-3) / 1e12, 2),
        "fwd_tflops_at_median": round(fl_fwd / (ms_fwd.median * 1e-3) / 1e12, 2),
        "roofline": {"kernel": f"{k_dq} (row statistics at its start) + {k_dkdv} (the whole backward)",
                     "bound": "mfma", "achieved": round(tf_bwd_main, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_bwd_main / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(
                         wl.name, "bwd_kernel", [k_dkdv, k_dq])},
        "roofline_fwd": {"kernel": k_fwd, "bound": "mfma",
                         "achieved": round(tf_fwd, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf_fwd / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(wl.name, "fwd_kernel", [k_fwd])},
    }
    peak = mfma_peak_record("bf16")
    rec["mfma_peak"] = peak
    if "tflops" in peak:
        m = peak["tflops"]
        rec["fwd_pct_measured_mfma_peak"] = round(100 * tf_fwd / m, 2)
        rec["fwd_bwd_pct_measured_mfma_peak"] = round(100 * tf_step / m, 2)
        rec["roofline"]["frac_of_measured_peak"] = round(tf_bwd_main / m, 4)
        rec["roofline_fwd"]["frac_of_measured_peak"] = round(tf_fwd / m, 4)
    rec["device"] = None if args.no_device_sample else device_sample(torch, buf.step)
    rec["context"] = {"note": "the pages' figures on their own hardware; context only",
                      "source": "IO感知计算如何重塑Transformer内存优化技术格局 (bxzpzcl.cn), "
                                "sections 技术演进时间线 and NVIDIA CUDA平台优化",
                      "items": PAGE_CONTEXT}
    if not args.no_footprint and wl.name == "long_causal_16k":
        del buf
        rec["footprint"] = footprint_sweep(torch, wl)
    if not args.no_other_configs and wl.name == "long_causal_16k":
        rec["other_configs"] = other_configs(torch, inp, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x)
        rec["cpu_baseline"]["gpu_over_cpu"] = round(rec["value"] / rec["cpu_baseline"]["value"], 1)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
