#!/usr/bin/env python3
"""Throughput of the FlashAttention-2 backward on one MI355X (gfx950).

One step = one complete backward call (fab_bwd: preprocess D = rowsum(dO*O), the key-tile
outer dK/dV kernel and the query-tile outer dQ kernel) over the headline workload -- bf16,
grouped-query (32 query heads on 8 kv heads), causal, B=2, S=4096, D=128 -- with every input
(Q, K, V, dO and the forward's O and LSE) already resident in HBM.  The forward that produces
O and LSE is not part of a step; it is timed on its own afterwards and reported beside the
metric (`forward`, counting 4*B*H*Sq*Sk*D FLOPs, halved when causal).

Metric: attention-backward TFLOP/s counting 10*B*H*Sq*Sk*D FLOPs per step, halved when causal
(the five contractions over the pairs the method must visit), and its fraction of MI355X's
dense bf16 MFMA peak (2516.6 TFLOP/s).

Printed (rank 0, one JSON line): the step throughput, a `roofline` object for the dominant
kernel (its own algorithmic FLOPs per launch over its average launch time, timed with events
on the launch stream) and a `cpu_baseline` object (the fp64 oracle's backward on a bounded
sample of the same workload, timed on this host's cores before the GPU is touched).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
       python bench.py --only {bwd,dkdv,dq,preprocess,fwd,copy}   (a launch loop for rocprofv3)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}  # dense, AMD public spec
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "flashattention_backward_amd", "csrc")

# Contractions each kernel performs per allowed (b, h, query, key) pair, in units of 2*D FLOPs:
# the dK/dV kernel forms S, dP, dV and dK; the dQ kernel dQ alone from stored dS, or S, dP and
# dQ where it recomputes dS.
KERNEL_CONTRACTIONS = {"stored_ds": {"bwd_dkdv": 4, "bwd_dq": 1},
                       "recompute": {"bwd_dkdv": 4, "bwd_dq": 3}}
MODES = ("best", "stored_ds", "recompute")
KERNEL_SOURCE = {"bwd_dkdv": "bwd16.hip", "bwd_dq": "bwd16.hip", "bwd_dkdv_ds": "bwd16.hip",
                 "bwd_dq_ds": "bwd16.hip", "preprocess": "preprocess.hip"}


def allowed_pairs(w) -> float:
    return w.allowed_pairs()


def source_digest(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the kernel's sources with // comments and blank space
    removed, so that only a change to the code itself invalidates recorded counters."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kernel], "common.h", "launch.h"):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def recorded_value(kernel: str, workload: str, what: str, key: str):
    """A figure from a committed rocprofv3 counter summary (profiles/<kernel>_<workload>_<what>.md,
    line `key: value`), if it was taken on the current kernel source (same digest); else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_{what}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    dig = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    val = re.search(key + r":\s*([0-9.eE+-]+)", text)
    if not dig or not val or dig.group(1) != source_digest(kernel):
        return None
    return float(val.group(1))


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) on the current source."""
    return recorded_value(kernel, workload, "hbm_traffic", "hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- CPU baseline
def _oracle_group(args):
    q, k, v, do, causal, scale = args
    from threadpoolctl import threadpool_limits

    import oracle
    with threadpool_limits(1):
        t0 = time.perf_counter()
        o, lse = oracle.attention_forward(q, k, v, causal, scale)
        t1 = time.perf_counter()
        oracle.attention_backward(do, q, k, v, o, lse, causal, scale)
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def blas_build() -> str:
    """NumPy's BLAS as its build configuration reports it (name, version, configuration)."""
    import numpy as np
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        cfg = blas.get("openblas configuration") or ""
        return f"{blas.get('name', '?')} {blas.get('version', '?')}" + (f" ({cfg.strip()})" if cfg else "")
    except Exception as e:  # an older NumPy without dict mode
        return f"unknown ({type(e).__name__})"


def cpu_baseline(w, q, k, v, do, max_groups=None):
    """The fp64 oracle (as it stands) on a bounded sample: whole (batch, kv-head) groups, one
    single-threaded worker process per group, one group per available core.  Runs before the
    GPU is initialised (workers are forked)."""
    import multiprocessing as mp
    import numpy as np
    cores = len(os.sched_getaffinity(0))
    groups = [(b, g) for b in range(w.B) for g in range(w.H_kv)]
    n = min(len(groups), cores if max_groups is None else max_groups)
    sample = groups[:n]
    G = w.group
    tasks = []
    for b, g in sample:
        hs = slice(g * G, (g + 1) * G)
        tasks.append((q[b:b + 1, hs].double().numpy(), k[b:b + 1, g:g + 1].double().numpy(),
                      v[b:b + 1, g:g + 1].double().numpy(), do[b:b + 1, hs].double().numpy(),
                      w.causal, w.scale))
    t0 = time.perf_counter()
    pool = mp.get_context("fork").Pool(n)
    try:
        times = pool.map(_oracle_group, tasks)
    finally:
        # close + join lets the workers exit on their own; leaving a `with` block would
        # terminate() them with SIGTERM instead
        pool.close()
        pool.join()
    wall = time.perf_counter() - t0
    bwd_wall = max(t[1] for t in times)
    pairs = n * G * w.Sq * w.Sk / (2 if w.causal else 1)
    flops = 10.0 * w.D * pairs
    return {
        "value": flops / bwd_wall / 1e12,
        "unit": "TFLOP/s",
        "cores": n,
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle backward for {n} of {len(groups)} (batch, kv-head) groups "
                   f"({n * G} of {w.B * w.H} query heads) of {w.name}, one single-threaded "
                   f"process per group; backward wall {bwd_wall:.2f} s (forward, untimed in "
                   f"value: {max(t[0] for t in times):.2f} s); total {wall:.2f} s; NumPy BLAS: "
                   f"{blas_build()}, one thread per process"),
    }


# ----------------------------------------------------------------------------- GPU timing
class Bwd:
    """Preallocated buffers and raw C-ABI calls for one workload (no allocation per step)."""

    def __init__(self, w, q, k, v, do, mode="best"):
        import torch

        import flashattention_backward_amd as fab
        self.w, self.fab, self.L = w, fab, fab.lib()
        dev = torch.device("cuda:0")
        self.q, self.k, self.v, self.do = (x.to(dev) for x in (q, k, v, do))
        self.o, self.lse = fab.fwd(self.q, self.k, self.v, causal=w.causal, scale=w.scale,
                                   window_size=w.window)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.k)
        self.dv = torch.empty_like(self.v)
        self.code = fab.DTYPE_CODES[str(self.q.dtype).replace("torch.", "")]
        # the workspace size selects the mode: the library's recommendation ("best"), or one
        # forced (the stored-dS size falls back to the recompute size where that mode cannot run)
        nb = fab.bwd_workspace_bytes(w.B, w.H, w.H_kv, w.Sq, w.Sk, w.D, self.code,
                                     store_ds={"best": None, "stored_ds": True, "recompute": False}[mode])
        nmin = fab.bwd_workspace_bytes(w.B, w.H, w.H_kv, w.Sq, w.Sk, w.D, self.code, store_ds=False)
        self.mode = "stored_ds" if nb > nmin else "recompute"
        self.plan = fab.bwd_plan(w.B, w.H, w.H_kv, w.Sq, w.Sk, w.D, self.code, nb)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        self.dims = (w.B, w.H, w.H_kv, w.Sq, w.Sk, w.D, self.code, int(w.causal), w.window,
                     float(w.scale))
        torch.cuda.synchronize()

    def _ok(self, st):
        if st != 0:
            raise RuntimeError(self.L.fab_last_error().decode())

    def bwd(self):
        self._ok(self.L.fab_bwd(self.do.data_ptr(), self.q.data_ptr(), self.k.data_ptr(),
                                self.v.data_ptr(), self.o.data_ptr(), self.lse.data_ptr(),
                                self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(),
                                self.ws.data_ptr(), self.ws.numel(), *self.dims, self.stream))

    def fwd(self):
        """The supporting forward into the preallocated O and LSE (not part of the metric)."""
        w = self.w
        self._ok(self.L.fab_fwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                self.o.data_ptr(), self.lse.data_ptr(), w.B, w.H, w.H_kv, w.Sq, w.Sk,
                                w.D, self.code, int(w.causal), w.window, float(w.scale), self.stream))

    def preprocess(self):
        w = self.w
        self._ok(self.L.fab_bwd_preprocess(self.do.data_ptr(), self.o.data_ptr(), self.lse.data_ptr(),
                                           self.ws.data_ptr(), self.ws.numel(),
                                           w.B, w.H, w.Sq, w.D, self.code, self.stream))

    def dkdv(self):
        self._ok(self.L.fab_bwd_dkdv(self.do.data_ptr(), self.q.data_ptr(), self.k.data_ptr(),
                                     self.v.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                                     self.dk.data_ptr(), self.dv.data_ptr(), *self.dims, self.stream))

    def dq_(self):
        self._ok(self.L.fab_bwd_dq(self.do.data_ptr(), self.q.data_ptr(), self.k.data_ptr(),
                                   self.v.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                                   self.dq.data_ptr(), *self.dims, self.stream))


def settle(fn, seconds=0.3):
    """Untimed calls of fn() until the GPU has been busy for about `seconds`, so that the
    timed region starts at the steady clock rather than during the clock ramp."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def time_launches(fn, steps, warmup):
    """Average milliseconds per call of fn() over `steps` calls, timed with events recorded
    on the stream the library launches on (torch's current stream)."""
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_ms(fn, calls):
    """Milliseconds of each of `calls` calls of fn(), each between its own pair of events
    recorded on the launch stream (inputs stay resident; caches are not flushed)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def call_stats(ms):
    """Median, minimum and 90th percentile (linear interpolation) of per-call times."""
    x = sorted(ms)
    def pct(q):
        pos = q * (len(x) - 1)
        lo = int(pos)
        hi = min(lo + 1, len(x) - 1)
        return x[lo] + (x[hi] - x[lo]) * (pos - lo)
    return {"calls": len(x), "median": round(pct(0.5), 4), "min": round(x[0], 4),
            "p90": round(pct(0.9), 4)}


PEAK_CLOCK_MHZ = 2400.0  # the clock the dense MFMA peaks assume (MI355X spec)


def device_info():
    """Name, architecture and compute units of cuda:0 as the runtime reports them."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count}


def clock_under_load(fn, ms_target=60.0):
    """Median shader clock (MHz) while `fn` runs back to back, outside the timed region:
    about ms_target of calls are queued, then the current GFX clock is read (amdsmi, through
    torch.cuda.clock_rate) until they have finished.  None where the clock cannot be read."""
    import torch
    try:
        torch.cuda.clock_rate(0)
    except Exception:
        return None
    t = time_launches(fn, 3, 1)
    n = max(4, int(ms_target / max(t, 1e-3)))
    done = torch.cuda.Event()
    for _ in range(n):
        fn()
    done.record()
    samples = []
    while not done.query():
        try:
            c = float(torch.cuda.clock_rate(0))
        except Exception:
            break
        if c > 0:
            samples.append(c)
        time.sleep(0.002)
    torch.cuda.synchronize()
    if not samples:
        return None
    samples.sort()
    return samples[len(samples) // 2]


def bench_workload(w, steps, warmup, with_cpu, inputs=None, mode="best"):
    import torch
    q, k, v, do = inputs if inputs is not None else workloads.make_inputs(w)
    cpu = cpu_baseline(w, q, k, v, do) if with_cpu else None
    b = Bwd(w, q, k, v, do, mode=mode)
    torch.cuda.synchronize()
    settle(b.bwd)
    # the timed region: `steps` whole backward calls, synchronised on both sides
    for _ in range(warmup):
        b.bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        b.bwd()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = e0.elapsed_time(e1) / steps
    # the distribution over single calls (a separate loop after the timed region)
    calls = call_stats(per_call_ms(b.bwd, max(steps, 20)))
    # per-kernel launch times (separate loops, same stream; in the stored-dS mode the dQ loop
    # reads the dS that the dK/dV loop stored)
    k_ms = {"preprocess": time_launches(b.preprocess, steps, warmup),
            "bwd_dkdv": time_launches(b.dkdv, steps, warmup),
            "bwd_dq": time_launches(b.dq_, steps, warmup)}
    # the supporting forward, reported beside the metric (4 of the 10 counted units per pair);
    # it rewrites the same O and LSE, so the backward's inputs do not change
    fwd_ms = time_launches(b.fwd, steps, warmup)
    # the clock the backward runs at (a separate loop, after everything timed above)
    clk = clock_under_load(b.bwd)
    fwd_tflops = 0.4 * w.bwd_flops() / (fwd_ms * 1e-3) / 1e12
    flops = w.bwd_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    # the kernels of the path, named by role and mode (in the stored-dS mode the dK/dV kernel
    # also writes dS and the dQ kernel is the contraction over it)
    tag = "_ds" if b.mode == "stored_ds" else ""
    names = {"bwd_dkdv": "bwd_dkdv" + tag, "bwd_dq": "bwd_dq" + tag, "preprocess": "preprocess"}
    dom = max(("bwd_dkdv", "bwd_dq"), key=lambda n: k_ms[n])
    kflops = 2.0 * w.D * KERNEL_CONTRACTIONS[b.mode][dom] * allowed_pairs(w)
    achieved = kflops / (k_ms[dom] * 1e-3) / 1e12
    es = 4 if w.dtype == "fp32" else 2
    pre_bytes = w.B * w.H * w.Sq * (2 * w.D * es + 4 + 8)  # read dO, O, LSE; write {LSE', D}
    kernels = {}
    for role in ("bwd_dkdv", "bwd_dq"):
        kf = 2.0 * w.D * KERNEL_CONTRACTIONS[b.mode][role] * allowed_pairs(w)
        kernels[names[role]] = {"ms": round(k_ms[role], 4), "bound": "mfma",
                                "achieved_TFLOPs": round(kf / (k_ms[role] * 1e-3) / 1e12, 2),
                                "frac_of_peak": round(kf / (k_ms[role] * 1e-3) / 1e12 / peak, 4),
                                "mfma_busy": recorded_value(names[role], w.name, "counters", "mfma_busy_frac"),
                                "traffic": recorded_traffic(names[role], w.name)}
    if b.mode == "stored_ds":
        # dQ = scale dS K streams dS from HBM: its algorithmic bytes are dS (2 bytes per allowed
        # pair), K once and dQ once
        qb = 2.0 * allowed_pairs(w) + (w.B * w.H_kv * w.Sk + w.B * w.H * w.Sq) * w.D * es
        kd = kernels[names["bwd_dq"]]
        kd.update({"bound": "hbm", "algorithmic_bytes": qb,
                   "achieved_GBps": round(qb / (k_ms["bwd_dq"] * 1e-3) / 1e9, 1),
                   "frac_of_hbm_peak": round(qb / (k_ms["bwd_dq"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    kernels["preprocess"] = {"ms": round(k_ms["preprocess"], 4), "bound": "hbm", "algorithmic_bytes": pre_bytes,
                             "achieved_GBps": round(pre_bytes / (k_ms["preprocess"] * 1e-3) / 1e9, 1),
                             "frac_of_hbm_peak": round(pre_bytes / (k_ms["preprocess"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "on_path": b.plan != "recompute",
                             "traffic": recorded_traffic("preprocess", w.name)}
    if b.plan == "recompute":
        # step 1 runs in the dQ kernel's prologue: its cost is what fab_bwd takes beyond the
        # dK/dV kernel and the dQ kernel without it (one launch gap included)
        kernels["preprocess"]["fused_in_dq_ms_estimate"] = round(ms - k_ms["bwd_dkdv"] - k_ms["bwd_dq"], 4)
    line = {
        "metric": "attention-backward TFLOP/s (bf16, causal) and % of MI355X dense MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "Sq": w.Sq, "Sk": w.Sk,
                   "D": w.D, "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(tflops / peak, 4),
        "mode": b.mode,
        "plan": b.plan,
        "workspace_bytes": int(b.ws.numel()),
        "wall_ms_per_step": round(wall_ms, 4),
        "per_call_ms": calls,
        "caches": "L2 and MALL are not flushed between calls",
        "device": dict(device_info(), clock_mhz_under_load=clk,
                       frac_of_peak_at_measured_clock=(round(tflops / (peak * clk / PEAK_CLOCK_MHZ), 4)
                                                       if clk else None)),
        "kernel_ms": {n: round(t, 4) for n, t in k_ms.items()},
        "kernels": kernels,
        "preprocess_GBps": round(pre_bytes / (k_ms["preprocess"] * 1e-3) / 1e9, 1),
        "forward": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tflops, 2),
                    "frac_of_peak": round(fwd_tflops / peak, 4)},
        "roofline": {
            "kernel": names[dom],
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(names[dom], w.name),
            "mfma_busy": recorded_value(names[dom], w.name, "counters", "mfma_busy_frac"),
            "flops_per_launch": kflops,
        },
        "cpu_baseline": cpu,
    }
    return line


def only_mode(w, what, steps, warmup, mode="best"):
    """A bare launch loop for rocprofv3 (no timing, no CPU baseline)."""
    import torch
    if what == "copy":
        # calibration: a plain device copy of known size for the HBM counters
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(warmup + steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": warmup + steps}), flush=True)
        return
    b = Bwd(w, *workloads.make_inputs(w), mode=mode)
    fn = {"bwd": b.bwd, "dkdv": b.dkdv, "dq": b.dq_, "preprocess": b.preprocess, "fwd": b.fwd}[what]
    if what in ("dkdv", "dq"):
        b.preprocess()
    if what == "dq":
        b.dkdv()  # the stored-dS dQ kernel reads what the dK/dV kernel stores
    for _ in range(warmup + steps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"only": what, "workload": w.name, "launches": warmup + steps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one JSON line per named workload (no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["bwd", "dkdv", "dq", "preprocess", "fwd", "copy"])
    ap.add_argument("--mode", choices=MODES, default="best",
                    help="how dQ is formed: the library's recommendation for the workload (default), "
                         "from the dS the dK/dV kernel stores, or by recomputing S and dP")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    w = workloads.get(args.workload)
    if args.only:
        only_mode(w, args.only, args.steps, args.warmup, args.mode)
        return
    if args.all:
        for name in workloads.WORKLOADS:
            print(json.dumps(bench_workload(workloads.get(name), args.steps, args.warmup, False,
                                            mode=args.mode)), flush=True)
        return
    line = bench_workload(w, args.steps, args.warmup, not args.no_cpu_baseline, mode=args.mode)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
