#!/usr/bin/env python3
"""Throughput of the 3-D max-pooling path on one MI355X.

One step runs the whole path once over the five named synthetic workloads:
the forward (window max + int32 argmax) of all five, then the backward of
the four that have one, each through the C ABI on the current stream:

  adaptive_f32_divisible  float32 (2,3,8,8,8) -> (4,4,4)      fwd + gather bwd
  adaptive_bf16_ties      bfloat16 (4,16,10,10,10) -> (8,8,8) fwd + accumulate bwd
  fixed_bf16_k2s2         bfloat16 (16,64,16,112,112) k2 s2   fwd only
  fixed_f16_k3s2          float16 (8,128,32,56,56) k3 s2      fwd + accumulate bwd
  adaptive_f32_large      float32 (32,256,16,32,32) -> (5,7,7) fwd + accumulate bwd

Inputs (x, grad_output) are drawn once on the CPU from fixed seeds and are
resident in HBM before timing; outputs are preallocated.  The metric is
effective HBM bandwidth: algorithmic bytes (every input read once, every
output written once: |x|+|y|+|idx| forward, |gy|+|idx|+|gx| backward) per
second, as a fraction of the 8 TB/s peak.

Timing passes:
  1. ``value``: K whole steps launched back to back between two
     synchronisations (host clock).
  2. ``per_op_step``: the same K steps with every call's kernel time taken
     by the library's timing hook (mp3d_time_next_call: hipExtLaunchKernel
     events that carry the kernel's own start and end, no extra packets).
  3. ``per_config``: each workload on its own, K iterations of [untimed read
     of a 1 GiB buffer, which evicts L2 and the 256 MB memory-side cache and
     leaves them clean; forward; backward], the kernel time of each call by
     the timing hook; median, min, p90, and forward + backward combined
     against the 70 % target.  The roofline of the dominant kernel (largest
     median) comes from this pass.
  Variants (values-only forward, int64 indices, padding, ordered and
  index-free backward, float64, the divisible gather at scale) and the
  small shapes of the PR #308 page's latency table are timed the same way.

Beside the GPU figures, the CPU oracle is timed on the same workloads
(``cpu_baseline``: one thread; ``cpu_baseline_threads``: the host's CPUs, up
to 16, each thread running the unchanged oracle on a range of planes).

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this path runs on one
GPU (planes shard across GPUs with no communication, so more GPUs are not
measured here).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
TARGET_FRAC = 0.70
METRIC = "effective HBM GB/s (bytes read+written / time) fwd+bwd; % of MI355X HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the PR #308 page's own latency for float16 (2,8,4,4,4) adaptive backward
# on its Moore Threads GPU (Performance table): context, not a target
PR308_CONTEXT_US = 3.0


def kernel_source_hash() -> str:
    """Hash of the HIP sources; stored traffic counters are reported only
    while it matches the hash they were measured at."""
    from bwd_max_pool3d_amd import _build
    h = hashlib.sha256()
    headers = sorted(os.path.join(_build.CSRC, f) for f in os.listdir(_build.CSRC)
                     if f.endswith(".hpp"))
    for path in _build.sources() + headers:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Hip:
    """Events of the HIP runtime already loaded by torch (same soname as the
    one libmp3d.so links against, so one runtime serves both)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.pool = []
        self.used = 0

    def pair(self):
        while self.used + 2 > len(self.pool):
            ev = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed (%d)" % rc)
            self.pool.append(ev.value)
        a, b = self.pool[self.used], self.pool[self.used + 1]
        self.used += 2
        return a, b

    def reset(self):
        self.used = 0

    def elapsed_us(self, a, b) -> float:
        f = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return f.value * 1e3


class Op:
    """One C-ABI call, with its inputs and preallocated outputs."""

    def __init__(self, wl, kind, fn, nbytes, elems, note, out_elems=None):
        self.wl, self.kind, self.fn, self.nbytes, self.elems, self.note = (
            wl, kind, fn, nbytes, elems, note)
        self.out_elems = out_elems     # pooled outputs (y / gy elements) per call
        self.us = []           # kernel times, microseconds

    @property
    def name(self):
        return "%s.%s" % (self.wl.name if hasattr(self.wl, "name") else self.wl, self.kind)


def stats(v):
    s = sorted(v)
    n = len(s)
    return {"median": s[n // 2], "min": s[0], "p90": s[min(n - 1, (9 * n) // 10)],
            "mean": sum(s) / n, "n": n}


def op_row(op, key="median"):
    st = stats(op.us)
    t = st[key]
    return {"op": op.name, "us": round(t, 3), "us_median": round(st["median"], 3),
            "us_min": round(st["min"], 3), "us_p90": round(st["p90"], 3),
            "us_mean": round(st["mean"], 3), "n": st["n"], "bytes": op.nbytes,
            "GB_s": round(op.nbytes / (t * 1e-6) / 1e9, 1),
            "elems_per_s": round(op.elems / (t * 1e-6), 1),
            "out_elems_per_s": (round(op.out_elems / (t * 1e-6), 1)
                                if op.out_elems is not None else None),
            "frac_of_peak": round(op.nbytes / (t * 1e-6) / 1e9 / PEAK_GBS, 4),
            "note": op.note}


def build_ops(torch, mp, workloads, variants=True):
    """The step's ops (forwards, then backwards) and, apart from the step,
    the variants."""
    fwd_ops, bwd_ops, vo_ops, ord_ops, exf_ops, exb_ops = [], [], [], [], [], []
    for wl in workloads.WORKLOADS:
        x = wl.make_x().cuda()
        N, C, D, H, W = wl.shape
        if wl.adaptive:
            o3 = tuple(wl.out)
        else:
            o3 = tuple(mp.mp3d_out_size(X, k, s) for X, k, s in zip(wl.shape[2:], wl.kernel, wl.stride))
        oshape = (N, C) + o3
        y = torch.empty(oshape, dtype=x.dtype, device="cuda")
        idx = torch.empty(oshape, dtype=torch.int32, device="cuda")
        es = x.element_size()
        nin, nout = x.numel(), y.numel()
        fbytes = nin * es + nout * es + nout * 4
        if wl.adaptive:
            f = (lambda x=x, o3=o3, y=y, idx=idx: mp.amp3d_forward(x, o3, out=(y, idx)))
        else:
            f = (lambda x=x, wl=wl, y=y, idx=idx: mp.mp3d_forward(x, wl.kernel, wl.stride, out=(y, idx)))
        fwd_ops.append(Op(wl, "fwd", f, fbytes, nin, "forward", out_elems=nout))
        if wl.adaptive:
            v = (lambda x=x, o3=o3, y=y: mp.amp3d_forward(x, o3, out=y, indices=False))
        else:
            v = (lambda x=x, wl=wl, y=y: mp.mp3d_forward(x, wl.kernel, wl.stride, out=y,
                                                         indices=False))
        vo_ops.append(Op(wl, "fwd_values", v, nin * es + nout * es, nin, "values-only forward"))
        if wl.backward:
            gy = wl.make_gy(oshape).cuda()
            gx = torch.empty(wl.shape, dtype=x.dtype, device="cuda")
            bbytes = nout * es + nout * 4 + nin * es
            b = (lambda gy=gy, idx=idx, wl=wl, gx=gx: mp.mp3d_backward(
                gy, idx, wl.shape, kernel=wl.kernel, stride=wl.stride, out=gx))
            bwd_ops.append(Op(wl, "bwd", b, bbytes, nin, "backward", out_elems=nout))
            o = (lambda gy=gy, idx=idx, wl=wl, gx=gx: mp.mp3d_backward(
                gy, idx, wl.shape, kernel=wl.kernel, stride=wl.stride, overlap=2, out=gx))
            ord_ops.append(Op(wl, "bwd_ordered", o, bbytes, nin, "ordered backward"))
            geo = dict(kernel=None) if wl.adaptive else dict(kernel=wl.kernel, stride=wl.stride)
            rc = (lambda x=x, y=y, gy=gy, gx=gx, geo=geo: mp.mp3d_backward_recompute(
                x, y, gy, out=gx, **geo))
            ord_ops.append(Op(wl, "bwd_recompute", rc, nin * es + 2 * nout * es + nin * es, nin,
                              "index-free backward (argmax recomputed from x and y)"))
            ws = torch.empty(mp.recompute_workspace_size(x.dtype, N, C, o3), dtype=torch.uint8,
                             device="cuda")
            rw = (lambda x=x, y=y, gy=gy, gx=gx, geo=geo, ws=ws: mp.mp3d_backward_recompute(
                x, y, gy, out=gx, workspace=ws, **geo))
            ord_ops.append(Op(wl, "bwd_recompute_ws", rw, nin * es + 2 * nout * es + nin * es,
                              nin, "index-free backward through a workspace (the forward into "
                              "it, its argmax checked against y)"))
            ro = (lambda x=x, y=y, gy=gy, gx=gx, geo=geo: mp.mp3d_backward_recompute(
                x, y, gy, out=gx, overlap=2, **geo))
            ord_ops.append(Op(wl, "bwd_recompute_ordered", ro, nin * es + 2 * nout * es + nin * es,
                              nin, "ordered index-free backward, one pass"))
            rwo = (lambda x=x, y=y, gy=gy, gx=gx, geo=geo, ws=ws: mp.mp3d_backward_recompute(
                x, y, gy, out=gx, overlap=2, workspace=ws, **geo))
            ord_ops.append(Op(wl, "bwd_recompute_ws_ordered", rwo,
                              nin * es + 2 * nout * es + nin * es, nin,
                              "ordered index-free backward through a workspace"))
        elif variants and not wl.adaptive:
            # the divisible gather at scale: this workload's windows tile
            # every axis, so its backward is the gather (overlap 0)
            gy = wl.make_gy(oshape).cuda()
            gx = torch.empty(wl.shape, dtype=x.dtype, device="cuda")
            g = (lambda gy=gy, idx=idx, wl=wl, gx=gx: mp.mp3d_backward(
                gy, idx, wl.shape, kernel=wl.kernel, stride=wl.stride, overlap=0, out=gx))
            exb_ops.append(Op(wl, "bwd_gather", g, nout * es + nout * 4 + nin * es, nin,
                              "divisible backward (gather: no zero pass, no atomics)"))
        if not variants:
            continue
        idx64 = torch.empty(oshape, dtype=torch.int64, device="cuda")
        if wl.adaptive:
            f64 = (lambda x=x, o3=o3, y=y, i=idx64: mp.amp3d_forward(
                x, o3, out=(y, i), index_dtype=torch.int64))
        else:
            f64 = (lambda x=x, wl=wl, y=y, i=idx64: mp.mp3d_forward(
                x, wl.kernel, wl.stride, out=(y, i), index_dtype=torch.int64))
        exf_ops.append(Op(wl, "fwd_i64", f64, nin * es + nout * es + nout * 8, nin,
                          "forward, int64 indices"))
        if not wl.adaptive:
            pad = tuple(k // 2 for k in wl.kernel)
            po3 = tuple(mp.mp3d_out_size_ex(X, k, s, p) for X, k, s, p in
                        zip(wl.shape[2:], wl.kernel, wl.stride, pad))
            pshape = (N, C) + po3
            py = torch.empty(pshape, dtype=x.dtype, device="cuda")
            pidx = torch.empty(pshape, dtype=torch.int32, device="cuda")
            npo = py.numel()
            fp = (lambda x=x, wl=wl, pad=pad, py=py, pidx=pidx: mp.mp3d_forward_ex(
                x, wl.kernel, wl.stride, pad, out=(py, pidx)))
            exf_ops.append(Op(wl, "fwd_pad", fp, nin * es + npo * es + npo * 4, nin,
                              "forward, padding k//2"))
            if wl.backward:
                fp()
                pgy = wl.make_gy(pshape).cuda()
                pgx = torch.empty(wl.shape, dtype=x.dtype, device="cuda")
                bp = (lambda g=pgy, i=pidx, wl=wl, pad=pad, gx=pgx: mp.mp3d_backward_ex(
                    g, i, wl.shape, wl.kernel, wl.stride, pad, out=gx))
                exb_ops.append(Op(wl, "bwd_pad", bp, npo * es + npo * 4 + nin * es, nin,
                                  "backward, padding k//2"))
    for wl in workloads.WORKLOADS:
        if not variants or not wl.backward or wl.shape[0] <= 4:
            continue
        x = wl.make_x().to(torch.float64).cuda()
        if wl.adaptive:
            o3 = tuple(wl.out)
        else:
            o3 = tuple(mp.mp3d_out_size(X, k, s) for X, k, s in zip(wl.shape[2:], wl.kernel, wl.stride))
        oshape = wl.shape[:2] + o3
        y = torch.empty(oshape, dtype=torch.float64, device="cuda")
        idx = torch.empty(oshape, dtype=torch.int32, device="cuda")
        gy = wl.make_gy(oshape).to(torch.float64).cuda()
        gx = torch.empty_like(x)
        nin, nout = x.numel(), y.numel()
        if wl.adaptive:
            f = (lambda x=x, o3=o3, y=y, idx=idx: mp.amp3d_forward(x, o3, out=(y, idx)))
        else:
            f = (lambda x=x, wl=wl, y=y, idx=idx: mp.mp3d_forward(x, wl.kernel, wl.stride,
                                                                out=(y, idx)))
        f()
        b = (lambda gy=gy, idx=idx, wl=wl, gx=gx: mp.mp3d_backward(
            gy, idx, wl.shape, kernel=wl.kernel, stride=wl.stride, out=gx))
        exf_ops.append(Op(wl, "fwd_f64", f, nin * 8 + nout * 12, nin, "forward, float64"))
        exb_ops.append(Op(wl, "bwd_f64", b, nout * 12 + nin * 8, nin, "backward, float64"))
        bo = (lambda gy=gy, idx=idx, wl=wl, gx=gx: mp.mp3d_backward(
            gy, idx, wl.shape, kernel=wl.kernel, stride=wl.stride, overlap=2, out=gx))
        exb_ops.append(Op(wl, "bwd_f64_ordered", bo, nout * 12 + nin * 8, nin,
                          "ordered backward, float64"))
    return fwd_ops, bwd_ops, (vo_ops + exf_ops + ord_ops + exb_ops) if variants else []


_CPU_INPUTS: dict = {}     # seeded workload tensors, drawn once for both oracle runs


def host_threads() -> int:
    """Host threads for the multi-threaded oracle run: the CPUs this process
    may use, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def host_cpu() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def cpu_baseline(target_s: float, threads: int = 1):
    """The CPU oracle on the same fraction of every workload's planes (so
    the byte mix matches the GPU step), sized to about ``target_s`` seconds.
    With ``threads`` > 1 the planes are split into that many contiguous
    ranges, each run by the unchanged oracle on a thread of its own (the
    ctypes call releases the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    import oracle
    from bwd_max_pool3d_amd import workloads

    orc = oracle.get()
    code = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    pool = ThreadPoolExecutor(threads) if threads > 1 else None

    def storage(t):
        t = t.contiguous()
        if t.dtype == torch.float32:
            return t.numpy()
        return t.view(torch.int16).numpy().view(np.uint16)

    cache = _CPU_INPUTS

    def draw(wl, kind, shape=None):
        if (wl.name, kind) not in cache:
            cache[(wl.name, kind)] = wl.make_x() if kind == "x" else wl.make_gy(shape)
        return cache[(wl.name, kind)]

    def ranges(n):
        cuts = np.linspace(0, n, min(threads, n) + 1).astype(int)
        return [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:])]

    def each(fn, parts):
        if pool is None:
            return [fn(*q) for q in parts]
        return list(pool.map(lambda q: fn(*q), parts))

    def run(frac):
        total_bytes = 0
        total_elems = 0
        elapsed = 0.0
        planes_used = []
        for wl in workloads.WORKLOADS:
            N, C, D, H, W = wl.shape
            P = N * C
            np_ = max(1, int(round(P * frac)))
            planes_used.append("%s:%d/%d" % (wl.name, np_, P))
            x = draw(wl, "x").reshape(P, 1, D, H, W)[:np_].contiguous()
            c = code[x.dtype]
            if wl.adaptive:
                o3, k, s = tuple(wl.out), (0, 0, 0), (0, 0, 0)
            else:
                k, s = wl.kernel, wl.stride
                o3 = tuple(orc.fixed_out(X, ka, sa) for X, ka, sa in zip(wl.shape[2:], k, s))
            es = x.element_size()
            xs = storage(x)
            parts = ranges(np_)
            t0 = time.perf_counter()
            fw = each(lambda a, b: orc.forward(xs[a:b], c, o3, k, s), parts)
            elapsed += time.perf_counter() - t0
            nin, nout = xs.size, sum(y.size for y, _ in fw)
            total_bytes += nin * es + nout * (es + 4)
            total_elems += nin
            if wl.backward:
                gy = draw(wl, "gy", (P, 1) + o3)[:np_].contiguous()
                gys = storage(gy)
                jobs = [(a, b, fw[j][1]) for j, (a, b) in enumerate(parts)]
                t0 = time.perf_counter()
                each(lambda a, b, idx: orc.backward(gys[a:b], idx, c, (b - a, 1, D, H, W),
                                                    side=False), jobs)
                elapsed += time.perf_counter() - t0
                total_bytes += nout * (es + 4) + nin * es
                total_elems += nin
        return total_bytes, elapsed, planes_used, total_elems

    probe = 1.0 / 512 * threads
    b, t, _, _ = run(probe)
    want = probe * target_s / max(t, 1e-3)
    frac = min(1.0, want)
    # when the whole step takes well under the target, it is run up to three
    # times and the median rate is reported
    reps = min(3, max(1, int(round(want)))) if want > 1.0 else 1
    runs = [run(frac) for _ in range(reps)]
    if pool is not None:
        pool.shutdown()
    mid = sorted(runs, key=lambda r: r[0] / r[1])[len(runs) // 2]
    rate, erate = mid[0] / mid[1], mid[3] / mid[1]
    b, t, used = runs[0][0], sum(r[1] for r in runs), runs[0][2]
    who = "one thread" if threads == 1 else "%d threads over contiguous plane ranges" % threads
    times = "" if reps == 1 else ", median of %d runs" % reps
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "elems_per_s": round(erate, 1),
            "sample": "plain C oracle, %s, forward+backward on %.4f of each "
                      "workload's planes (%s)%s: %.3g GB of algorithmic bytes per run, %.1f s "
                      "in all" % (who, frac, ", ".join(used), times, b / 1e9, t),
            "host_cpu": host_cpu()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-oracle sample size in seconds (0 skips the leg)")
    ap.add_argument("--small-iters", type=int, default=1000,
                    help="iterations of the per-workload pass for the workloads under 100 MB "
                         "(launch-bound; the large ones take --steps)")
    ap.add_argument("--only", default=None,
                    help="time only the ops whose name contains this text (profiling aid; "
                         "the JSON then covers that subset)")
    ap.add_argument("--no-variants", action="store_true",
                    help="report the step and the per-workload pass only, without the "
                         "variant ops and the small-shape latencies")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the step, run a plain 1 GiB device copy 10 times "
                         "(reference kernel for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU; --gpus %d is not supported "
              "(planes shard across GPUs with no communication)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import bwd_max_pool3d_amd as mp
    from bwd_max_pool3d_amd import workloads

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": a.numel() * 4, "launches": 10}))
        return

    hip = Hip()
    stream = torch.cuda.current_stream()

    # practical peak: a plain 1 GiB device-to-device copy (read + write)
    ca = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    cb = torch.empty_like(ca)
    for _ in range(3):
        cb.copy_(ca)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        cb.copy_(ca)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * ca.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del ca, cb
    torch.cuda.empty_cache()

    print("[bench] building inputs", file=sys.stderr, flush=True)
    fwd_ops, bwd_ops, var_ops = build_ops(torch, mp, workloads, variants=not args.no_variants)
    ops = fwd_ops + bwd_ops
    for op in fwd_ops:          # the forwards' idx feeds the backwards
        op.fn()
    if args.only:
        ops = [op for op in ops if args.only in op.name]
        var_ops = [op for op in var_ops if args.only in op.name]
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    torch.cuda.synchronize()

    def timed(op, sink):
        a, b = hip.pair()
        mp.mp3d_time_next_call(a, b)
        op.fn()
        sink.append((op, a, b))

    def collect(sink):
        torch.cuda.synchronize()
        for op, a, b in sink:
            op.us.append(hip.elapsed_us(a, b))
        hip.reset()

    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()

    # Pass 1, the figure of merit: K whole steps back to back.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)

    # Pass 2: the same steps, each call's kernel time from the timing hook.
    sink = []
    t2 = time.perf_counter()
    for _ in range(args.steps):
        for op in ops:
            timed(op, sink)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    collect(sink)
    step_rows = [op_row(op, "mean") for op in ops if op.us]
    print("[bench] timed %d steps, kernel times per call" % args.steps, file=sys.stderr, flush=True)

    # Pass 3: each workload alone, flushed before every iteration.
    for op in ops:
        op.us = []
    by_wl = {}
    for op in ops:
        by_wl.setdefault(op.wl.name, []).append(op)
    for name, wops in by_wl.items():
        wops.sort(key=lambda o: 0 if o.kind == "fwd" else 1)
        # the small workloads are launch-bound: many more iterations
        iters = args.steps if sum(o.nbytes for o in wops) > 100e6 else max(args.steps, args.small_iters)
        for _ in range(iters):
            sink = []
            flush_buf.sum()
            for op in wops:
                timed(op, sink)
            collect(sink)
    print("[bench] per-workload pass", file=sys.stderr, flush=True)
    per_config = []
    for name, wops in by_wl.items():
        rows = {op.kind: op_row(op) for op in wops}
        comb = [sum(v) for v in zip(*[op.us for op in wops])]
        cst = stats(comb)
        nbytes = sum(op.nbytes for op in wops)
        elems = sum(op.elems for op in wops)
        large = nbytes > 100e6
        gbs = nbytes / (cst["median"] * 1e-6) / 1e9
        per_config.append({
            "workload": name, "ops": [op.kind for op in wops], "bytes": nbytes,
            "us_median": round(cst["median"], 3), "us_min": round(cst["min"], 3),
            "us_p90": round(cst["p90"], 3), "us_mean": round(cst["mean"], 3),
            "GB_s": round(gbs, 1), "GB_s_at_min": round(nbytes / (cst["min"] * 1e-6) / 1e9, 1),
            "elems_per_s": round(elems / (cst["median"] * 1e-6), 1),
            "frac_of_peak": round(gbs / PEAK_GBS, 4),
            "target_frac": TARGET_FRAC if large else None,
            "meets_target": (gbs / PEAK_GBS >= TARGET_FRAC) if large else None,
            "per_op": rows})

    roofline = None
    if ops:
        dom_op = max(ops, key=lambda o: stats(o.us)["median"])
        dom = op_row(dom_op, "mean")
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
            if tr.get("source_hash") == kernel_source_hash() and dom["op"] in tr.get("ops", {}):
                traffic = tr["ops"][dom["op"]]["hbm_bytes"]
        roofline = {"bound": "hbm", "achieved": dom["GB_s"], "peak": PEAK_GBS, "unit": "GB/s",
                    "frac": round(dom["GB_s"] / PEAK_GBS, 4), "traffic": traffic,
                    "kernel": dom["op"], "algorithmic_bytes": dom["bytes"], "avg_us": dom["us"],
                    "timing": "mean kernel time over the per-workload pass (timing hook), "
                              "launches after an untimed 1 GiB read"}

    # Small shapes of the PR #308 page's latency table: adaptive backward.
    latency = []
    if not args.no_variants and not args.only:
        for dt, shape in workloads.PR308_SHAPES:
            tdt = workloads.DTYPES[dt]
            x = workloads.draw(shape, "normal", tdt, 7).cuda()
            for out in (tuple(max(v // 2, 1) for v in shape[2:]), (3, 3, 3)):
                y, idx = mp.amp3d_forward(x, out)
                gy = workloads.draw(y.shape, "normal", tdt, 8).cuda()
                gx = torch.empty_like(x)
                op = Op("pr308", "%s_%s_to_%s" % (dt, "x".join(map(str, shape)),
                                                  "x".join(map(str, out))),
                        lambda gy=gy, idx=idx, shape=shape, gx=gx: mp.mp3d_backward(
                            gy, idx, shape, out=gx), 0, x.numel(), "adaptive backward")
                for _ in range(20):
                    op.fn()
                sink = []
                for _ in range(200):
                    timed(op, sink)
                collect(sink)
                # per call with launches back to back, as a latency harness
                # sees it (event pair around 200 calls)
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                for _ in range(200):
                    op.fn()
                ev1.record(stream)
                torch.cuda.synchronize()
                kt = stats(op.us)
                latency.append({"dtype": dt, "shape": list(shape), "out": list(out),
                                "kernel_us_median": round(kt["median"], 3),
                                "kernel_us_min": round(kt["min"], 3),
                                "per_call_us_back_to_back": round(ev0.elapsed_time(ev1) * 1e3 / 200, 3)})
        print("[bench] small-shape latencies", file=sys.stderr, flush=True)

    # Variants: flushed, one call at a time, kernel time from the hook.
    for op in var_ops:
        op.fn()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for op in var_ops:
            sink = []
            flush_buf.sum()
            timed(op, sink)
            collect(sink)
    del flush_buf
    print("[bench] variants", file=sys.stderr, flush=True)

    ms_step = (t1 - t0) * 1e3 / args.steps
    step_bytes = sum(op.nbytes for op in ops)
    value = step_bytes / (ms_step * 1e-3) / 1e9 if ops else 0.0
    vrows = lambda kinds: [op_row(op) for op in var_ops if op.kind in kinds]
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "ms_per_step_timed_calls": round((t3 - t2) * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "five 3-D max-pool workloads per step: forward of all five, "
                               "backward of the four with one (adaptive f32 2x3x8^3->4^3; "
                               "adaptive bf16 4x16x10^3->8^3; fixed bf16 16x64x16x112x112 "
                               "k2s2 fwd only; fixed f16 8x128x32x56x56 k3s2; adaptive f32 "
                               "32x256x16x32x32->5x7x7)",
                   "step_bytes": step_bytes, "storage_dtypes": "f32, bf16, f16; idx int32",
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "copy_GB_s": round(copy_gbs, 1),
        "roofline": roofline,
        "per_config": per_config,
        "per_op_step": step_rows,
        "latency_pr308_shapes": {
            "context": "PR #308 page, Performance table: about %.1f us for float16 (2,8,4,4,4) "
                       "adaptive backward on a Moore Threads GPU (other hardware; context, "
                       "not a target; the page prints no output_size)" % PR308_CONTEXT_US,
            "rows": latency},
        "values_only_forward": vrows(("fwd_values",)),
        "ordered_backward": vrows(("bwd_ordered",)),
        "index_free_backward": [op_row(op) for op in var_ops if op.kind.startswith("bwd_recompute")],
        "int64_index_forward": vrows(("fwd_i64",)),
        "padded": vrows(("fwd_pad", "bwd_pad")),
        "float64": vrows(("fwd_f64", "bwd_f64", "bwd_f64_ordered")),
        "gather_backward": vrows(("bwd_gather",)),
    }
    if args.cpu_seconds > 0:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        nt = host_threads()
        result["cpu_baseline_threads"] = (cpu_baseline(args.cpu_seconds / 2, nt)
                                          if nt > 1 else None)
    else:
        result["cpu_baseline"] = None
        result["cpu_baseline_threads"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
