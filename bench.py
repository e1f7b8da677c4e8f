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
second, over the whole step, and as a fraction of the 8 TB/s peak.

Timing: K steps launched back to back between two synchronisations give
the step time and the metric; a second pass of K steps with a HIP event
pair around every op on its launch stream gives the per-op durations and
the roofline of the dominant op (those events cost a few microseconds per
op, so that pass is not the metric).  The values-only forward of each
workload (no index written), the forward with int64 indices, the fixed
workloads with padding k//2 (forward and backward), the ordered backward
(overlap=2), the index-free backward (argmax recomputed from x and y; one
pass, and two through a workspace) and
float64 forward and backward of the two large overlapping workloads are
timed the same way, apart from the step, each launch after an untimed read
of a 512 MiB buffer that leaves the caches clean, and reported on their own
(median per op: launched one op at a time, an event pair can catch a host
stall).

Beside the GPU figures, the CPU oracle is timed on the same workloads
(``cpu_baseline``: one thread; ``cpu_baseline_threads``: the host's CPUs, up
to 16, each thread running the unchanged oracle on a range of planes).

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this path runs on one
GPU (planes shard across GPUs with no communication, so more GPUs are not
measured here).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
METRIC = "effective HBM GB/s (bytes read+written / time) fwd+bwd; % of MI355X HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


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


class Op:
    """One C-ABI call of the step, with its inputs and preallocated outputs."""

    def __init__(self, wl, kind, fn, nbytes, elems, note):
        self.wl, self.kind, self.fn, self.nbytes, self.elems, self.note = (
            wl, kind, fn, nbytes, elems, note)
        self.ms = []

    @property
    def name(self):
        return "%s.%s" % (self.wl.name, self.kind)


def build_ops(torch, mp, workloads, variants=True):
    """The step's ops (forwards, then backwards) and, apart from the step,
    the variants: the values-only forward of each workload (idx NULL:
    |x|+|y| bytes) and the ordered (bit-reproducible) backward."""
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
        fwd_ops.append(Op(wl, "fwd", f, fbytes, nin, "forward"))
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
            bwd_ops.append(Op(wl, "bwd", b, bbytes, nin, "backward"))
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
        if not variants:
            continue
        # int64 indices (torch's index type): general forward kernel
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
            # padding k // 2 on every axis (the usual "same"-style pooling)
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
    # float64 (x and gy widened exactly) on the two large overlapping workloads
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
    # the variants run in the step's order: forwards, then backwards
    return fwd_ops + bwd_ops, (vo_ops + exf_ops + ord_ops + exb_ops) if variants else []


_CPU_INPUTS: dict = {}     # seeded workload tensors, drawn once for both oracle runs


def host_threads() -> int:
    """Host threads for the multi-threaded oracle run: the CPUs this process
    may use, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


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
            if wl.backward:
                gy = draw(wl, "gy", (P, 1) + o3)[:np_].contiguous()
                gys = storage(gy)
                jobs = [(a, b, fw[j][1]) for j, (a, b) in enumerate(parts)]
                t0 = time.perf_counter()
                each(lambda a, b, idx: orc.backward(gys[a:b], idx, c, (b - a, 1, D, H, W),
                                                    side=False), jobs)
                elapsed += time.perf_counter() - t0
                total_bytes += nout * (es + 4) + nin * es
        return total_bytes, elapsed, planes_used

    probe = 1.0 / 512 * threads
    b, t, _ = run(probe)
    frac = min(1.0, probe * target_s / max(t, 1e-3))
    b, t, used = run(frac)
    if pool is not None:
        pool.shutdown()
    who = "one thread" if threads == 1 else "%d threads over contiguous plane ranges" % threads
    return {"value": round(b / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "plain C oracle, %s, forward+backward on %.4f of each "
                      "workload's planes (%s): %.3g GB of algorithmic bytes in %.1f s"
                      % (who, frac, ", ".join(used), b / 1e9, t)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-oracle sample size in seconds (0 skips the leg)")
    ap.add_argument("--only", default=None,
                    help="time only the ops whose name contains this text (profiling aid; "
                         "the JSON then covers that subset)")
    ap.add_argument("--no-variants", action="store_true",
                    help="report the step alone, without the variant ops (values-only "
                         "forward, int64 indices, padding, ordered backward); for profiles "
                         "whose per-kernel averages must cover the step's launches only")
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
    ops, vo_ops = build_ops(torch, mp, workloads, variants=not args.no_variants)
    if args.only:
        # forward ops must still run once so their idx feeds the backward
        for op in ops:
            op.fn()
        ops = [op for op in ops if args.only in op.name]
        vo_ops = [op for op in vo_ops if args.only in op.name]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()

    # Pass 1, the figure of merit: K whole steps back to back, nothing
    # between the launches (an event pair around each op costs a few
    # microseconds of GPU time per op).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for step in range(args.steps):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)

    # Pass 2: the same K steps with HIP events around every op on its launch
    # stream, for the per-op durations and the roofline of the dominant op.
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for step in range(args.steps):
        for op, (e0, e1) in zip(ops, evs[step]):
            e0.record(stream)
            op.fn()
            e1.record(stream)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for step in range(args.steps):
        for op, (e0, e1) in zip(ops, evs[step]):
            op.ms.append(e0.elapsed_time(e1))
    print("[bench] timed %d steps with per-op events" % args.steps, file=sys.stderr, flush=True)

    # Variants (not part of the step): same events, K times each.  Each
    # launch is preceded by an untimed read of a 512 MiB buffer: it writes
    # back whatever the previous variant left dirty in L2 and the 256 MB
    # memory-side cache and leaves clean lines, so a variant's time does not
    # depend on which variant ran before it.
    flush_buf = torch.ones(1 << 27, dtype=torch.float32, device="cuda") if vo_ops else None
    for op in vo_ops:
        op.fn()
    vo_evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in vo_ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for step in range(args.steps):
        for op, (e0, e1) in zip(vo_ops, vo_evs[step]):
            flush_buf.sum()
            e0.record(stream)
            op.fn()
            e1.record(stream)
    torch.cuda.synchronize()
    del flush_buf
    for step in range(args.steps):
        for op, (e0, e1) in zip(vo_ops, vo_evs[step]):
            op.ms.append(e0.elapsed_time(e1))

    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_ev = (t3 - t2) * 1e3 / args.steps
    step_bytes = sum(op.nbytes for op in ops)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    def op_row(op, median=False):
        # step ops: the mean (it matches the profiler's average per launch);
        # variants, timed one op at a time: the median, since a host stall
        # while the queue is empty can land inside one event pair
        avg = sum(op.ms) / len(op.ms)
        srt = sorted(op.ms)
        med = srt[len(srt) // 2]
        p90 = srt[min(len(srt) - 1, (9 * len(srt)) // 10)]
        t = med if median else avg
        return {"op": op.name, "ms": round(t, 5), "ms_mean": round(avg, 5),
                "ms_min": round(srt[0], 5), "ms_median": round(med, 5),
                "ms_p90": round(p90, 5), "bytes": op.nbytes,
                "GB_s": round(op.nbytes / (t * 1e-3) / 1e9, 1),
                "elems_per_s": round(op.elems / (t * 1e-3), 1),
                "frac_of_peak": round(op.nbytes / (t * 1e-3) / 1e9 / PEAK_GBS, 4)}

    per_op = [op_row(op) for op in ops]
    dom = max(per_op, key=lambda r: r["ms"])
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash() and dom["op"] in tr.get("ops", {}):
            traffic = tr["ops"][dom["op"]]["hbm_bytes"]
    roofline = {"bound": "hbm", "achieved": dom["GB_s"], "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["GB_s"] / PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom["op"], "algorithmic_bytes": dom["bytes"], "avg_ms": dom["ms"]}
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "ms_per_step_with_op_events": round(ms_step_ev, 5),
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
        "per_op": per_op,
        "values_only_forward": [op_row(op, True) for op in vo_ops if op.kind == "fwd_values"],
        "ordered_backward": [op_row(op, True) for op in vo_ops if op.kind == "bwd_ordered"],
        "index_free_backward": [op_row(op, True) for op in vo_ops
                                if op.kind.startswith("bwd_recompute")],
        "int64_index_forward": [op_row(op, True) for op in vo_ops if op.kind == "fwd_i64"],
        "padded": [op_row(op, True) for op in vo_ops if op.kind in ("fwd_pad", "bwd_pad")],
        "float64": [op_row(op, True) for op in vo_ops
                    if op.kind in ("fwd_f64", "bwd_f64", "bwd_f64_ordered")],
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
