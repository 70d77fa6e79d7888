#!/usr/bin/env python3
"""Benchmark of the MI355X convolution weight gradient (one GPU).

A step is one full weight-gradient call (stage 1 + the slab reduce when the
plan has several slices) on inputs already resident in HBM.  The default
workload is the 3x3 fp32 wgrad, N=32, C=K=64, H=W=56, pad 1.  Prints one
JSON line:

  value           TFLOP/s of the whole call over K back-to-back steps (after
                  W warm-up steps and --prewarm-s seconds of untimed steps
                  that bring the GPU to its clocks under load)
  roofline        the stage-1 kernel alone, its duration taken from HIP events
                  on its own dispatch in each of K further back-to-back steps
                  right after the timed region (kept out of that region: a
                  launch that carries events costs the call GPU time),
                  against the MI355X peak of its bound (f32 MFMA or HBM);
                  traffic = HBM bytes per launch from the FETCH_SIZE /
                  WRITE_SIZE counter table in profiles/hbm_traffic.md when
                  it was taken on the current kernel source, else null
  whole_call_roofline_frac  the same roofline fraction for the whole call
                  (stage 1 + the slab reduce, the time behind value)
  cold_cache      per-call event times with a cache flush before each call (a
                  read of a clean 1 GiB buffer)
  cpu_baseline    the CPU oracle (test infrastructure) timed on the host cores,
                  with the host CPU model; for 1x1 workloads also numpy's
                  float64 BLAS closed form dW = dY^T X on the same images

  python bench.py --peaks   achievable streaming-read bandwidth (buffers of the
                  workloads' input sizes, hot and cold) and MFMA rates, beside
                  the published peaks; one JSON line

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--n N] [--no-cpu] [--bias]

With --bias every step is conv_wgrad_bias (the weight gradient and the fused
bias gradient db = sum dY); value still counts the weight-gradient FLOPs.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {  # MI355X published peaks
    "hbm_gbs": 8000.0,
    "mfma_tflops": {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6},
}
DEFAULT_CONFIG = "c2_3x3_f32"

# Stage-1 kernel source of each plan variant; with the shared headers and the
# planner it identifies the code a counter measurement was taken on.
CSRC = os.path.join(ROOT, "implicit_gemm_amd", "csrc")
VARIANT_SOURCE = {0: "dense_lds.hip", 1: "dense_rows.hip", 2: "dense_1x1.hip", 3: "dense16_rows.hip",
                  10: "direct_elem.hip",
                  11: "grouped16.hip", 12: "depthwise_mfma.hip", 13: "grouped16.hip"}
SHARED_SOURCES = ("device_common.h", "kernels.h", "plan.h", "plan.cpp")
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
CPU_SAMPLE_FLOPS = 1.0e12   # at most ~20 s of oracle work on 16 host cores per run
CPU_SAMPLE_SECONDS = 10.0   # runs repeat until about this much oracle time


def source_digest(variant):
    """sha256 (16 hex digits) of the stage-1 kernel source, shared headers and planner."""
    import hashlib
    h = hashlib.sha256()
    for name in (VARIANT_SOURCE[int(variant)],) + SHARED_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, digest):
    """HBM bytes per stage-1 launch from the counter table, if taken on this source."""
    try:
        with open(TRAFFIC_TABLE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 9 and cells[0] == workload and cells[2] == digest:
            try:
                return int(cells[8].replace(",", ""))
            except ValueError:
                return None
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """HIP events through the runtime torch already loaded (same SONAME)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b):
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def measure_peaks(hip):
    """Achievable peaks beside the published ones: a 16-byte streaming read of
    buffers the size of the workloads' inputs (hot: back to back; cold: after
    a read of 1 GiB of other data), and loops of independent MFMA chains.
    Each figure is the median of 10 dispatch-stamped launches at the best of
    several grid sizes."""
    import torch
    from implicit_gemm_amd import probes
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()

    def timed(launch, reps=10, before=None):
        for _ in range(3):
            launch(None, None)
        ms = []
        for _ in range(reps):
            if before:
                before()
            launch(e0, e1)
            ms.append(hip.elapsed_ms(e0, e1))
        return statistics.median(ms)

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    probe = torch.empty((), dtype=torch.float32, device="cuda")
    sink = torch.empty(65536 * 256, dtype=torch.float32, device="cuda")
    reads = []
    for nbytes in (51417088, 308356608, 1 << 30, 10737418240):
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        for cold in ((False, True) if nbytes <= (1 << 30) else (False,)):
            best = None
            for blocks in (512, 1024, 2048, 4096):
                ms = timed(lambda a, b: probes.peak_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream, a, b),
                           before=(lambda: torch.amax(flush, dim=0, out=probe)) if cold else None)
                if best is None or ms < best[1]:
                    best = (blocks, ms)
            reads.append({"bytes": nbytes, "cold": cold, "blocks": best[0], "us": round(best[1] * 1e3, 2),
                          "gbs": round(nbytes / (best[1] * 1e-3) / 1e9, 1),
                          "frac_of_published": round(nbytes / (best[1] * 1e-3) / 1e9 / PEAK["hbm_gbs"], 4)})
        del buf
    mfma = []
    for name, code, iters, per_round in (("f32", 0, 5000, 16384), ("bf16", 1, 10000, 131072),
                                         ("f16", 2, 10000, 131072)):
        best = None
        for blocks in (1024, 2048):
            ms = timed(lambda a, b: probes.peak_mfma(code, iters, blocks, sink.data_ptr(), stream, a, b), reps=5)
            tf = blocks * 4 * iters * per_round / (ms * 1e-3) / 1e12
            if best is None or tf > best[1]:
                best = (blocks, tf)
        mfma.append({"dtype": name, "blocks": best[0], "tflops": round(best[1], 1),
                     "frac_of_published": round(best[1] / PEAK["mfma_tflops"][name], 4)})
    torch.cuda.synchronize()
    hip.destroy(e0)
    hip.destroy(e1)
    return {"read": reads, "mfma": mfma, "published": PEAK}


def roofline_for(shape, dtype, seconds, traffic=None):
    import wgrad_data as wd
    flops = shape.flops()
    nbytes = shape.algorithmic_bytes(wd.IN_BYTES[dtype])
    t_mfma = flops / (PEAK["mfma_tflops"][dtype] * 1e12)
    t_hbm = nbytes / (PEAK["hbm_gbs"] * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    if shape.groups > 1 and shape.Cg <= 8:
        bound = "hbm"  # direct small-group path: its metric is achieved HBM bandwidth
    if bound == "mfma":
        achieved = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK["mfma_tflops"][dtype],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK["mfma_tflops"][dtype], 4),
                "traffic": traffic}
    achieved = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_gbs"], "unit": "GB/s",
            "frac": round(achieved / PEAK["hbm_gbs"], 4), "traffic": traffic}


def cpu_baseline(wl, x, dy, reps):
    """The fp64 oracle on the host cores, on the first images of the workload
    (all of them unless that exceeds CPU_SAMPLE_FLOPS), in TFLOP/s."""
    import oracle
    s = wl.shape
    threads = oracle.default_threads()
    per_image = s.flops() / s.N
    n_s = int(max(1, min(s.N, CPU_SAMPLE_FLOPS // per_image)))
    xs, dys = x[:n_s], dy[:n_s]
    # At least `reps` runs, and more until about CPU_SAMPLE_SECONDS of oracle work.
    times = []
    while len(times) < reps or (sum(times) < CPU_SAMPLE_SECONDS and len(times) < 200):
        t0 = time.perf_counter()
        oracle.wgrad_ref(xs, dys, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, nthreads=threads)
        times.append(time.perf_counter() - t0)
    reps = len(times)
    t = statistics.median(times)
    what = "whole workload" if n_s == s.N else "first %d of %d images" % (n_s, s.N)
    out = {"value": round(per_image * n_s / t / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": "%s (%s), median of %d runs, fp64 C oracle, %.2f s per run"
                     % (what, wl.name, reps, t),
           "cpu_model": cpu_model()}
    if s.R == 1 and s.S == 1 and s.stride == 1 and s.pad == 0 and s.groups == 1:
        # A 1x1 weight gradient is one product, dW = dY^T X over all pixels:
        # numpy's float64 BLAS on the same images, one image at a time.
        import numpy as np
        t0 = time.perf_counter()
        acc = np.zeros((s.K, s.C))
        for i in range(n_s):
            acc += dys[i].reshape(-1, s.K).astype(np.float64).T @ xs[i].reshape(-1, s.C).astype(np.float64)
        tb = time.perf_counter() - t0
        out["blas_closed_form"] = {"value": round(per_image * n_s / tb / 1e12, 5), "unit": "TFLOP/s",
                                   "sample": "%s, numpy float64 dY^T X per image (widening included), "
                                             "one run, %.2f s" % (what, tb)}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--split-k", type=int, default=-1)
    ap.add_argument("--n", type=int, default=0, help="batch of an N-swept workload (default 64)")
    ap.add_argument("--cold", type=int, default=20, help="cold-cache calls (0 = skip)")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed steps after the warm-up steps (clock ramp)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--bias", action="store_true",
                    help="time conv_wgrad_bias (dW and the fused bias gradient db = sum dY)")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--peaks", action="store_true",
                    help="measure the achievable streaming-read bandwidth and MFMA rates and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 3 device-to-device copies of 1 GiB (scale for HBM byte counters)")
    ap.add_argument("--digest", action="store_true",
                    help="print the stage-1 source digest of --config and exit (no GPU needed)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the weight-gradient path runs on a single MI355X "
              "(--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import implicit_gemm_amd as iga
    import wgrad_data as wd

    if args.digest:
        s = wd.workload(args.config).shape
        d = iga.make_desc(s.N, s.C, s.H, s.W, s.K, s.R, s.S, s.pad, s.stride, s.dilation, s.groups,
                          {"f32": 0, "bf16": 1, "f16": 2}[wd.workload(args.config).dtype], args.split_k)
        v = int(iga.get_plan(d).variant)
        print(json.dumps({"workload": args.config, "variant": v, "source": VARIANT_SOURCE[v],
                          "digest": source_digest(v)}))
        return 0

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.peaks:
        print(json.dumps({"peaks": measure_peaks(Hip())}))
        return 0
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "copies": 3}))
        return 0
    wl = wd.workload(args.config)
    s = wl.shape
    if wl.n_sweep:
        # N-swept workload: N = 64 unless --n picks another point of the sweep.
        n = args.n if args.n else 64
        if n not in wl.n_sweep:
            print("--n must be one of %s for %s" % (wl.n_sweep, wl.name), file=sys.stderr)
            return 2
        s = s.with_n(n)
        wl = wd.Workload(wl.name, s, wl.dtype, wl.x_dist, wl.dy_dist, wl.seed, wl.note)
    elif args.n:
        print("--n applies only to an N-swept workload", file=sys.stderr)
        return 2
    log("workload", wl.name, s, wl.dtype)
    x_h, dy_h = wd.make_inputs(wl)
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    x = torch.from_numpy(x_h).to(tdt).to(dev)
    dy = torch.from_numpy(dy_h).to(tdt).to(dev)
    d = iga.desc_for(x, dy, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, args.split_k)
    plan = iga.get_plan(d)
    dw = torch.empty((s.K, s.R, s.S, s.Cg), dtype=torch.float32, device=dev)
    ws_bytes = int(plan.ws_bytes)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    hip = Hip()
    torch.cuda.synchronize()

    db = torch.empty((s.K,), dtype=torch.float32, device=dev)

    def step(ev0=0, ev1=0):
        if args.bias:
            iga.conv_wgrad_bias_timed(d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), db.data_ptr(),
                                      ws.data_ptr() if ws_bytes else 0, ws_bytes, sp, ev0, ev1)
        else:
            iga.conv_wgrad_timed(d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(),
                                 ws.data_ptr() if ws_bytes else 0, ws_bytes, sp, ev0, ev1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Clock warm-up: the GPU leaves its idle clocks only after some time under
    # load, so untimed steps run until --prewarm-s seconds have passed.
    t_pre = time.perf_counter()
    prewarm_steps = 0
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        prewarm_steps += 10

    # Timed region: K back-to-back steps, no per-call events (a launch that
    # carries timing events costs the call several microseconds of GPU time).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Stage-1 kernel durations: the next K back-to-back steps, with HIP events
    # that take the stage-1 dispatch's own start and end timestamps.
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(*evs[i])
    torch.cuda.synchronize()
    k_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)

    # Cold-cache calls (outside the timed region): before each, a read of a
    # 1 GiB buffer (written once beforehand) evicts the inputs from the L2s and
    # the 256 MB MALL and leaves clean lines, so the call neither hits the
    # caches nor competes with the write-back of a flush's dirty lines.
    cold = None
    if args.cold > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        probe = torch.empty((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        e0, e1, e2 = hip.event(), hip.event(), hip.event()
        whole, stage1 = [], []
        for _ in range(args.cold):
            torch.amax(flush, dim=0, out=probe)   # queued just before the call: no idle gap
            hip.record(e0, sp)
            step(e1, e2)
            e3 = hip.event()
            hip.record(e3, sp)
            whole.append(hip.elapsed_ms(e0, e3))
            stage1.append(hip.elapsed_ms(e1, e2))
            hip.destroy(e3)
        whole.sort()
        cold = {"call_ms_median": round(statistics.median(whole), 5), "call_ms_min": round(whole[0], 5),
                "call_ms_p90": round(whole[int(0.9 * (len(whole) - 1))], 5),
                "stage1_ms_median": round(statistics.median(stage1), 5),
                "tflops_median": round(s.flops() / (statistics.median(whole) * 1e-3) / 1e12, 3)}
        del flush, probe

    torch.cuda.synchronize()
    dw_h = dw.cpu().numpy()
    zeros = int((dw_h == 0).sum())
    finite = bool(np.isfinite(dw_h).all())

    ms_per_step = wall / args.steps * 1e3
    value = s.flops() / (wall / args.steps) / 1e12
    stage1_avg_s = statistics.mean(k_ms) * 1e-3
    roof = roofline_for(s, wl.dtype, stage1_avg_s,
                        None if args.bias else measured_traffic(wl.name, source_digest(plan.variant)))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, x_h, dy_h, args.cpu_reps)

    out = {
        "metric": "wgrad TFLOP/s and % of MFMA-or-HBM roofline per conv shape, 1xMI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_steps": prewarm_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded PCG64 per image)",
        "config": {"workload": wl.name, "note": wl.note, "N": s.N, "C": s.C, "H": s.H, "W": s.W,
                   "K": s.K, "R": s.R, "S": s.S, "pad": s.pad, "stride": s.stride,
                   "dilation": s.dilation, "groups": s.groups, "split_k": args.split_k,
                   "ks_count": int(plan.ks_count), "path": int(plan.path), "variant": int(plan.variant),
                   "bias_gradient": bool(args.bias),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "whole_call_roofline_frac": roofline_for(s, wl.dtype, ms_per_step * 1e-3)["frac"],
        "stage1_ms_mean": round(stage1_avg_s * 1e3, 5),
        "cold_cache": cold,
        "cpu_baseline": cpu,
        "check": {"zeros": zeros, "finite": finite},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
