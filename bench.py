#!/usr/bin/env python3
"""Benchmark of the MI355X convolution weight gradient (one GPU).

A step is one full weight-gradient call (stage 1 + the slab fold when the
plan has several slices) on inputs already resident in HBM.  With no
--config, one run measures every workload of the study and prints ONE JSON
line whose headline is the largest single-GPU workload, the 1x1 fp32 wgrad
C=96 K=64 512x512 at N=192 (32.2 GB of X and dY, so every step reads its
inputs from HBM; no cache holds them):

  value, ms_per_step  whole-call TFLOP/s over K back-to-back steps between
                  synchronisations (after W warm-up steps and --prewarm-s
                  seconds of untimed steps that bring the GPU to its clocks)
  roofline        the dominant (stage-1) kernel: algorithmic bytes or FLOPs
                  per launch / its mean duration from HIP events stamped by
                  its own dispatch in K further steps, against the MI355X
                  peak of its bound; traffic = HBM bytes per launch from the
                  FETCH_SIZE / WRITE_SIZE counter table (profiles/
                  hbm_traffic.md) when it was taken on the current source
  whole_call_roofline_frac  the same fraction for the whole call (value)
  cpu_baseline    the CPU oracle (test infrastructure) on the host cores, on a
                  bounded sample of the workload, with the host CPU model
  configs         one record per workload (the five of the study, the 1x1
                  case at N=64 and N=192): the cold whole call -- each call
                  after a read of a clean 1 GiB buffer that evicts the inputs
                  from the L2s and the 256 MB MALL, HIP events on the stream
                  around stage 1 + fold, median / min / p90 of --cold calls --
                  with its roofline fraction; the stage-1 kernel alone, cold
                  and hot (dispatch-stamped events, in calls of their own);
                  the hot back-to-back call; counter traffic; cpu_baseline

  python bench.py --config NAME [--n N]   only that workload (its record is
                  the headline; value is then the hot back-to-back figure)
  python bench.py --peaks   achievable streaming-read bandwidth and MFMA
                  rates beside the published peaks; one JSON line

With --bias every call is conv_wgrad_bias (the weight gradient and the fused
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

PEAK = {  # MI355X published peaks (and the unit counts the probes normalise by)
    "hbm_gbs": 8000.0,
    "mfma_tflops": {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6},
    "cus": 256,
    "clock_ghz": 2.4,
}
DEFAULT_CONFIG = "c2_3x3_f32"

# Stage-1 kernel source of each plan variant; with the shared headers and the
# planner it identifies the code a counter measurement was taken on.
CSRC = os.path.join(ROOT, "implicit_gemm_amd", "csrc")
VARIANT_SOURCE = {0: "dense_lds.hip", 1: "dense_rows.hip", 2: "dense_1x1.hip", 3: "dense16_rows.hip",
                  4: "dense16_rows.hip", 5: "dense16_taps.hip", 6: "dense16_taps.hip",
                  20: "conv_igemm.hip", 21: "conv_igemm.hip",
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


def measured_traffic(workload, digest, n):
    """HBM bytes per stage-1 launch from the counter table, if taken on this source.

    Table rows: | workload | N | kernel | source digest | dispatches | FETCH_SIZE KiB |
    WRITE_SIZE KiB | fetch scale | write scale | traffic bytes | algorithmic bytes |"""
    try:
        with open(TRAFFIC_TABLE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 11 and cells[0] == workload and cells[1] == str(n) and cells[3] == digest:
            try:
                return int(cells[9].replace(",", ""))
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
    best = None
    for blocks in (1024, 2048):   # the 16x16x32 bf16 form of the 16-bit kernels
        ms = timed(lambda a, b: probes.peak_mfma16(10000, blocks, sink.data_ptr(), stream, a, b), reps=5)
        tf = blocks * 4 * 10000 * 131072 / (ms * 1e-3) / 1e12
        if best is None or tf > best[1]:
            best = (blocks, tf)
    mfma.append({"dtype": "bf16 (16x16x32)", "blocks": best[0], "tflops": round(best[1], 1),
                 "frac_of_published": round(best[1] / PEAK["mfma_tflops"]["bf16"], 4)})
    lds = []
    for mode, name, width in ((0, "ds_read_b64_tr_b16", 8), (1, "ds_read_b64", 8), (2, "ds_read_b128", 16)):
        for blocks in (256, 512, 1024):   # 1, 2 and 4 workgroups per CU
            ms = timed(lambda a, b: probes.peak_lds(mode, 4000, blocks, sink.data_ptr(), stream, a, b), reps=5)
            nbytes = blocks * 256 * 4000 * 8 * width
            lds.append({"read": name, "workgroups_per_cu": blocks // PEAK["cus"],
                        "bytes_per_clk_per_cu": round(nbytes / (ms * 1e-3) / (PEAK["clock_ghz"] * 1e9) / PEAK["cus"], 1)})
    torch.cuda.synchronize()
    hip.destroy(e0)
    hip.destroy(e1)
    return {"read": reads, "mfma": mfma, "lds": lds, "published": PEAK}


def roofline_for(shape, dtype, seconds, traffic=None, math="exact"):
    """Roofline of one call: algorithmic FLOPs against the MFMA peak of the dtype the
    products run in, algorithmic bytes against HBM, whichever takes longer.  BF16x3
    runs three bf16 products per fp32 product, so its MFMA work is 3x the FLOPs at
    the bf16 peak."""
    import wgrad_data as wd
    flops = shape.flops()
    nbytes = shape.algorithmic_bytes(wd.IN_BYTES[dtype])
    mfma_dtype, mult = ("bf16", 3) if math == "bf16x3" else (dtype, 1)
    peak_mfma = PEAK["mfma_tflops"][mfma_dtype]
    t_mfma = mult * flops / (peak_mfma * 1e12)
    t_hbm = nbytes / (PEAK["hbm_gbs"] * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    if shape.groups > 1 and shape.Cg <= 8:
        bound = "hbm"  # direct small-group path: its metric is achieved HBM bandwidth
    if bound == "mfma":
        achieved = mult * flops / seconds / 1e12
        out = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_mfma,
               "unit": "TFLOP/s", "frac": round(achieved / peak_mfma, 4), "traffic": traffic}
        if mult > 1:
            out["note"] = "BF16x3: MFMA work is three bf16 products per fp32 product"
        return out
    achieved = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_gbs"], "unit": "GB/s",
            "frac": round(achieved / PEAK["hbm_gbs"], 4), "traffic": traffic}


# (workload, batch of an N-swept workload, extended-descriptor options)
ALL_RECORDS = [("c1_1x1_tiny_f32", None, {}), ("c2_3x3_f32", None, {}), ("c3_dw7x7_bf16", None, {}),
               ("c4a_grp3x3_cpg4_f16", None, {}), ("c4b_grp3x3_cpg8_f16", None, {}),
               ("c5_1x1_big_f32", 64, {}),
               ("c2_3x3_f32", None, {"math": "bf16x3"}),
               ("g_patch16_f32", None, {}), ("g_patch16_f32", None, {"fold_width": 0}),
               ("l_3x3_c512_f32", None, {"direction": "fwd"}), ("l_3x3_c512_f32", None, {"direction": "fwd", "split_k": 1}),
               ("l_3x3_c512_f32", None, {"direction": "dgrad"}), ("l_3x3_c512_bf16", None, {"direction": "fwd"}),
               ("l_3x3_c512_bf16", None, {"direction": "dgrad"})]
HEADLINE = ("c5_1x1_big_f32", 192, {})
FAMILY = {0: "dense_lds", 1: "dense_rows", 2: "dense_1x1", 3: "dense16_rows", 4: "dense16_rows_bf16x3",
          5: "dense16_taps", 6: "dense16_taps_bf16x3",
          10: "direct_elem", 11: "grouped16", 12: "depthwise_mfma", 13: "grouped16_rows"}


def resolve(name, n):
    """Workload and shape for a configuration name (N-swept workloads at batch n, default 64)."""
    import wgrad_data as wd
    wl = wd.workload(name)
    s = wl.shape
    if wl.n_sweep:
        n = n or 64
        if n not in wl.n_sweep:
            raise SystemExit("--n must be one of %s for %s" % (wl.n_sweep, wl.name))
        s = s.with_n(n)
        wl = wd.Workload(wl.name, s, wl.dtype, wl.x_dist, wl.dy_dist, wl.seed, wl.note, wl.n_sweep)
    elif n:
        raise SystemExit("--n applies only to an N-swept workload")
    return wl, s


def device_inputs(wl, s, dev):
    """x, dy on the device (the seeded per-image draws of wgrad_data), filled in
    chunks of images through pinned host staging so host memory stays bounded."""
    import os as _os
    from concurrent.futures import ThreadPoolExecutor
    import torch
    import wgrad_data as wd
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    x = torch.empty((s.N, s.H, s.W, s.C), dtype=tdt, device=dev)
    dy = torch.empty((s.N, s.Ho, s.Wo, s.K), dtype=tdt, device=dev)
    per_img = (s.H * s.W * s.C + s.Ho * s.Wo * s.K) * 4
    chunk = max(1, min(s.N, (1 << 31) // per_img))
    if chunk >= s.N:
        xh, dyh = wd.make_inputs(wl)
        x.copy_(torch.from_numpy(xh).to(tdt))
        dy.copy_(torch.from_numpy(dyh).to(tdt))
        return x, dy
    xs = torch.empty((chunk, s.H, s.W, s.C), dtype=torch.float32, pin_memory=True)
    dys = torch.empty((chunk, s.Ho, s.Wo, s.K), dtype=torch.float32, pin_memory=True)
    xa, dya = xs.numpy(), dys.numpy()
    threads = min(16, max(1, len(_os.sched_getaffinity(0))))

    def fill(i, n):
        wd.draw_images(wl.seed, wd.X_ID, n, 1, s.H, s.W, s.C, wl.x_dist, out=xa[i:i + 1], threads=1)
        wd.draw_images(wl.seed, wd.DY_ID, n, 1, s.Ho, s.Wo, s.K, wl.dy_dist, out=dya[i:i + 1], threads=1)

    with ThreadPoolExecutor(threads) as ex:
        for n0 in range(0, s.N, chunk):
            cnt = min(chunk, s.N - n0)
            list(ex.map(lambda i: fill(i, n0 + i), range(cnt)))
            if wl.dtype != "f32":
                raise SystemExit("chunked staging is for fp32 workloads")
            x[n0:n0 + cnt].copy_(xs[:cnt], non_blocking=True)
            dy[n0:n0 + cnt].copy_(dys[:cnt], non_blocking=True)
            torch.cuda.synchronize()   # the staging buffers are refilled by the next chunk
    return x, dy


def cpu_baseline(wl, s, seconds):
    """The fp64 oracle on the host cores, on the first images of the workload
    (as many as fit about seconds / 3 of oracle time per run; at least three
    runs and about `seconds` in all), in TFLOP/s."""
    import oracle
    import wgrad_data as wd
    threads = oracle.default_threads()
    per_image = s.flops() / s.N
    # Size the sample from one timed image.
    x1, dy1 = wd.make_inputs(wl, 0, 1)
    t0 = time.perf_counter()
    oracle.wgrad_ref(x1, dy1, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, nthreads=threads)
    t_img = max(time.perf_counter() - t0, 1e-6)
    n_s = int(max(1, min(s.N, (seconds / 3.0) / t_img)))
    xs, dys = wd.make_inputs(wl, 0, n_s)
    times = []
    while len(times) < 3 or (sum(times) < seconds and len(times) < 200):
        t0 = time.perf_counter()
        oracle.wgrad_ref(xs, dys, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    what = "whole workload" if n_s == s.N else "first %d of %d images" % (n_s, s.N)
    out = {"value": round(per_image * n_s / t / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": "%s of %s, median of %d runs, fp64 C oracle, %.2f s per run"
                     % (what, wl.name, len(times), t),
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


def _pct(vals, q):
    v = sorted(vals)
    return v[int(q * (len(v) - 1))]


def measure(wl, s, x, dy, args, hip, cold_reps, bias=False, opts=None):
    """Time one workload on resident inputs (extended-descriptor options opts: math,
    fold_width); returns (record, wall seconds per step of the timed region -- K
    back-to-back calls whose stage-1 dispatches stamp HIP events -- and the mean
    stage-1 duration from those events, in seconds)."""
    import numpy as np
    import torch
    import implicit_gemm_amd as iga
    import wgrad_data as wd
    opts = opts or {}
    math = opts.get("math", "exact")
    dev = x.device
    d = iga.desc2_for(x, dy, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, args.split_k, math,
                      opts.get("fold_width", -1))
    plan2 = iga.get_plan2(d)
    plan = plan2.base
    dw = torch.empty((s.K, s.R, s.S, s.Cg), dtype=torch.float32, device=dev)
    db = torch.empty((s.K,), dtype=torch.float32, device=dev)
    ws_bytes = int(plan.ws_bytes)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    wsp = ws.data_ptr() if ws_bytes else 0

    dbp = db.data_ptr() if bias else 0

    def step(ev0=0, ev1=0, whole=False):
        if whole:
            iga.conv_wgrad2_call_timed(d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), dbp, wsp, ws_bytes, sp,
                                       ev0, ev1)
        elif ev0 or ev1:
            iga.conv_wgrad2_timed(d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), dbp, wsp, ws_bytes, sp, ev0, ev1)
        else:
            iga.conv_wgrad2(d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), dbp, wsp, ws_bytes, sp)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Clock warm-up: the GPU leaves its idle clocks only after some time under load.
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            step()
        torch.cuda.synchronize()

    # Timed region: K back-to-back steps between synchronisations, each
    # stage-1 dispatch stamping its own start and end into a pair of HIP
    # events (the dominant kernel's launch duration, on the stream it runs on).
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        step(a, b)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    k_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    # The same K steps without events (host wall time per plain call).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_plain = (time.perf_counter() - t0) / args.steps

    # Cold calls: before each, a read of a clean 1 GiB buffer evicts the inputs
    # from the L2s and the MALL (queued just before the call, so the GPU never
    # idles).  Three series, interleaved call by call so that they see the same
    # conditions.  Series 1 (the cold figure): the whole call, from the start
    # of its first kernel to the end of its last (stage 1 + fold + the gap
    # between them), stamped by the dispatches themselves.  Series 2: events
    # on the stream around the plain call (they add their own marker time,
    # reported beside it as the floor of two markers with nothing between);
    # it bounds series 1 from above, so where the median of series 1 is the
    # larger the dispatch stamps are not trusted and series 2 is used.
    # Series 3: the stage-1 dispatch alone.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    probe = torch.empty((), dtype=torch.float32, device=dev)
    e0, e1, e2, e3 = hip.event(), hip.event(), hip.event(), hip.event()
    torch.cuda.synchronize()
    whole, stream_ev, floor, stage1 = [], [], [], []
    for _ in range(cold_reps):
        torch.amax(flush, dim=0, out=probe)
        step(e0, e1, whole=True)
        whole.append(hip.elapsed_ms(e0, e1))
        torch.amax(flush, dim=0, out=probe)
        hip.record(e0, sp)
        step()
        hip.record(e1, sp)
        stream_ev.append(hip.elapsed_ms(e0, e1))
        torch.amax(flush, dim=0, out=probe)
        step(e2, e3)
        stage1.append(hip.elapsed_ms(e2, e3))
    for _ in range(min(cold_reps, 20)):
        torch.amax(flush, dim=0, out=probe)
        hip.record(e0, sp)
        hip.record(e1, sp)
        floor.append(hip.elapsed_ms(e0, e1))
    for e in (e0, e1, e2, e3):
        hip.destroy(e)
    del flush, probe
    torch.cuda.synchronize()
    dw_h = dw.cpu().numpy()

    if not whole:   # --cold 0 (profiling runs): the hot figures stand in
        whole, stage1 = [wall_plain * 1e3], k_ms
    source = "first kernel start to last kernel end, dispatch-stamped events"
    whole_disp = whole
    if stream_ev and statistics.median(stream_ev) < statistics.median(whole):
        whole = stream_ev
        source = "events on the stream around the call (the dispatch-stamped median was the larger)"
    cold_med = statistics.median(whole) * 1e-3
    digest = source_digest(plan.variant)
    used_math = "bf16x3" if int(plan2.math) == 1 else "exact"
    tag = wl.name + ("+bf16x3" if used_math == "bf16x3" else "") + \
        ("+nofold" if opts.get("fold_width", -1) in (0, 1) and wl.name.startswith("g_patch") else "")
    traffic = None if bias else measured_traffic(tag, digest, s.N)
    rec = {
        "workload": wl.name, "note": wl.note, "dtype": wl.dtype,
        "N": s.N, "C": s.C, "H": s.H, "W": s.W, "K": s.K, "R": s.R, "S": s.S, "pad": s.pad,
        "stride": s.stride, "dilation": s.dilation, "groups": s.groups,
        "kernel": FAMILY.get(int(plan.variant), str(plan.variant)), "variant": int(plan.variant),
        "ks_count": int(plan.ks_count), "split_k": args.split_k, "bias_gradient": bool(bias),
        "math": used_math, "fold_width": int(plan2.fold_width), "record": tag,
        "flops": s.flops(), "algorithmic_bytes": s.algorithmic_bytes(wd.IN_BYTES[wl.dtype]),
        "cold_call_us": {"median": round(cold_med * 1e6, 2), "min": round(min(whole) * 1e3, 2),
                         "p90": round(_pct(whole, 0.9) * 1e3, 2), "calls": cold_reps,
                         "timing": source},
        "cold_call_dispatch_stamped_us": round(statistics.median(whole_disp) * 1e3, 2),
        "cold_call_stream_events_us": round(statistics.median(stream_ev) * 1e3, 2) if stream_ev else None,
        "stream_event_floor_us": round(statistics.median(floor) * 1e3, 2) if floor else None,
        "tflops": round(s.flops() / cold_med / 1e12, 3),
        "roofline": roofline_for(s, wl.dtype, cold_med, traffic, used_math),
        "stage1_cold_us": round(statistics.median(stage1) * 1e3, 2),
        "stage1_cold_frac": roofline_for(s, wl.dtype, statistics.median(stage1) * 1e-3, None, used_math)["frac"],
        "hot_call_us": round(wall_plain * 1e6, 2),
        "timed_region_us_per_step": round(wall * 1e6, 2),
        "hot_stage1_us": round(statistics.mean(k_ms) * 1e3, 2),
        "hot_stage1_frac": roofline_for(s, wl.dtype, statistics.mean(k_ms) * 1e-3, None, used_math)["frac"],
        "source_digest": digest,
        "check": {"zeros": int((dw_h == 0).sum()), "finite": bool(np.isfinite(dw_h).all())},
    }
    if s.flops() < 1e6:
        rec["roofline"]["note"] = "launch-latency bound (roofline time ~1 ns): the call time is its latency"
    return rec, wall, statistics.mean(k_ms) * 1e-3


def cpu_baseline_igemm(wl, s, direction, seconds):
    """The fp64 forward or data-gradient oracle on the host cores, on the first
    images of the workload (as many as fit about seconds / 3 per run; at least
    three runs and about `seconds` in all), in TFLOP/s."""
    import oracle
    import wgrad_data as wd
    threads = oracle.default_threads()
    w = wd.draw_filter(wl.seed, s.K, s.R, s.S, s.Cg, wd.Dist("normal", 0.05), wl.dtype)

    def run(n):
        x, dy = wd.make_inputs(wl, 0, n)
        t0 = time.perf_counter()
        if direction == "fwd":
            oracle.fwd_ref(x, w, s.pad, s.stride, s.dilation, s.groups, nthreads=threads)
        else:
            oracle.dgrad_ref(dy, w, s.H, s.W, s.pad, s.stride, s.dilation, s.groups, nthreads=threads)
        return time.perf_counter() - t0

    t_img = max(run(1), 1e-6)
    n_s = int(max(1, min(s.N, (seconds / 3.0) / t_img)))
    times = []
    while len(times) < 3 or (sum(times) < seconds and len(times) < 200):
        times.append(run(n_s))
    t = statistics.median(times)
    per_image = s.flops() / s.N
    what = "whole workload" if n_s == s.N else "first %d of %d images" % (n_s, s.N)
    return {"value": round(per_image * n_s / t / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%s of %s (%s), median of %d runs, fp64 C oracle, %.2f s per run"
                      % (what, wl.name, direction, len(times), t),
            "cpu_model": cpu_model()}


def measure_igemm(wl, s, args, hip, cold_reps, opts):
    """Time the forward convolution or the data gradient (conv_fwd / conv_dgrad) of a
    workload's shape: hot back-to-back calls and cold calls (stream events around
    the implicit GEMM + fold after a 1 GiB clean read)."""
    import numpy as np
    import torch
    import implicit_gemm_amd as iga
    import wgrad_data as wd
    direction = iga.DIRECTION_FWD if opts["direction"] == "fwd" else iga.DIRECTION_DGRAD
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    x, dy = wd.make_inputs(wl)
    w = wd.draw_filter(wl.seed, s.K, s.R, s.S, s.Cg, wd.Dist("normal", 0.05), wl.dtype)
    src = torch.from_numpy(x if direction == iga.DIRECTION_FWD else dy).to(tdt).to(dev)
    wt = torch.from_numpy(w).to(tdt).to(dev)
    split_k = opts.get("split_k", args.split_k)
    d = iga.make_desc2(s.N, s.C, s.H, s.W, s.K, s.R, s.S, s.pad, s.stride, s.dilation, s.groups,
                       {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype], split_k)
    plan2 = iga.get_igemm_plan(d, direction)
    plan = plan2.base
    out = torch.empty(int(plan.E), dtype=torch.float32, device=dev)
    ws_bytes = int(plan.ws_bytes)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    f = iga.conv_fwd if direction == iga.DIRECTION_FWD else iga.conv_dgrad

    def step(ev0=0, ev1=0):
        if ev0 or ev1:
            iga.conv_igemm_call_timed(d, direction, src.data_ptr(), wt.data_ptr(), out.data_ptr(),
                                      ws.data_ptr() if ws_bytes else 0, ws_bytes, sp, ev0, ev1)
        else:
            f(d, src.data_ptr(), wt.data_ptr(), out.data_ptr(), ws.data_ptr() if ws_bytes else 0, ws_bytes, sp)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    # Hot whole calls stamped by their own dispatches (GPU time of K calls).
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        step(a, b)
    torch.cuda.synchronize()
    k_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    # Cold calls after a clean 1 GiB read, stamped the same way.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    probe = torch.empty((), dtype=torch.float32, device=dev)
    e0, e1 = hip.event(), hip.event()
    whole = []
    for _ in range(cold_reps):
        torch.amax(flush, dim=0, out=probe)
        step(e0, e1)
        whole.append(hip.elapsed_ms(e0, e1))
    hip.destroy(e0)
    hip.destroy(e1)
    del flush, probe
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    if not whole:   # --cold 0 (profiling runs): the hot figure stands in
        whole = k_ms
    cold_med = statistics.median(whole) * 1e-3
    hot = statistics.mean(k_ms) * 1e-3
    esz = wd.IN_BYTES[wl.dtype]
    w_bytes = s.K * s.R * s.S * s.Cg * esz
    if direction == iga.DIRECTION_FWD:
        nbytes = s.N * s.H * s.W * s.C * esz + w_bytes + s.N * s.Ho * s.Wo * s.K * 4
    else:
        nbytes = s.N * s.Ho * s.Wo * s.K * esz + w_bytes + s.N * s.H * s.W * s.C * 4
    flops = s.flops()
    peak_mfma = PEAK["mfma_tflops"]["f32"]   # the kernel's products run on f32 MFMA for every dtype
    t_roof = max(flops / (peak_mfma * 1e12), nbytes / (PEAK["hbm_gbs"] * 1e9))
    bound = "mfma" if flops / (peak_mfma * 1e12) >= nbytes / (PEAK["hbm_gbs"] * 1e9) else "hbm"

    tag = "%s+%s%s" % (wl.name, opts["direction"], "+split%d" % split_k if split_k >= 1 else "")
    digest = source_digest(int(plan.variant))
    traffic = measured_traffic(tag, digest, s.N)

    def roof(t):
        if bound == "mfma":
            a = flops / t / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                    "frac": round(a / peak_mfma, 4), "traffic": traffic,
                    "note": "16-bit inputs are widened and multiplied on f32 MFMA"}
        a = nbytes / t / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK["hbm_gbs"], "unit": "GB/s",
                "frac": round(a / PEAK["hbm_gbs"], 4), "traffic": traffic}

    return {
        "workload": wl.name, "record": tag, "direction": opts["direction"], "note": wl.note, "dtype": wl.dtype,
        "N": s.N, "C": s.C, "H": s.H, "W": s.W, "K": s.K, "R": s.R, "S": s.S, "pad": s.pad,
        "stride": s.stride, "dilation": s.dilation, "groups": s.groups,
        "kernel": "igemm_" + opts["direction"], "variant": int(plan.variant), "ks_count": int(plan.ks_count),
        "split_k": split_k, "fold_width": int(plan2.fold_width), "flops": flops, "algorithmic_bytes": nbytes,
        "cold_call_us": {"median": round(cold_med * 1e6, 2), "min": round(min(whole) * 1e3, 2),
                         "p90": round(_pct(whole, 0.9) * 1e3, 2), "calls": cold_reps,
                         "timing": "first kernel start to last kernel end, dispatch-stamped events"},
        "tflops": round(flops / cold_med / 1e12, 3),
        "roofline": roof(cold_med),
        "hot_call_us": round(hot * 1e6, 2), "hot_frac": roof(hot)["frac"], "hot_roofline": roof(hot),
        "hot_wall_us": round(wall * 1e6, 2),
        "roofline_time_us": round(t_roof * 1e6, 2),
        "source_digest": digest,
        "check": {"zeros": int((o == 0).sum()), "finite": bool(np.isfinite(o).all())},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None, help="only this workload (default: all, headline 1x1 N=192)")
    ap.add_argument("--split-k", type=int, default=-1)
    ap.add_argument("--n", type=int, default=0, help="batch of an N-swept workload (default 64)")
    ap.add_argument("--cold", type=int, default=50, help="cold-cache calls per series (1x1 512x512: at most 15)")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed steps after the warm-up steps (clock ramp)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle seconds for the headline cpu_baseline (3 s per other record)")
    ap.add_argument("--math", default="exact", choices=["exact", "bf16x3"],
                    help="with --config: arithmetic for fp32 inputs (bf16x3 where a kernel covers the shape)")
    ap.add_argument("--fold-width", type=int, default=-1, help="with --config: width fold (-1 auto, 0 off)")
    ap.add_argument("--direction", default="wgrad", choices=["wgrad", "fwd", "dgrad"],
                    help="with --config: time the forward convolution or the data gradient instead")
    ap.add_argument("--bias", action="store_true",
                    help="time conv_wgrad_bias (dW and the fused bias gradient db = sum dY)")
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

    import torch
    import implicit_gemm_amd as iga

    if args.digest:
        wl, s = resolve(args.config, args.n) if args.config else resolve(*HEADLINE[:2])
        d = iga.make_desc2(s.N, s.C, s.H, s.W, s.K, s.R, s.S, s.pad, s.stride, s.dilation, s.groups,
                           {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype], args.split_k, args.math, args.fold_width)
        if args.direction == "wgrad":
            v = int(iga.get_plan2(d).base.variant)
        else:
            dirn = iga.DIRECTION_FWD if args.direction == "fwd" else iga.DIRECTION_DGRAD
            v = int(iga.get_igemm_plan(d, dirn).base.variant)
        print(json.dumps({"workload": wl.name, "N": s.N, "variant": v, "source": VARIANT_SOURCE[v],
                          "digest": source_digest(v)}))
        return 0

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    iga.load()
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

    dev = torch.device("cuda:0")
    hip = Hip()
    records = []
    if args.config:
        plan_runs = []
        head_name, head_n = args.config, args.n
        head_opts = {}
        if args.math != "exact":
            head_opts["math"] = args.math
        if args.fold_width != -1:
            head_opts["fold_width"] = args.fold_width
    else:
        plan_runs = ALL_RECORDS
        head_name, head_n, head_opts = HEADLINE

    def cold_reps_for(s):
        return min(args.cold, 15) if s.flops() > 1e11 else args.cold

    big = None   # device inputs of the N-swept workload at the headline batch, shared by its records
    hwl, hs = resolve(head_name, head_n)
    for name, n, opts in plan_runs:
        wl, s = resolve(name, n)
        log("record", wl.name, s, wl.dtype, opts)
        if "direction" in opts:
            rec = measure_igemm(wl, s, args, hip, args.cold, opts)
            if not args.no_cpu:
                rec["cpu_baseline"] = cpu_baseline_igemm(wl, s, opts["direction"], 3.0)
            records.append(rec)
            log(json.dumps(rec))
            torch.cuda.empty_cache()
            continue
        if wl.n_sweep and hwl.name == wl.name and s.N <= hs.N:
            if big is None:
                big = device_inputs(hwl, hs, dev)
            x, dy = big[0][:s.N], big[1][:s.N]
        else:
            x, dy = device_inputs(wl, s, dev)
        rec, _, _ = measure(wl, s, x, dy, args, hip, cold_reps_for(s), args.bias, opts)
        if not args.no_cpu:
            rec["cpu_baseline"] = cpu_baseline(wl, s, 3.0)
        records.append(rec)
        log(json.dumps(rec))
        del x, dy
        torch.cuda.empty_cache()

    if args.config and args.direction != "wgrad":
        opts = {"direction": args.direction}
        rec = measure_igemm(hwl, hs, args, hip, args.cold, opts)
        wall = rec["hot_call_us"] * 1e-6
        print(json.dumps({
            "metric": "wgrad TFLOP/s and % of MFMA-or-HBM roofline per conv shape, 1xMI355X",
            "value": round(hs.flops() / wall / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": hwl.dtype,
            "data": "synthetic (seeded PCG64 per image)",
            "config": {"workload": hwl.name, "direction": args.direction, "N": hs.N, "C": hs.C, "H": hs.H,
                       "W": hs.W, "K": hs.K, "R": hs.R, "S": hs.S, "pad": hs.pad, "stride": hs.stride,
                       "split_k": args.split_k, "ks_count": rec["ks_count"], "kernel": rec["kernel"],
                       "parallelism": "single GPU"},
            "roofline": rec["hot_roofline"], "cpu_baseline": None, "check": rec["check"], "configs": [rec]}),
            flush=True)
        return 0

    log("headline", hwl.name, hs, hwl.dtype)
    if big is None:
        big = device_inputs(hwl, hs, dev)
    rec, wall, stage1_s = measure(hwl, hs, big[0], big[1], args, hip, cold_reps_for(hs), args.bias, head_opts)
    cpu = None if args.no_cpu else cpu_baseline(hwl, hs, args.cpu_seconds)
    if cpu:
        rec["cpu_baseline"] = cpu
    records.append(rec)
    log(json.dumps(rec))
    roof = roofline_for(hs, hwl.dtype, stage1_s, rec["roofline"]["traffic"], rec["math"])
    out = {
        "metric": "wgrad TFLOP/s and % of MFMA-or-HBM roofline per conv shape, 1xMI355X",
        "value": round(hs.flops() / wall / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hwl.dtype,
        "data": "synthetic (seeded PCG64 per image)",
        "config": {"workload": hwl.name, "note": hwl.note, "N": hs.N, "C": hs.C, "H": hs.H, "W": hs.W,
                   "K": hs.K, "R": hs.R, "S": hs.S, "pad": hs.pad, "stride": hs.stride,
                   "dilation": hs.dilation, "groups": hs.groups, "split_k": args.split_k,
                   "ks_count": rec["ks_count"], "kernel": rec["kernel"], "bias_gradient": bool(args.bias),
                   "math": rec["math"], "fold_width": rec["fold_width"],
                   "parallelism": "single GPU"},
        "roofline": roof,
        "whole_call_roofline_frac": roofline_for(hs, hwl.dtype, wall, None, rec["math"])["frac"],
        "stage1_ms_mean": round(stage1_s * 1e3, 5),
        "cpu_baseline": cpu,
        "check": rec["check"],
        "configs": records,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
