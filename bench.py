#!/usr/bin/env python3
"""Benchmark of the grouped-convolution forward engine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-others]
                    [--backward data|filter]

One step = one gconv_fwd call (host validation, route selection, the kernel and
its fused epilogue) on one batch of the workload.  The default workload is the
layer timed in the discuss.pytorch.org thread "F.conv2d runs x15 slower in
mixed-precision/half-precision mode": x [1,512,256,256], w [512,128,3,3],
groups=4, padding 1, no bias, here in fp16 with fp32 accumulation.

Timing: W untimed warm-up steps, then K steps bracketed by
torch.cuda.synchronize().  Inputs are seeded synthetic tensors already resident
in HBM; successive steps rotate over enough copies of the input/output buffers
(>= 512 MB in total) that a step never finds its operands in the 256 MB
Infinity Cache.  The same calls are also captured into a HIP graph (the buffer
sets in turn, at least 16 launches) and replayed, one HIP event pair on the
replay stream around each replay: each replay is one sample of the per-launch
device time (median, p10, p90 reported), and their mean is what the roofline
object uses.  A hot-cache figure repeats the call on one buffer set.

Prints ONE JSON line.  `value` is effective TFLOP/s (2*N*Cout*OH*OW*C/g*KH*KW per
step, padding taps included, divided by the step time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_TFLOPS = {"f16": 2500.0,  # dense MFMA, published
               "bf16": 2500.0,
               "f32": 157.3}   # fp32 vector / fp32 MFMA, published
METRIC = "grouped-conv fwd effective TFLOP/s & GB/s, % roofline, ms per call (1 GPU)"
# The pages' own figure for the headline layer: 60.74 ms median for fp16 (apex O2)
# on a Titan RTX with cuDNN 7.6.3, i.e. 77.31 GFLOP / 60.74 ms.
PAGE_FP16_MS = 60.74


def flops(wl, exact=False):
    from depthwise_convolution_gconv_amd import gconv_out_shape
    ys = gconv_out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    if wl.layout in ("nchw", "nhwc"):
        if wl.layout == "nchw":
            N, Co, OH, OW = ys
            _, Cg, KH, KW = wl.w_shape
            H, W = wl.x_shape[2], wl.x_shape[3]
        else:
            N, OH, OW, Co = ys
            _, KH, KW, Cg = wl.w_shape
            H, W = wl.x_shape[1], wl.x_shape[2]
        if not exact:
            return 2 * N * Co * OH * OW * Cg * KH * KW
        rows = sum(1 for o in range(OH) for k in range(KH)
                   if 0 <= o * wl.stride - wl.pad + k * wl.dilation < H)
        cols = sum(1 for o in range(OW) for k in range(KW)
                   if 0 <= o * wl.stride - wl.pad + k * wl.dilation < W)
        return 2 * N * Co * Cg * rows * cols
    B, To, C = ys
    K = wl.w_shape[2]
    if not exact:
        return 2 * B * To * C * K
    taps = sum(1 for t in range(To) for k in range(K)
               if 0 <= t * wl.stride - wl.pad + k * wl.dilation < wl.x_shape[1])
    return 2 * B * C * taps


def alg_bytes(wl):
    """|x| + |w| + |bias| + |y| in bytes, each touched once."""
    from depthwise_convolution_gconv_amd import gconv_out_shape
    es = 4 if wl.dtype == "f32" else 2
    ys = gconv_out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    n = math.prod(wl.x_shape) + math.prod(wl.w_shape) + math.prod(ys)
    if wl.has_bias:
        n += wl.w_shape[0]
    return n * es


# Arithmetic unit and peak of each kernel (TFLOP/s), with the derivation.  The
# vector-ALU figures hold for the plain (non-packed) instructions the kernels are
# built with: the measurement loops show gfx950 issuing a wave64 v_fma_f32 every
# ~2.3 cycles per SIMD at 8 waves per SIMD (the published fp32 vector peak
# assumes 2 cycles) and a wave64 v_dot2_f32_f16 every ~4.3 cycles.
CLOCK_GHZ, CUS = 2.4, 256
UNITS = {
    "mfma32x32x16": ("mfma", None, "published dense fp16/bf16 MFMA peak (v_mfma_f32_32x32x16_{f16,bf16}, "
                     "32768 FLOP per 32 cycles per SIMD, 256 CUs x 4 SIMDs x 2.4 GHz)"),
    "mfma32x32x2": ("mfma", 157.3, "published fp32 MFMA peak (v_mfma_f32_32x32x2_f32)"),
    "mfma4x4x4": ("mfma", 518.0, "v_mfma_f32_4x4x4_16b_{f16,bf16} has no published peak: 2048 FLOP per "
                  "instruction, which the MFMA-only loop issues every 9.7 cycles per SIMD (518 TFLOP/s "
                  "measured at 2.4 GHz)"),
    "dot2": ("alu", 157.3, "v_dot2_f32_{f16,bf16}: 64 lanes x 4 FLOP per 4 cycles per SIMD, 256 CUs x 4 SIMDs "
             "x 2.4 GHz"),
    "valu": ("alu", 157.3, "published fp32 vector peak (64 lanes x 2 FLOP per 2 cycles per SIMD, 256 CUs x 4 "
             "SIMDs x 2.4 GHz), which plain v_fma_f32 nearly reaches on gfx950 (measured 2.3 cycles per "
             "wave64 instruction)"),
}


def kernel_unit(kernel, dtype):
    """Key into UNITS of the arithmetic a kernel runs on."""
    if kernel.endswith("mfma32x32x16"):
        return "mfma32x32x16"
    if kernel.endswith("mfma32x32x2"):
        return "mfma32x32x2"
    if kernel in ("direct2d_g4", "conv2d_nhwc_g4_mfma") and dtype != "f32":
        return "mfma4x4x4"
    if kernel == "conv2d_nhwc_g4k3_row" and dtype != "f32":
        return "dot2"
    return "valu"


def compute_peak(wl, kernel):
    """(bound name, peak TFLOP/s, derivation) of the arithmetic unit the kernel runs on."""
    unit = kernel_unit(kernel, wl.dtype)
    bound, peak, how = UNITS[unit]
    if unit == "mfma32x32x16":
        peak = PEAK_TFLOPS[wl.dtype]
    return bound, round(peak, 1), how


def source_digest(kernel_file):
    path = os.path.join(ROOT, "depthwise_convolution_gconv_amd", "csrc", kernel_file)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


# Source file of each kernel (as gconv_last_kernel names it).
KERNEL_FILES = {"igemm_fwd_mfma32x32x16": "igemm.hip", "igemm_rows_mfma32x32x16": "igemm_rows.hip",
                "igemm_defer_mfma32x32x16": "igemm_defer.hip",
                "igemm_fwd_f32_mfma32x32x2": "igemm_f32.hip",
                "direct2d_g4": "direct2d.hip", "direct2d_tiled": "direct2d.hip",
                "direct2d_naive": "direct2d.hip", "dw2d_rows": "dw2d.hip", "dw2d_band": "dw2d.hip",
                "dw1d_btc_tile": "dw1d_ntc.hip", "dw1d_btc_window": "dw1d_ntc.hip",
                "dw1d_btc_tile_flip": "dw1d_ntc.hip",
                "dw1d_btc_generic": "dw1d_ntc.hip", "dw2d_nhwc_tile": "nhwc.hip",
                "igemm_nhwc_mfma32x32x16": "igemm_nhwc.hip", "conv2d_nhwc_g4": "nhwc.hip",
                "conv2d_nhwc_g4k3": "nhwc.hip", "conv2d_nhwc_g4k3_row": "nhwc.hip",
                "conv2d_nhwc_g4_mfma": "nhwc.hip", "dw2d_nhwc_pair": "nhwc.hip",
                "conv2d_nhwc_generic": "nhwc.hip"}


def counters_traffic(wl_name, kernel_file):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{wl_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != source_digest(kernel_file):
        return None
    return rec.get("hbm_bytes_per_launch")


def measure(wl, steps, warmup, rotate_bytes=512 << 20, route=None):
    """Time `steps` gconv_fwd calls on rotating buffer sets.  Returns a dict.

    step_ms: `steps` back-to-back calls from Python (host validation, route
    selection and launch included), bracketed by one pair of HIP events on the
    launch stream.  kernel samples: the same calls captured once into a HIP graph
    (the buffer sets in turn, at least 16 launches) and replayed at least 20
    times (about `steps` launches), one pair of HIP events on the replay stream
    around each replay; each sample is the average device duration of one launch
    of that replay, without the host in the loop.  hot samples: the call on one
    buffer set repeated back to back in a graph of its own.  The graph's first
    replay is checked bit for bit against the eager result of the same buffer
    set."""
    import torch
    import depthwise_convolution_gconv_amd as gc
    from depthwise_convolution_gconv_amd.workloads import make_inputs

    dev = torch.device("cuda", 0)
    x, w, b = make_inputs(wl)
    x, w = x.to(dev), w.to(dev)
    b = b.to(dev) if b is not None else None
    ys = gc.gconv_out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    ws_bytes = alg_bytes(wl)
    nsets = min(32, max(1, math.ceil(rotate_bytes / ws_bytes)))
    calls, outs, sets = [], [], []
    for i in range(nsets):
        xi = x if i == 0 else x.clone()
        wi = w if i == 0 else w.clone()
        bi = None if b is None else (b if i == 0 else b.clone())
        yi = torch.empty(ys, dtype=x.dtype, device=dev)
        outs.append(yi)
        sets.append((xi, wi, bi, yi))
        calls.append(gc.PreparedCall(xi, wi, bi, yi, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout,
                                     route=route))
    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        calls[i % nsets]()
    kernel = gc.gconv_last_kernel()
    torch.cuda.synchronize()
    ref0 = outs[0].clone()

    # eager: back-to-back calls
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        calls[i % nsets]()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t_start.elapsed_time(t_end) / steps

    # graph replay: the buffer sets in turn, at least 16 launches per graph (so that
    # the start of a replay is spread over as many launches), no host work in between
    gstream = torch.cuda.Stream(dev)
    gcalls = [gc.PreparedCall(*t, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout, route=route,
                              stream=gstream) for t in sets]
    glaunches = nsets * math.ceil(16 / nsets)
    graph = torch.cuda.CUDAGraph()
    outs[0].zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gstream):
        for i in range(glaunches):
            gcalls[i % nsets]()
    with torch.cuda.stream(gstream):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(outs[0], ref0):
        raise RuntimeError("graph replay differs from the eager result")
    # One event pair per replay: each replay is one sample (the average launch of
    # its passes over the buffer sets), at least 20 of them.
    reps = max(20, round(steps / glaunches))
    cold = replay_samples(graph, gstream, reps, glaunches)
    del graph
    # Hot cache: the call on one buffer set, repeated back to back, so its operands
    # stay in the L2 / Infinity Cache between launches.
    # The graph holds several launches, so that one replay's own start-up cost is
    # spread as it is for the cold graph.
    hot_n = max(nsets, 16)
    hot_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(hot_graph, stream=gstream):
        for _ in range(hot_n):
            gcalls[0]()
    with torch.cuda.stream(gstream):
        hot_graph.replay()
    torch.cuda.synchronize()
    hot = replay_samples(hot_graph, gstream, max(20, round(steps / hot_n)), hot_n)
    del hot_graph
    return {"step_ms": step_ms, "kernel_ms_avg": sum(cold) / len(cold), "kernel_samples": cold,
            "hot_samples": hot, "graph_launches": reps * glaunches, "wall_s": wall, "kernel": kernel,
            "rotation_sets": nsets}


def replay_samples(graph, stream, reps, launches):
    """Replays `graph` `reps` times on `stream`, one HIP event pair around each
    replay; returns the per-launch milliseconds of each replay."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):   # replay() launches on the current stream
        for e0, e1 in evs:
            e0.record(stream)
            graph.replay()
            e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) / launches for e0, e1 in evs]


def stats(samples_ms):
    """Median, p10, p90 (ms) and the count of a list of samples."""
    import numpy as np
    a = np.asarray(samples_ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "samples": int(a.size)}


def measure_dw1d_backward(wl, kind, steps, rotate_bytes=512 << 20):
    """Per-call device time of the input gradient (kind "data") or the filter and
    bias gradients (kind "filter", two kernels per call) of the depthwise conv1d of
    workload `wl`, from a replayed HIP graph of one call per rotating buffer set
    (one event pair per replay on the replay stream).  Returns (per-call ms of each
    replay, kernel name)."""
    import torch
    import depthwise_convolution_gconv_amd as gc
    from depthwise_convolution_gconv_amd.workloads import draw, make_inputs

    dev = torch.device("cuda", 0)
    x, w, _ = make_inputs(wl)
    B, T, C = wl.x_shape
    K = wl.w_shape[2]
    To = gc.gconv_out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, "ntc")[1]
    dy = draw((B, To, C), 1.0, 4000 + wl.index, wl.dtype)
    x, w, dy = x.to(dev), w.to(dev), dy.to(dev)
    nsets = min(32, max(1, math.ceil(rotate_bytes / bwd_bytes(wl, kind))))
    sets = []
    for i in range(nsets):
        xi, dyi = (x, dy) if i == 0 else (x.clone(), dy.clone())
        if kind == "data":
            sets.append((dyi, w, torch.empty_like(xi)))
        else:
            ws = torch.empty(gc.gconv_dw1d_bwd_filter_workspace(wl.x_shape, wl.w_shape, wl.stride, wl.pad,
                                                                wl.dilation, wl.dtype), dtype=torch.uint8, device=dev)
            sets.append((xi, dyi, torch.empty_like(w), torch.empty(C, dtype=w.dtype, device=dev), ws))
    gstream = torch.cuda.Stream(dev)

    def call(st):
        if kind == "data":
            gc.gconv_dw1d_bwd_data(st[0], st[1], T, wl.stride, wl.pad, wl.dilation, dx=st[2], stream=gstream)
        else:
            gc.gconv_dw1d_bwd_filter(st[0], st[1], K, wl.stride, wl.pad, wl.dilation, dw=st[2], db=st[3],
                                     workspace=st[4], stream=gstream)

    with torch.cuda.stream(gstream):
        for st in sets[:3]:
            call(st)
    kernel = gc.gconv_last_kernel()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gstream):
        for st in sets:
            call(st)
    with torch.cuda.stream(gstream):
        graph.replay()
    torch.cuda.synchronize()
    samples = replay_samples(graph, gstream, max(20, round(steps / nsets)), nsets)
    del graph
    return samples, kernel


def bwd_bytes(wl, kind):
    """Algorithmic bytes of one backward call: dy + w + dx (data), x + dy + dw + db (filter)."""
    es = 4 if wl.dtype == "f32" else 2
    B, T, C = wl.x_shape
    K = wl.w_shape[2]
    To = (T + 2 * wl.pad - wl.dilation * (K - 1) - 1) // wl.stride + 1
    if kind == "data":
        return (B * To * C + C * K + B * T * C) * es
    return (B * T * C + B * To * C + C * K + C) * es


def bwd_entry(wl, kind, steps, name=None, peaks=None):
    samples, kernel = measure_dw1d_backward(wl, kind, steps)
    ms = sum(samples) / len(samples)
    byts = bwd_bytes(wl, kind)
    B, T, C = wl.x_shape
    K = wl.w_shape[2]
    To = (T + 2 * wl.pad - wl.dilation * (K - 1) - 1) // wl.stride + 1
    f = 2 * B * To * C * K
    gbs = byts / (ms * 1e-3) / 1e9
    rf = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": round(gbs / PEAK_HBM_GBS, 4),
          "traffic": counters_traffic(name, "dw1d_ntc.hip" if kind == "data" else "dw1d_wgrad.hip")
          if name else None}
    if peaks:
        rf["measured_peak"] = peaks["hbm_stream_copy"]["gb_per_s"]
        rf["frac_of_measured"] = round(gbs / rf["measured_peak"], 4)
    return {"kernel": kernel, "kernel_ms_avg": round(ms, 5), "kernel_ms": stats(samples),
            "tflops": round(f / (ms * 1e-3) / 1e12, 3), "gb_per_s": round(gbs, 1), "roofline": rf}


def autotune_entries(workloads, steps):
    import torch
    import depthwise_convolution_gconv_amd as gc
    from depthwise_convolution_gconv_amd.workloads import make_inputs
    out = {}
    for name, wl in workloads.items():
        ms = {}
        for r in ("direct", "igemm"):
            try:
                ms[r] = round(measure(wl, max(10, steps // 10), 2, route=r)["kernel_ms_avg"], 5)
            except gc.GconvError:
                pass
        x, w, b = (None if t is None else t.cuda() for t in make_inputs(wl))
        gc.gconv_autotune_clear()
        tuned = gc.gconv_autotune(x, w, b, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout, reps=5)
        gc.gconv_autotune_clear()
        del x, w, b
        torch.cuda.empty_cache()
        out[name] = {"static": route_of(wl), "tuned": tuned, "kernel_ms_by_route": ms}
    return out


_PEAKS = None


def peaks_lib():
    """libgconv_peaks.so: the MFMA-only loop and streaming-copy kernels (csrc/peaks.hip)."""
    global _PEAKS
    if _PEAKS is None:
        import ctypes
        path = os.path.join(ROOT, "depthwise_convolution_gconv_amd", "libgconv_peaks.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build with python -m depthwise_convolution_gconv_amd.build")
        L = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.gconv_peak_mfma_flop.argtypes = [i32, i32]
        L.gconv_peak_mfma_flop.restype = ctypes.c_double
        L.gconv_peak_mfma.argtypes = [i32, vp, i32, i32, vp, vp]
        L.gconv_peak_mfma.restype = i32
        L.gconv_peak_stream_copy.argtypes = [vp, vp, i64, vp]
        L.gconv_peak_stream_copy.restype = i32
        L.gconv_peak_tile_copy.argtypes = [vp, vp, i64, i32, vp]
        L.gconv_peak_tile_copy.restype = i32
        _PEAKS = L
    return _PEAKS


# Loops of the measurement library: name -> (kind, FLOP per instruction per wave,
# workgroups of 4 waves per CU, i.e. waves per SIMD).  Each runs at the
# occupancy where its rate levels off: two waves per SIMD for the long 32x32
# MFMAs (one leaves the issue gaps between instructions open), four for the
# short 4x4x4 MFMA, eight for the vector-ALU loops (one wave's loop bookkeeping
# issues beside the others' arithmetic).
PEAK_LOOPS = {"mfma_f16_32x32x16": (0, 2 * 32 * 32 * 16, 2), "mfma_f32_32x32x2": (1, 2 * 32 * 32 * 2, 2),
              "mfma_f16_4x4x4_16b": (2, 2 * 16 * 64, 4), "mfma_bf16_4x4x4_16b": (3, 2 * 16 * 64, 4),
              "valu_fma_f32": (4, 2 * 64, 8), "valu_dot2_f16": (5, 4 * 64, 8)}


def mfma_peak(kind, flop_per_instr, wgs_per_cu=1, iters=20000, reps=3):
    """Rate of an arithmetic-only loop of the measurement library (PEAK_LOOPS),
    `wgs_per_cu` workgroups of 4 waves per CU, in TFLOP/s; the core clock during the
    loop (shader clock counter over the 100 MHz real-time counter, wave 0 of
    workgroup 0); and the cycles one SIMD spends per instruction at that clock."""
    import torch
    L = peaks_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * wgs_per_cu
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert L.gconv_peak_mfma(kind, out.data_ptr(), blocks, 100, clk.data_ptr(), st) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        assert L.gconv_peak_mfma(kind, out.data_ptr(), blocks, iters, clk.data_ptr(), st) == 0
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    c = clk.cpu().tolist()
    ghz = (c[2] - c[0]) / ((c[3] - c[1]) / 100e6) / 1e9 if c[3] > c[1] else None
    tflops = L.gconv_peak_mfma_flop(kind, iters) * blocks / t / 1e12
    cyc = None
    if ghz:
        cyc = flop_per_instr * 4 / (tflops * 1e12 / (cus * ghz * 1e9))
    return {"tflops": round(tflops, 1), "clock_ghz": None if ghz is None else round(ghz, 3),
            "cycles_per_instr_per_simd": None if cyc is None else round(cyc, 2), "waves_per_simd": wgs_per_cu}


def measure_peaks(conformer=None):
    """What this GPU sustains: every arithmetic loop of PEAK_LOOPS, the library's
    own streaming copy and torch's device copy of 1 GiB, and, given the Conformer
    depthwise workload, a plain copy of its tensor on its kernel's tile grid."""
    out = {name: mfma_peak(kind, fpi, wgs) for name, (kind, fpi, wgs) in PEAK_LOOPS.items()}
    out["hbm_stream_copy"] = {"gb_per_s": stream_peak_gbs(),
                              "how": "csrc/peaks.hip stream_copy, 1 GiB, 10 launches; read + write bytes"}
    out["hbm_torch_copy"] = {"gb_per_s": copy_peak_gbs(), "how": "torch copy_ of 1 GiB, 10 launches"}
    if conformer is not None:
        B, T, C = conformer.x_shape
        out["conformer_tile_copy"] = tile_copy_floor(B * T, C)
    out["clock"] = {"ghz_during_mfma_f16_loop": out["mfma_f16_32x32x16"]["clock_ghz"],
                    "ghz_during_valu_loop": out["valu_fma_f32"]["clock_ghz"], "peak_ghz": CLOCK_GHZ}
    return out


def stream_peak_gbs(nbytes=1 << 30, reps=10):
    """HBM bandwidth (read + write bytes per second) of the library's own streaming
    copy: one non-temporal 16-byte load and store per thread."""
    import torch
    L = peaks_lib()
    src = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    n16 = nbytes // 16
    assert L.gconv_peak_stream_copy(src.data_ptr(), dst.data_ptr(), n16, st) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.gconv_peak_stream_copy(src.data_ptr(), dst.data_ptr(), n16, st)
    e1.record()
    torch.cuda.synchronize()
    ok = bool(torch.equal(src, dst))
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    if not ok:
        raise RuntimeError("stream copy check failed")
    return round(gbs, 1)


def tile_copy_floor(rows, C, steps=200, rotate_bytes=512 << 20):
    """Per-launch time of a plain copy of a rows x C fp32 tensor on the grid of the
    (batch, steps, channels) depthwise kernel (tiles of 32 rows x 64 channels, one
    workgroup each, 16-byte loads, non-temporal stores), rotated over cold buffer
    sets and replayed from a HIP graph like the convolution itself."""
    import torch
    L = peaks_lib()
    nbytes = rows * C * 4
    nsets = min(32, max(1, math.ceil(rotate_bytes / (2 * nbytes))))
    bufs = [(torch.ones(rows * C, dtype=torch.float32, device="cuda"),
             torch.empty(rows * C, dtype=torch.float32, device="cuda")) for _ in range(nsets)]
    gs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gs):
        for a, b in bufs:
            L.gconv_peak_tile_copy(a.data_ptr(), b.data_ptr(), rows, C, gs.cuda_stream)
    with torch.cuda.stream(gs):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(bufs[0][0], bufs[0][1]):
        raise RuntimeError("tile copy check failed")
    samples = replay_samples(graph, gs, max(20, round(steps / nsets)), nsets)
    del graph, bufs
    torch.cuda.empty_cache()
    us = 1e3 * sum(samples) / len(samples)
    return {"us_per_launch": round(us, 2), "gb_per_s": round(2 * nbytes / (us * 1e-6) / 1e9, 1),
            "bytes_per_launch": 2 * nbytes, "ms_per_launch": stats(samples),
            "how": "csrc/peaks.hip tile_copy: 32 x 64 fp32 tiles, one workgroup each, 16-byte loads and "
                   "non-temporal stores, cold buffer sets replayed from a HIP graph"}


def copy_peak_gbs(nbytes=1 << 30, reps=10):
    """HBM bandwidth a plain device copy reaches on this GPU (read + write bytes per
    second), the measured counterpart of the published 8 TB/s."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


MEASURED_KEY = {"mfma32x32x16": "mfma_f16_32x32x16", "mfma32x32x2": "mfma_f32_32x32x2",
                "mfma4x4x4": "mfma_bf16_4x4x4_16b", "dot2": "valu_dot2_f16", "valu": "valu_fma_f32"}


def roofline(wl, kernel, kernel_ms, traffic, peaks=None):
    """Roofline object of one kernel: the bound (HBM or the kernel's arithmetic unit,
    whichever takes longer at the published peaks), the achieved rate from the
    algorithmic FLOP or bytes and the average launch time, and its fraction of the
    published peak; with `peaks` (measure_peaks()) also of the measured one."""
    f = flops(wl)
    byts = alg_bytes(wl)
    cname, cpeak, how = compute_peak(wl, kernel)
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    t_cmp = f / (cpeak * 1e12)
    t = kernel_ms * 1e-3
    if t_hbm >= t_cmp:
        rf = {"bound": "hbm", "achieved": round(byts / t / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": round(byts / t / 1e9 / PEAK_HBM_GBS, 4), "traffic": traffic,
              "compute_peak": {"unit": kernel_unit(kernel, wl.dtype), "tflops": cpeak, "derivation": how}}
        if peaks:
            m = peaks["hbm_stream_copy"]["gb_per_s"]
            rf["measured_peak"] = m
            rf["frac_of_measured"] = round(rf["achieved"] / m, 4)
        return rf
    rf = {"bound": cname, "achieved": round(f / t / 1e12, 2), "peak": cpeak, "unit": "TFLOP/s",
          "frac": round(f / t / 1e12 / cpeak, 4), "traffic": traffic, "peak_derivation": how}
    if peaks:
        key = MEASURED_KEY[kernel_unit(kernel, wl.dtype)]
        if wl.dtype == "f16" and key == "mfma_bf16_4x4x4_16b":
            key = "mfma_f16_4x4x4_16b"
        m = peaks[key]["tflops"]
        rf["measured_peak"] = m
        rf["measured_peak_of"] = key
        rf["frac_of_measured"] = round(rf["achieved"] / m, 4)
    return rf


def cpu_baseline(wl, target_s=10.0):
    """The fp64 oracle, unmodified, timed on the host cores on a random sample
    of the workload's outputs (each evaluated one by one)."""
    import numpy as np
    import oracle
    from depthwise_convolution_gconv_amd.workloads import as_f64, make_inputs
    from depthwise_convolution_gconv_amd import gconv_out_shape
    x, w, b = make_inputs(wl)
    xd, wd, bd = as_f64(x), as_f64(w), as_f64(b)
    ys = gconv_out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    total = math.prod(ys)
    per_point = 2 * math.prod(wl.w_shape[1:])
    rng = np.random.default_rng(12345)

    def run(n):
        idx = rng.integers(0, total, n)
        t0 = time.perf_counter()
        if wl.layout == "nchw":
            oracle.conv2d_at(xd, wd, idx, bd, wl.stride, wl.pad, wl.dilation, wl.groups)
        else:
            oracle.dwconv1d_btc_at(xd, wd, idx, bd, wl.stride, wl.pad, wl.dilation)
        return time.perf_counter() - t0

    # Size the sample in two steps: a tiny first probe is dominated by the thread
    # start-up, so a second one of about a second sets the rate.
    n, dt = 4096, 0.0
    for goal in (1.0, target_s):
        dt = run(n)
        n = int(min(max(n, n * goal / max(dt, 1e-6)), 50_000_000))
    dt = run(n)
    return {"value": round(per_point * n / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n} random outputs of the workload, each evaluated by the oracle's point "
                      f"function (fp64, {per_point} FLOP each, padding taps counted), {dt:.1f} s"}


def route_of(wl):
    import depthwise_convolution_gconv_amd as gc
    return gc.gconv_select_route(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups,
                                 wl.layout, wl.dtype)


def kernel_file(kernel):
    return KERNEL_FILES[kernel]


def timing(m):
    """Timing object of one workload for the JSON line."""
    return {"avg_per_launch": round(m["kernel_ms_avg"], 5), "cold": stats(m["kernel_samples"]),
            "hot": stats(m["hot_samples"]), "graph_launches": m["graph_launches"],
            "rotation_sets": m["rotation_sets"],
            "how": "HIP graph of the cold buffer sets in turn (at least 16 launches), one event pair per "
                   "replay on the replay stream (cold); one buffer set repeated back to back (hot, operands "
                   "in L2 / Infinity Cache)"}


def measure_entry(wl, steps, peaks=None):
    """Timing and roofline of one non-headline workload (a dict for the JSON line)."""
    route = route_of(wl)
    m = measure(wl, max(20, steps // 2), 5)
    rf = roofline(wl, m["kernel"], m["kernel_ms_avg"], counters_traffic(wl.name, kernel_file(m["kernel"])), peaks)
    e = {"route": route, "kernel": m["kernel"], "ms_per_step": round(m["step_ms"], 5),
         "kernel_ms": timing(m),
         "tflops": round(flops(wl) / (m["kernel_ms_avg"] * 1e-3) / 1e12, 3),
         "gb_per_s": round(alg_bytes(wl) / (m["kernel_ms_avg"] * 1e-3) / 1e9, 1),
         "roofline": rf}
    floor = conformer_floor(wl, m, peaks)
    if floor:
        e["tile_copy_floor"] = floor
    return e


def conformer_floor(wl, m, peaks):
    """For the Conformer depthwise workload: its kernel time against the plain copy of
    the same tensor on the same tile grid (measure_peaks)."""
    if not peaks or "conformer_tile_copy" not in peaks or wl.name != "c3_dw1d_btc_f32":
        return None
    fl = peaks["conformer_tile_copy"]["us_per_launch"]
    return {"copy_us_per_launch": fl, "kernel_us_per_launch": round(m["kernel_ms_avg"] * 1e3, 2),
            "kernel_over_copy": round(m["kernel_ms_avg"] * 1e3 / fl, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured peaks (arithmetic loops, copies)")
    ap.add_argument("--peaks-only", action="store_true", help="only print the measured peaks")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--backward", choices=["data", "filter"], default=None,
                    help="only time the backward of the Conformer depthwise conv1d (input or filter gradient)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 plain device copies of 256 MiB (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the forward conv shards by batch or group with no communication; "
              "multi-GPU runs are not part of this engine).", file=sys.stderr)
        sys.exit(2)

    import torch
    from depthwise_convolution_gconv_amd.workloads import HEADLINE, NEXT_WORKLOADS, WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate_copy:
        nbytes = 256 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": nbytes, "copy_bytes_written_per_launch": nbytes,
                          "launches": 5}))
        return

    if args.backward:
        print(json.dumps({"backward": args.backward, "workload": "c3_dw1d_btc_f32",
                          **bwd_entry(WORKLOADS["c3_dw1d_btc_f32"], args.backward, args.steps,
                                      "n5_dw1d_bwd_data_f32" if args.backward == "data"
                                      else "n6_dw1d_bwd_filter_f32")}))
        return

    if args.peaks_only:
        print(json.dumps({"measured_peaks": measure_peaks(WORKLOADS["c3_dw1d_btc_f32"])}))
        return

    name = args.workload or HEADLINE
    wl = {**WORKLOADS, **NEXT_WORKLOADS}[name]
    route = route_of(wl)
    m = measure(wl, args.steps, args.warmup)
    kfile = kernel_file(m["kernel"])
    peaks = None if args.no_peaks else measure_peaks(WORKLOADS["c3_dw1d_btc_f32"])
    f = flops(wl)
    value = f / (m["step_ms"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (f / (PAGE_FP16_MS * 1e-3) / 1e12), 2) if name == "c2_p2layer_f16" else None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) x, N(0,1/fan_in) w; no dataset)",
        "config": {"workload": name, "x": list(wl.x_shape), "w": list(wl.w_shape), "groups": wl.groups,
                   "stride": wl.stride, "pad": wl.pad, "dilation": wl.dilation, "bias": wl.has_bias,
                   "layout": wl.layout, "route": route, "kernel": m["kernel"],
                   "rotation_sets": m["rotation_sets"]},
        "gb_per_s": round(alg_bytes(wl) / (m["step_ms"] * 1e-3) / 1e9, 1),
        "kernel_ms": timing(m),
        "roofline": roofline(wl, m["kernel"], m["kernel_ms_avg"], counters_traffic(name, kfile), peaks),
    }
    floor = conformer_floor(wl, m, peaks)
    if floor:
        out["tile_copy_floor"] = floor
    if peaks:
        out["measured_peaks"] = peaks
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    if not args.no_others:
        out["others"] = {oname: measure_entry(owl, args.steps, peaks)
                         for oname, owl in WORKLOADS.items() if oname != name}
        # Strided depthwise layers (beyond the five workloads above).
        out["next"] = {oname: measure_entry(owl, args.steps, peaks)
                       for oname, owl in NEXT_WORKLOADS.items() if oname != name}
        # Per-shape route tuning: each route that runs the workload, timed as above,
        # beside the static choice and the route gconv_autotune records.
        out["autotune"] = autotune_entries(WORKLOADS, args.steps)
        # Backward of the Conformer depthwise conv1d (same shapes as its forward).
        conf = WORKLOADS["c3_dw1d_btc_f32"]
        for bname, kind in (("n5_dw1d_bwd_data_f32", "data"), ("n6_dw1d_bwd_filter_f32", "filter")):
            out["next"][bname] = bwd_entry(conf, kind, args.steps, bname, peaks)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
