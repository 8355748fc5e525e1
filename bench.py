"""Benchmark of the MX quantize-dequantize hot path on one MI355X.

One step = one pass of the whole path over the resident 8192 x 57344 bf16
layer (the largest Llama-3.1-70B layer shape the pages benchmark, read as
M x K; values N(0, 0.02^2) with 1/1024 subnormal-range and 1/1024
saturating groups):
  mx_qdq      MXFP4 and MXFP8, rotation none / 16 / 64 / 128 (normalised
              Hadamard, bf16), bf16 out                       -- 8 launches
  mx_quantize MXFP4 and MXFP8, rotation none / 128, codes + E8M0 scales
                                                               -- 4 launches
value = algorithmic bytes of the step / step time (GB = 1e9 B).  Algorithmic
bytes per element: QDQ 2 + 2; quantize 2 + 0.5 + 1/32 (MXFP4) or 2 + 1 + 1/32
(MXFP8); the rotation matrix (<= 32 KiB) is not counted.

Each launch is bracketed by HIP events on the stream it runs on (the binding
launches on torch's current stream): one event before the step's first
launch and one after every launch, so that consecutive launches share the
event between them (each event record costs the GPU a few microseconds; two
per launch made the step 1.5% slower).  The roofline entry is the launch of
the step with the longest average duration: its algorithmic bytes over that
duration, against 8 TB/s.

Beside the step:
  - measured ceilings: a 16-byte streaming copy, read-only and write-only
    kernel (bench_ceiling.hip, built outside the library; the best of six
    launch shapes each) and the runtime's device-to-device copy, all on the
    layer's bytes; every kernel also reports its fraction of the copy
    ceiling;
  - the other workloads, each timed on its own seeded input: MXFP4 QDQ of a
    128 x 4096 activation (launch-bound, timed by graph replay), MXFP8 QDQ
    and quantize of 8192 x 8192, MXFP4 QDQ with rotation 32 of 4096 x 8192,
    MXFP4 quantize with rotation 128 and without of 8192 x 28672, and MXFP4
    and MXFP8 QDQ with rotation none / 16 / 64 of the 8192 x 8192 and
    28672 x 8192 layers; inputs under 1 GB are evicted from the 256 MB
    last-level cache between timed launches by a 512 MiB write;
  - dequantize, the layer read as 57344 x 8192, fp32 sources (QDQ without
    rotation, with rotation 16, and with rotation 128 on the fp32 matrix
    cores), the rotation alone (r = 16, 128), NVFP4,
    blocked scales and the GEMM that consumes the quantized layer.
The CPU baseline runs the oracle (unchanged) on a bounded row sample of the
same layer and variants, on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
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

PEAK_GBPS = 8000.0
METRIC = "effective HBM GB/s (and % of MI355X peak) for MXFP4/MXFP8 QDQ per layer"
WORKLOAD = "c5b"


def variants():
    out = []
    for fmt in (0, 1):
        for r in (0, 16, 64, 128):
            out.append(("qdq", fmt, r))
    for fmt in (0, 1):
        for r in (0, 128):
            out.append(("quantize", fmt, r))
    return out


def bytes_per_element(op, fmt):
    if op == "qdq":
        return 4.0
    return 2.0 + (0.5 if fmt == 0 else 1.0) + 1.0 / 32.0


def name_of(op, fmt, r):
    return f"{op}_{'mxfp4' if fmt == 0 else 'mxfp8'}_rot{r}"


STEP_SOURCES = ("unrot.hip", "rot.hip", "rotl.hip", "mx_device.h")  # what the step's kernels are built from


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "microscaling_quantize_dequantize_amd", "csrc")
    for f in STEP_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_name):
    """HBM bytes per launch (fetched + written) from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != source_hash():
        return None
    k = d.get("kernels", {}).get(kernel_name)
    return None if k is None else k["total_bytes"]


def cpu_baseline(x_bits, rots, rows, rows_1t):
    import numpy as np

    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))

    def run(sample, t):
        total = 0.0
        t0 = time.perf_counter()
        for op, fmt, r in variants():
            R = rots[r][0] if r else None
            if op == "qdq":
                oracle.qdq(fmt, sample, R, r, threads=t)
            else:
                oracle.quantize(fmt, sample, R, r, threads=t)
            total += sample.size * bytes_per_element(op, fmt)
        return total, time.perf_counter() - t0

    sample = np.ascontiguousarray(x_bits[:rows])
    total_bytes, dt = run(sample, threads)
    b1, dt1 = run(np.ascontiguousarray(x_bits[:rows_1t]), 1)
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0-{rows - 1} of the 8192x57344 layer ({sample.size} elements), all 12 step "
                      f"variants, {dt:.1f} s wall on {threads} threads; single thread: rows 0-{rows_1t - 1}, "
                      f"{dt1:.1f} s", "seconds": round(dt, 2),
            "single_thread_value": round(b1 / dt1 / 1e9, 5),
            "host": host_cpu()}


def host_cpu():
    model, smt = None, None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        smt = open("/sys/devices/system/cpu/smt/active").read().strip() == "1"
    except OSError:
        pass
    return {"model": model, "nproc": os.cpu_count(), "smt": smt}


def timed(fn, reps):
    """Average and minimum duration (ms) of fn() over reps launches, each
    bracketed by events on torch's current stream."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(ms)), float(np.min(ms))


def timed_graph(fn, reps):
    """Average duration (ms) of fn() for kernels shorter than the host's launch
    path: reps launches captured back to back in one HIP graph, replayed
    three times (the library launches on torch's current stream, which is
    the capture stream while capturing, and records no memset)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    ms = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / reps)
    return float(min(ms)), float(min(ms))


GEMM_PEAK_TFLOPS = {0: 10100.0, 1: 5000.0}  # MI355X dense fp4 / fp8 matrix peaks


def ceiling_lib():
    """The streaming ceiling kernels (bench_ceiling.so, built by
    __graft_entry__.build())."""
    import ctypes
    path = os.path.join(ROOT, "bench_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit("bench_ceiling.so is missing: run `python __graft_entry__.py build` first")
    L = ctypes.CDLL(path)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    L.ceil_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    L.ceil_read.argtypes = [vp, i64, vp, u32, i32, i32, vp]
    L.ceil_write.argtypes = [vp, i64, u32, i32, i32, vp]
    for f in (L.ceil_copy, L.ceil_read, L.ceil_write):
        f.restype = i32
    return L


def _stream_ptr():
    import torch
    return torch.cuda.current_stream().cuda_stream


def measure_ceilings(L, x, copy_dst):
    """Best GB/s of the copy, read-only and write-only kernels over the
    launch shapes (64, 128 or 256 threads per workgroup; 1, 2 or 4 pieces
    per thread), and of the runtime's device-to-device copy, each on the
    bytes of x."""
    import torch
    nbytes = x.numel() * x.element_size()
    sink = torch.zeros(64, dtype=torch.int32, device=x.device)

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel returned {rc}")

    kinds = {
        "copy": (lambda t, u: check(L.ceil_copy(x.data_ptr(), copy_dst.data_ptr(), nbytes, t, u, _stream_ptr())),
                 2 * nbytes),
        "read": (lambda t, u: check(L.ceil_read(x.data_ptr(), nbytes, sink.data_ptr(), 0x9E3779B9, t, u,
                                                _stream_ptr())),
                 nbytes),
        "write": (lambda t, u: check(L.ceil_write(copy_dst.data_ptr(), nbytes, 0x3F803F80, t, u, _stream_ptr())),
                  nbytes),
    }
    out = {}
    for kind, (fn, b) in kinds.items():
        best = None
        for t, u in ((64, 1), (64, 2), (128, 1), (256, 1), (256, 2), (256, 4)):
            fn(t, u)
            avg, mn = timed(lambda: fn(t, u), 10)
            gbps = b / (avg * 1e-3) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, t, u, avg)
        out[kind] = {"GBps": round(best[0], 1), "threads": best[1], "pieces_per_thread": best[2],
                     "avg_us": round(best[3] * 1e3, 2), "bytes": int(b)}
    for _ in range(2):
        copy_dst.copy_(x)
    avg, _ = timed(lambda: copy_dst.copy_(x), 10)
    out["runtime_copy"] = {"GBps": round(2 * nbytes / (avg * 1e-3) / 1e9, 1), "avg_us": round(avg * 1e3, 2),
                           "bytes": int(2 * nbytes)}
    return out


def timed_flushed(fn, reps, flush):
    """As timed(), with flush() (a 512 MiB write that evicts the 256 MB
    last-level cache) between launches, outside the events."""
    import numpy as np
    import torch
    ms = []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.mean(ms)), float(np.min(ms))


# The other workloads: (name, [(op, fmt, rotation), ...]).  The 8192 x 57344
# layer is the step itself.
CONFIGS = [
    ("c1", [("qdq", 0, 0)]),
    ("c2", [("qdq", 1, 0), ("quantize", 1, 0)]),
    ("c3", [("qdq", 0, 32)]),
    ("c4", [("quantize", 0, 128), ("quantize", 0, 0)]),
    ("c5a", [("qdq", f, r) for f in (0, 1) for r in (0, 16, 64)]),
    ("c5c", [("qdq", f, r) for f in (0, 1) for r in (0, 16, 64)]),
]

CONFIG_TEXT = {
    "c1": "128x4096 activation, N(0,1) with 0.1% x50 outliers and 4 zero groups",
    "c2": "8192x8192, 0.5 * Student-t(4), every 64th row x1000",
    "c3": "4096x8192, N(0,1) with LogNormal(0,1) column scales",
    "c4": "8192x28672 down-projection input, Student-t(3)",
    "c5a": "8192x8192 layer, N(0,0.02^2) with subnormal-range and saturating groups",
    "c5c": "28672x8192 layer, N(0,0.02^2) with subnormal-range and saturating groups",
}


def progress(msg):
    """A phase of the run, on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_configs(mx, W, flush, copy_gbps):
    """Each workload on its own seeded input: average and minimum launch
    time, GB/s, fraction of 8 TB/s and of the copy ceiling, and the rotated
    over unrotated ratios."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    rows, ratios = [], {}
    for name, vs in CONFIGS:
        progress(f"workload {name}")
        xb = W.generate(name)
        M, K = xb.shape
        n = M * K
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        del xb
        dst = torch.empty_like(x)
        codes = {0: torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                 1: torch.empty((M, K), dtype=torch.uint8, device=dev)}
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        times = {}
        for op, fmt, r in vs:
            R = None
            if r:
                Rb = W.hadamard_rotation(r)
                R = torch.from_numpy(Rb.view(np.int16)).view(torch.bfloat16).to(dev)
            cv = codes[fmt]
            if op == "qdq":
                fn = (lambda fmt=fmt, R=R: mx.mx_qdq(fmt, x, rot=R, dst=dst))
            else:
                fn = (lambda fmt=fmt, R=R, cv=cv: mx.mx_quantize(fmt, x, rot=R, codes=cv, scales=scales))
            b = n * bytes_per_element(op, fmt)
            for _ in range(2):
                fn()
            if name == "c1":
                avg, mn = timed_graph(fn, 200)
                how = "graph replay of 200 back-to-back launches (L2-resident, launch-bound)"
            else:
                avg, mn = timed_flushed(fn, 10, flush) if 2 * b < 1e9 else timed(fn, 10)
                how = "events per launch" + (", cache evicted between launches" if 2 * b < 1e9 else "")
            gbps = b / (avg * 1e-3) / 1e9
            key = name_of(op, fmt, r)
            times[key] = avg
            rows.append({"config": name, "workload": CONFIG_TEXT[name], "M": M, "K": K, "kernel": key,
                         "bytes": int(b), "avg_us": round(avg * 1e3, 2), "min_us": round(mn * 1e3, 2),
                         "GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4),
                         "frac_of_copy": round(gbps / copy_gbps, 4), "elements_per_s": round(n / (avg * 1e-3), 1),
                         "timing": how})
        for key, t in times.items():
            op, f, rot = key.split("_")
            base = f"{op}_{f}_rot0"
            if rot != "rot0" and base in times:
                ratios[f"{name}_{op}_{rot}_over_rot0_{f}"] = round(t / times[base], 3)
        del x, dst, codes, scales
        torch.cuda.empty_cache()
    return rows, ratios


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--cpu-rows-1t", type=int, default=64)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the MX QDQ path shards by rows with no exchange, "
              "so one GPU's throughput is the measurement; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from microscaling_quantize_dequantize_amd import binding as mx
    from microscaling_quantize_dequantize_amd import workloads as W
    CL = ceiling_lib()

    dev = torch.device("cuda:0")
    progress("generating the 8192x57344 layer")
    x_bits = W.generate(WORKLOAD)
    M, K = x_bits.shape
    n = M * K
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    rots = {}
    for r in (16, 64, 128):
        Rb = W.hadamard_rotation(r)
        rots[r] = (Rb, torch.from_numpy(Rb.view(np.int16)).view(torch.bfloat16).to(dev))
    dst = torch.empty_like(x)
    codes = {0: torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
             1: torch.empty((M, K), dtype=torch.uint8, device=dev)}
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(x)

    var = variants()

    def launch(op, fmt, r):
        R = rots[r][1] if r else None
        if op == "qdq":
            mx.mx_qdq(fmt, x, rot=R, dst=dst)
        else:
            mx.mx_quantize(fmt, x, rot=R, codes=codes[fmt], scales=scales)

    def step(events=None):
        # events[i] and events[i + 1] bracket launch i
        if events is not None:
            events[0].record()
        for i, v in enumerate(var):
            launch(*v)
            if events is not None:
                events[i + 1].record()

    progress("step: warm-up and timed steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(var) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    progress("beside the step: dequantize, layout, NVFP4, blocked scales, GEMM")
    # beside the step: dequantize of the step's codes, the transposed layout
    # of the layer, and the GEMM that consumes quantized operands
    deq_out = torch.empty_like(x)
    extras = []
    for fmt in (0, 1):
        mx.mx_quantize(fmt, x, codes=codes[fmt], scales=scales)
        for _ in range(2):
            mx.mx_dequantize(fmt, codes[fmt], scales, K, dst=deq_out)
        avg, mn = timed(lambda: mx.mx_dequantize(fmt, codes[fmt], scales, K, dst=deq_out), 10)
        bts = n * ((0.5 if fmt == 0 else 1.0) + 1.0 / 32.0 + 2.0)
        extras.append({"kernel": f"dequantize_{'mxfp4' if fmt == 0 else 'mxfp8'}_bf16", "bytes": int(bts),
                       "avg_us": round(avg * 1e3, 2), "min_us": round(mn * 1e3, 2),
                       "GBps": round(bts / (avg * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(bts / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)})
    xt, dt_ = x.view(K, M), deq_out.view(K, M)  # the same bytes read as 57344 x 8192
    for fmt in (0, 1):
        mx.mx_qdq(fmt, xt, dst=dt_)
        avg, mn = timed(lambda: mx.mx_qdq(fmt, xt, dst=dt_), 10)
        extras.append({"kernel": f"qdq_{'mxfp4' if fmt == 0 else 'mxfp8'}_rot0_layout{K}x{M}", "bytes": 4 * n,
                       "avg_us": round(avg * 1e3, 2), "min_us": round(mn * 1e3, 2),
                       "GBps": round(4 * n / (avg * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(4 * n / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)})
    del deq_out
    # fp32 sources (fp32 in, fp32 out: 8 bytes per element): QDQ without
    # rotation, with rotation 16, and with rotation 128, whose contraction is
    # bound by the fp32 matrix cores (256 flops per element against their
    # 157.3 TFLOP/s)
    xf = x.float()
    df = torch.empty_like(xf)
    Rf = {r: torch.from_numpy(W.hadamard_rotation(r, "f32")).to(dev) for r in (16, 128)}
    for fmt, r in ((0, 0), (1, 0), (0, 16), (0, 128)):
        R = Rf[r] if r else None
        mx.mx_qdq(fmt, xf, rot=R, dst=df)
        avg, mn = timed(lambda: mx.mx_qdq(fmt, xf, rot=R, dst=df), 10)
        e = {"kernel": f"qdq_{'mxfp4' if fmt == 0 else 'mxfp8'}_f32_rot{r}", "bytes": 8 * n,
             "avg_us": round(avg * 1e3, 2), "min_us": round(mn * 1e3, 2),
             "GBps": round(8 * n / (avg * 1e-3) / 1e9, 1),
             "frac_of_peak": round(8 * n / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)}
        if r == 128:
            e.update({"flops": 2 * r * n, "TFLOPs": round(2 * r * n / (avg * 1e-3) / 1e12, 1),
                      "peak_TFLOPs": 157.3,
                      "frac_of_mfma_peak": round(2 * r * n / (avg * 1e-3) / 1e12 / 157.3, 4)})
        extras.append(e)
    del xf, df
    # the rotation alone (bf16 in, fp32 out: 2 + 4 bytes per element)
    yf = torch.empty((M, K), dtype=torch.float32, device=dev)
    for r in (16, 128):
        mx.mx_rotate(x, rots[r][1], dst=yf)
        avg, mn = timed(lambda: mx.mx_rotate(x, rots[r][1], dst=yf), 10)
        extras.append({"kernel": f"rotate_bf16_rot{r}", "bytes": 6 * n, "avg_us": round(avg * 1e3, 2),
                       "min_us": round(mn * 1e3, 2), "GBps": round(6 * n / (avg * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(6 * n / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)})
    del yf
    # NVFP4 (16-groups, E4M3 scales, per-tensor multiplier 448*6/amax) on the
    # same layer: QDQ and quantize, without rotation and with rotation 128
    gsc = (448.0 * 6.0 / x.abs().max().float()).reshape(1).contiguous()
    nv_scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    for op, r in (("qdq", 0), ("qdq", 128), ("quantize", 0), ("quantize", 128)):
        R = rots[r][1] if r else None
        if op == "qdq":
            fn = (lambda R=R: mx.mx_nvfp4_qdq(x, gsc, rot=R, dst=dst))
            bts = 4.0 * n
        else:
            fn = (lambda R=R: mx.mx_nvfp4_quantize(x, gsc, rot=R, codes=codes[0], scales=nv_scales))
            bts = n * (2.0 + 0.5 + 1.0 / 16.0)
        fn()
        avg, mn = timed(fn, 10)
        extras.append({"kernel": f"nvfp4_{op}_rot{r}", "bytes": int(bts), "avg_us": round(avg * 1e3, 2),
                       "min_us": round(mn * 1e3, 2), "GBps": round(bts / (avg * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(bts / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)})
    del nv_scales
    # blocked scale layout: the step's quantize with blocked scales, and the
    # re-blocking of row-major scales
    blk = torch.empty(mx.mx_blocked_scales_bytes(M, K), dtype=torch.uint8, device=dev)
    for fmt, r in ((0, 0), (0, 128), (1, 0)):
        R = rots[r][1] if r else None
        mx.mx_quantize_blocked(fmt, x, rot=R, codes=codes[fmt], blocked=blk)
        avg, mn = timed(lambda: mx.mx_quantize_blocked(fmt, x, rot=R, codes=codes[fmt], blocked=blk), 10)
        bts = n * (2.0 + (0.5 if fmt == 0 else 1.0)) + blk.numel()
        extras.append({"kernel": f"quantize_blocked_{'mxfp4' if fmt == 0 else 'mxfp8'}_rot{r}", "bytes": int(bts),
                       "avg_us": round(avg * 1e3, 2), "min_us": round(mn * 1e3, 2),
                       "GBps": round(bts / (avg * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(bts / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)})
    mx.mx_quantize(0, x, codes=codes[0], scales=scales)
    avg, mn = timed_graph(lambda: mx.mx_scales_to_blocked(scales, K, blocked=blk), 50)
    bts = scales.numel() + blk.numel()
    extras.append({"kernel": "scales_to_blocked", "bytes": int(bts), "avg_us": round(avg * 1e3, 2),
                   "min_us": round(mn * 1e3, 2), "GBps": round(bts / (avg * 1e-3) / 1e9, 1),
                   "frac_of_peak": round(bts / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4)})
    del blk
    # GEMM consumer: the layer's bytes read as two [8192 x 28672] operands
    # (activations and weights of a down projection), quantized, then
    # C[8192 x 8192] (bf16) = A_dq . B_dq^T on the scaled matrix cores, with
    # row-major and with blocked scales
    gm, gk = 8192, n // (2 * 8192)
    gx = x.view(2 * gm, gk)
    gc = torch.empty((gm, gm), dtype=torch.bfloat16, device=dev)
    for fmt in (0, 1):
        cq, sq = mx.mx_quantize(fmt, gx)
        a, b_, sa, sb = cq[:gm], cq[gm:], sq[:gm], sq[gm:]
        ba, bb = mx.mx_scales_to_blocked(sa, gk), mx.mx_scales_to_blocked(sb, gk)
        for layout, (xa, xb) in ((mx.ROWMAJOR, (sa, sb)), (mx.BLOCKED, (ba, bb))):
            for _ in range(2):
                mx.mx_matmul(fmt, a, xa, b_, xb, gk, c=gc, scale_layout=layout)
            avg, mn = timed(lambda: mx.mx_matmul(fmt, a, xa, b_, xb, gk, c=gc, scale_layout=layout), 10)
            tflops = 2.0 * gm * gm * gk / (avg * 1e-3) / 1e12
            extras.append({"kernel": f"matmul_{'mxfp4' if fmt == 0 else 'mxfp8'}_{gm}x{gm}x{gk}_bf16out"
                                     f"{'_blocked' if layout == mx.BLOCKED else ''}",
                           "flops": 2 * gm * gm * gk, "avg_us": round(avg * 1e3, 2), "min_us": round(mn * 1e3, 2),
                           "TFLOPs": round(tflops, 1), "bound": "mfma", "peak_TFLOPs": GEMM_PEAK_TFLOPS[fmt],
                           "frac_of_peak": round(tflops / GEMM_PEAK_TFLOPS[fmt], 4)})
        del cq, sq, a, b_, sa, sb, ba, bb
    del gc

    # measured ceilings on the layer's bytes
    progress("ceilings")
    ceilings = measure_ceilings(CL, x, copy_dst)
    copy_gbps = ceilings["copy"]["GBps"]
    for e in extras:
        if "GBps" in e:
            e["frac_of_copy"] = round(e["GBps"] / copy_gbps, 4)

    per = []
    step_bytes = 0.0
    for i, (op, fmt, r) in enumerate(var):
        ms = [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
        avg = float(np.mean(ms))
        b = n * bytes_per_element(op, fmt)
        step_bytes += b
        per.append({"kernel": name_of(op, fmt, r), "bytes": int(b), "avg_us": round(avg * 1e3, 2),
                    "median_us": round(float(np.median(ms)) * 1e3, 2), "min_us": round(min(ms) * 1e3, 2), "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_GBPS, 4),
                    "frac_of_copy": round(b / (avg * 1e-3) / 1e9 / copy_gbps, 4),
                    "elements_per_s": round(n / (avg * 1e-3), 1)})
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    dom = max(per, key=lambda p: p["avg_us"])
    achieved = dom["bytes"] / (dom["avg_us"] * 1e-6) / 1e9
    by = {p["kernel"]: p for p in per}
    ratio = {f"rot128_over_rot0_{f}": round(by[f"qdq_{f}_rot128"]["avg_us"] / by[f"qdq_{f}_rot0"]["avg_us"], 3)
             for f in ("mxfp4", "mxfp8")}
    ratio.update({f"quantize_rot128_over_rot0_{f}": round(
        by[f"quantize_{f}_rot128"]["avg_us"] / by[f"quantize_{f}_rot0"]["avg_us"], 3) for f in ("mxfp4", "mxfp8")})

    # the other workloads, on their own inputs (the step's buffers freed first)
    del x, dst, codes, scales, copy_dst
    torch.cuda.empty_cache()
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        if CL.ceil_write(flush_buf.data_ptr(), flush_buf.numel(), 0, 256, 1, _stream_ptr()) != 0:
            raise RuntimeError("flush write failed")

    config_rows, config_ratios = time_configs(mx, W, flush, copy_gbps)
    ratio.update(config_ratios)
    del flush_buf

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "8192x57344 bf16 layer, N(0,0.02^2) with subnormal-range and saturating "
                               "groups: MXFP4+MXFP8 QDQ (rotation none/16/64/128) and quantize "
                               "(rotation none/128)",
                   "M": M, "K": K, "launches_per_step": len(var), "bytes_per_step": int(step_bytes),
                   "copy_ceiling_GBps": round(copy_gbps, 1),
                   "value_frac_of_peak": round(value / PEAK_GBPS, 4)},
        "roofline": {"bound": "hbm", "kernel": dom["kernel"], "achieved": round(achieved, 1),
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": load_traffic(dom["kernel"])},
        "variants": per,
        "ratios": ratio,
        "ceilings": ceilings,
        "configs": config_rows,
        "outside_step": extras,
    }
    if not args.no_cpu:
        progress("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(x_bits, rots, args.cpu_rows, args.cpu_rows_1t)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
