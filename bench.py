#!/usr/bin/env python3
"""Benchmark of the dynamic quantized inner product on one MI355X.

One step = one dqip_forward of the 4096^3 workload (bf16 A with 1% x20
outliers quantized per row, constant int8 B, fp32 epilogue with ReLU, bf16
C): the row-quantization kernel and the int8-MFMA GEMM with its fused
dequantizing epilogue. `value` is 2*M*N*K / (wall time per step), inputs
resident in HBM, K steps back to back between two device synchronizations.

The same JSON line carries:
  roofline     -- the GEMM kernel's achieved int8 TOP/s (HIP events recorded
                  by the library around that kernel on the forward's stream)
                  against the 5.0 POP/s dense int8 MFMA peak;
  secondary    -- QuantizeLinear / DequantizeLinear on [64,256,56,56]
                  (GB/s, cold and warm cache), and the other inner-product
                  workloads (64x64x128 latency, the LSTM gate projections,
                  8192^3 with a B quantized on every call), the quantized
                  matrix products, the element-wise quantized operators
                  (GB/s against the 8 TB/s HBM peak), the general
                  QLinearConv layers and DynamicQuantizeLSTM over the
                  gate-projection workload (one call = the whole sequence);
  cpu_baseline -- the CPU oracle on a bounded sample of rows of the same
                  4096^3 workload, single-threaded.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, TOP/s
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, GB/s
FLUSH_BYTES = 512 << 20   # larger than the 256 MiB Infinity Cache


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_tensor(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


class Dqip:
    """One initialized context with its device inputs (bench-side helper)."""

    DT = {"f32": 0, "bf16": 1, "i8": 2, "u8": 3}
    ACT = {"identity": 0, "relu": 1, "leaky_relu": 2}

    def __init__(self, dq, torch, case):
        self.dq, self.case = dq, case
        M, N, K = case["M"], case["N"], case["K"]
        self.h = dq.dqip_init(M, N, K, self.DT[case["typeA"]], self.DT[case["typeB"]],
                              self.DT[case["typeC"]], case["constB"], case["bias"] is not None,
                              self.ACT[case["act"]], case["avoid"])
        self.A = dev_tensor(case["A"], torch)
        B = dev_tensor(case["B"], torch)
        sB = None if case.get("scaleB") is None else dev_tensor(case["scaleB"], torch)
        bias = None if case["bias"] is None else dev_tensor(case["bias"], torch)
        if case["constB"]:
            dq.dqip_set_params(self.h, B, sB, bias, None)
            self.B = None
            del B
        else:
            dq.dqip_set_params(self.h, None, None, bias, None)
            self.B = B
        cdt = torch.float32 if case["typeC"] == "f32" else torch.int16
        self.C = torch.empty((M, N), dtype=cdt, device="cuda")
        self.buf = torch.empty(dq.dqip_external_buffer_size(self.h), dtype=torch.uint8,
                               device="cuda")
        self.ops = 2.0 * M * N * K

    def forward(self):
        self.dq.dqip_forward(self.h, self.A, self.B, self.buf, self.C)

    def timed(self, torch, steps, warmup):
        """Back-to-back forwards: (wall ms per step, per-phase ms per call).
        The wall time comes from a pass without timing events; the per-phase
        kernel times from a second pass in which the library records HIP
        events around each phase on the forward's stream."""
        for _ in range(warmup):
            self.forward()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.forward()
        te = time.perf_counter()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        self.enqueue_us = (te - t0) * 1e6 / steps
        self.dq.dqip_profile_begin(self.h, steps)
        for _ in range(steps):
            self.forward()
        torch.cuda.synchronize()
        ms, calls = self.dq.dqip_profile_end(self.h)
        return (t1 - t0) * 1e3 / steps, [m / max(calls, 1) for m in ms]

    def release(self):
        self.dq.dqip_release(self.h)




def source_digest(files):
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, "dynamic_quantized_gemm_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record(kernel):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/), kept
    only while the kernel's sources are unchanged since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(kernel)
    if not entry or entry.get("source_sha256") != source_digest(entry.get("sources", [])):
        return None
    return entry


def _counter_means(csv_path, counter, match):
    """Mean Counter_Value (KiB) per dispatch of the kernels whose name
    contains `match`, from a rocprofv3 --pmc counter_collection.csv."""
    import csv

    vals = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and match in row["Kernel_Name"]:
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for '{match}' in {csv_path}")
    return list(vals.values())


def write_counters(copy_fetch_csv, copy_write_csv, specs):
    """Adds HBM-traffic records to profiles/traffic.json from rocprofv3 --pmc
    FETCH_SIZE / WRITE_SIZE runs, each spec "label=kernel substring=fetch
    csv=write csv=algorithmic bytes per dispatch=source,source,...". The
    counters (KiB per dispatch) are scaled by what the same counters read for
    the plain 1 GiB copy (--copy-calibration)."""
    n = 1 << 30
    big = lambda v: [x for x in v if x * 1024 > n / 2]  # the 1 GiB copies only
    cf = big(_counter_means(copy_fetch_csv, "FETCH_SIZE", "copyBuffer"))
    cw = big(_counter_means(copy_write_csv, "WRITE_SIZE", "copyBuffer"))
    f_scale = n / (1024 * sum(cf) / len(cf))
    w_scale = n / (1024 * sum(cw) / len(cw))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    for spec in specs:
        label, match, fcsv, wcsv, alg, srcs = spec.split("=")
        gf = _counter_means(fcsv, "FETCH_SIZE", match)
        gw = _counter_means(wcsv, "WRITE_SIZE", match)
        fetch = 1024 * sum(gf) / len(gf) * f_scale
        write = 1024 * sum(gw) / len(gw) * w_scale
        sources = [x for x in srcs.split(",") if x]
        rec[label] = {"kernel": match, "dispatches": [len(gf), len(gw)],
                      "fetch_bytes": round(fetch), "write_bytes": round(write),
                      "bytes_per_launch": round(fetch + write), "algorithmic_bytes": int(alg),
                      "traffic_over_algorithmic": round((fetch + write) / int(alg), 3),
                      "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
                      "copy_counter_kib": [round(sum(cf) / len(cf), 1), round(sum(cw) / len(cw), 1)],
                      "sources": sources, "source_sha256": source_digest(sources)}
        print(json.dumps({label: rec[label]}))
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def summarize_pmc(csv_path, match):
    """Mean of every counter per dispatch of the kernels whose name contains
    `match`, from a rocprofv3 --pmc counter_collection.csv (printed as JSON)."""
    import csv

    per = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if match in row["Kernel_Name"]:
                key = (row["Counter_Name"], row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    print(json.dumps({k: {"mean": round(sum(v) / len(v), 1), "dispatches": len(v)} for k, v in out.items()}))


def copy_calibration(torch, mib=1024, reps=10):
    """A plain device-to-device copy of known size, for scaling the L2
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps, "read_bytes_per_copy": n,
                      "write_bytes_per_copy": n}), flush=True)


def time_cold_warm(fn, torch, steps, flush):
    """((median, p10, p90) ms per call with the caches flushed before each
    call, mean ms per call back to back); HIP events on torch's current
    stream, which is the stream the library launches on. The flush READS a
    buffer twice the Infinity Cache's size: that evicts the call's data
    without leaving dirty lines whose write-back the timed call would pay
    for."""
    for _ in range(3):
        fn()
    cold = []
    for i in range(steps):
        _ = flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    e1.synchronize()
    pct = tuple(float(np.percentile(cold, q)) for q in (50, 10, 90))
    return pct, e0.elapsed_time(e1) / steps


def _bw_record(nbytes, cold, warm_ms):
    gb = nbytes / 1e9
    cold_ms = cold[0]
    return {"us_cold": round(cold_ms * 1e3, 2), "us_cold_p10": round(cold[1] * 1e3, 2),
            "us_cold_p90": round(cold[2] * 1e3, 2), "GBps_cold": round(gb / (cold_ms / 1e3), 1),
            "frac_cold": round(gb / (cold_ms / 1e3) / HBM_PEAK_GBS, 3),
            "us_warm": round(warm_ms * 1e3, 2), "GBps_warm": round(gb / (warm_ms / 1e3), 1)}


def achievable(dq, torch, reps=5):
    """What the chip reaches on its own, as context for the roofline
    fractions (the library's measurement probes): the int8 MFMA rate of a
    loop with nothing but the GEMM wave tile's MFMAs (one workgroup of four
    waves per CU, as the 4096^3 GEMM runs), with random and with all-zero
    operands, and the HBM rate of a plain 16-byte copy of 1 GiB (2 GiB moved
    per call). Median of `reps` launches, HIP events on torch's current
    stream (the stream the probes are launched on)."""
    def med_ms(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    out = {}
    wg, iters = 256, 2000
    sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
    ops = float(wg) * 4 * iters * 32 * 65536
    g = torch.Generator(device="cpu").manual_seed(0)
    rnd = torch.randint(-128, 128, (65536,), generator=g, dtype=torch.int8).cuda()
    zero = torch.zeros(65536, dtype=torch.int8, device="cuda")
    # the GEMM's instruction (16x16x64) with random and zero operands, and
    # the 32x32x32 shape with random operands for comparison
    for key, shape, buf in (("mfma_loop_TOPS_random_operands", 16, rnd),
                            ("mfma_loop_TOPS_zero_operands", 16, zero),
                            ("mfma32_loop_TOPS_random_operands", 32, rnd)):
        ms = med_ms(lambda: dq.dq_probe_mfma_loop(buf, shape, iters, wg, sink))
        out[key] = round(ops / (ms / 1e3) / 1e12, 1)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = med_ms(lambda: dq.dq_probe_copy(src, dst, n))
    out["copy_GBps"] = round(2.0 * n / (ms / 1e3) / 1e9, 1)
    out["copy_frac_of_8TBps"] = round(2.0 * n / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 3)
    del src, dst
    out["mfma_loop_frac_of_5POPS_random"] = round(out["mfma_loop_TOPS_random_operands"] / INT8_PEAK_TOPS, 3)
    out["how"] = (f"mfma: {wg} workgroups x 4 waves, each {iters} x 64 v_mfma_i32_16x16x64_i8 (the GEMM's "
                  f"instruction; mfma32: 32 v_mfma_i32_32x32x32_i8) on register operands (two alternating "
                  f"sets); copy: 1 GiB, four 16 B non-temporal loads a lane in flight; median of {reps} launches")
    return out


def bench_qdq(dq, torch, steps):
    """QuantizeLinear and DequantizeLinear, per axis, [64,256,56,56] fp32 <->
    int8: GB/s of algorithmic bytes (4 + 1 per element), cold (Infinity
    Cache flushed before every call) and warm (back to back)."""
    import workloads as W

    case = W.qdq_per_axis(seed=1)
    x = dev_tensor(case["x"], torch)
    s = dev_tensor(case["scale"], torch)
    z = dev_tensor(case["zp"], torch)
    n = x.numel()
    y = torch.empty(x.shape, dtype=torch.int8, device="cuda")
    r = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    q = lambda: dq.qlinear_quantize(x, s, z, dq.DQ_I8, y, axis=1)  # noqa: E731
    d = lambda: dq.qlinear_dequantize(y, dq.DQ_I8, s, z, r, axis=1)  # noqa: E731
    out = {}
    for name, fn in (("quantize", q), ("dequantize", d)):
        out[name] = _bw_record(5 * n, *time_cold_warm(fn, torch, steps, flush))
    del flush
    # steady state from HBM: back-to-back calls over five buffer sets (1.3 GB
    # each way), so no call finds its data in the 256 MiB Infinity Cache.
    # Fresh device allocations are slow to use for a while (the driver
    # still initializes them in the background), so the sets are allocated
    # and touched first, and the median of three timed loops is kept.
    R = 5
    xs = [x.clone() for _ in range(R)]
    ys = [torch.empty_like(y) for _ in range(R)]
    rs = [torch.empty_like(r) for _ in range(R)]
    for t in ys + rs:
        t.zero_()
    torch.cuda.synchronize()
    time.sleep(0.2)
    calls = {"quantize": lambda i: dq.qlinear_quantize(xs[i], s, z, dq.DQ_I8, ys[i], axis=1),
             "dequantize": lambda i: dq.qlinear_dequantize(ys[i], dq.DQ_I8, s, z, rs[i], axis=1)}
    for name, call in calls.items():
        for _ in range(2):
            for i in range(R):
                call(i)
        torch.cuda.synchronize()
        reps = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps * R):
                call(i % R)
            e1.record()
            e1.synchronize()
            reps.append(e0.elapsed_time(e1) / (steps * R))
        ms = float(np.median(reps))
        out[name].update({"us_stream": round(ms * 1e3, 2),
                          "GBps_stream": round(5.0 * n / 1e9 / (ms / 1e3), 1),
                          "frac_stream": round(5.0 * n / 1e9 / (ms / 1e3) / HBM_PEAK_GBS, 3)})
    del xs, ys, rs
    out["workload"] = "x fp32 [64,256,56,56] NCHW <-> int8, per-channel (axis 1) scale/zero point"
    out["bytes_per_call"] = 5 * n
    out["timing"] = ("cold: median (p10, p90) of calls each after a 512 MiB read flush; warm: back to back on "
                     "one buffer set; stream: back to back over 5 buffer sets (1.3 GB), median of 3 "
                     "loops")
    return out


def bench_qconv(dq, torch, steps):
    """The requantizing 1x1 QLinearConv, uint8 x [8,256,56,56] (x_zp 128),
    int8 w [256,256] per-channel scales, int32 bias, uint8 y: GB/s of
    algorithmic bytes (x + w + y + parameters), cold and warm."""
    import workloads as W

    c = W.qconv1x1()
    N, C, H, Wd = c["x"].shape
    M = c["w"].shape[0]
    x = dev_tensor(c["x"], torch)
    w = dev_tensor(c["w"], torch)
    xs = dev_tensor(np.array([c["x_scale"]], np.float32), torch)
    ys = dev_tensor(np.array([c["y_scale"]], np.float32), torch)
    xz = dev_tensor(np.array([c["x_zp"]], np.uint8), torch)
    yz = dev_tensor(np.array([c["y_zp"]], np.uint8), torch)
    ws = dev_tensor(c["w_scale"], torch)
    b = dev_tensor(c["bias"], torch)
    y = torch.empty((N, M, H, Wd), dtype=torch.uint8, device="cuda")
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    fn = lambda: dq.qlinear_conv1x1(x, dq.DQ_U8, xs, xz, w, dq.DQ_I8, ws, None, ys, yz,  # noqa: E731
                                    dq.DQ_U8, b, y)
    nbytes = N * C * H * Wd + N * M * H * Wd + M * C + 8 * M + 10
    out = _bw_record(nbytes, *time_cold_warm(fn, torch, steps, flush))
    out["TOPS_cold"] = round(2.0 * N * M * C * H * Wd / (out["us_cold"] * 1e-6) / 1e12, 1)
    out["workload"] = c["name"]
    out["bytes_per_call"] = nbytes
    del flush
    return out


def bench_qgemm(dq, torch, kind, steps, flush):
    """The quantized matrix products at 4096^3 (workloads.qgemm_case): TOP/s
    of 2MNK over the whole forward (A packing or per-tensor quantization and
    the GEMM), back to back and cold."""
    import workloads as W

    c = W.qgemm_case(kind)
    M, N, K = c["M"], c["N"], c["K"]
    a_t = dq.DQ_F32 if kind == "dqmm" else dq.DQ_U8
    y_t = dq.DQ_U8 if kind == "qgemm" else dq.DQ_F32
    h = dq.dq_qgemm_init(M, N, K, a_t, False, dq.DQ_I8, False, y_t, 1.0)
    try:
        dq.dq_qgemm_set_b(h, dev_tensor(c["B"], torch), dev_tensor(c["b_scale"], torch),
                          dev_tensor(c["b_zp"].astype(np.int8), torch))
        A = dev_tensor(c["A"], torch)
        a_s = None if kind == "dqmm" else dev_tensor(np.float32([c["a_scale"]]), torch)
        a_z = None if kind == "dqmm" else dev_tensor(np.uint8([c["a_zp"]]), torch)
        Cm = dev_tensor(c["C"], torch) if "C" in c else None
        bias = dev_tensor(c["bias"], torch) if "bias" in c else None
        ys = dev_tensor(np.float32([c["y_scale"]]), torch) if kind == "qgemm" else None
        yz = dev_tensor(np.uint8([c["y_zp"]]), torch) if kind == "qgemm" else None
        Y = torch.empty((M, N), dtype=torch.uint8 if kind == "qgemm" else torch.float32,
                        device="cuda")
        fn = lambda: dq.dq_qgemm_forward(h, A, a_s, a_z, Cm, bias, ys, yz, Y)  # noqa: E731
        cold, warm = time_cold_warm(fn, torch, steps, flush)
        info = dq.dq_qgemm_info(h)
    finally:
        dq.dq_qgemm_release(h)
    ops = 2.0 * M * N * K
    return {"workload": c["name"], "us_per_forward": round(warm * 1e3, 2),
            "TOPS": round(ops / (warm / 1e3) / 1e12, 1),
            "us_cold": round(cold[0] * 1e3, 2), "us_cold_p10": round(cold[1] * 1e3, 2),
            "us_cold_p90": round(cold[2] * 1e3, 2), "info": info}


def bench_elementwise(dq, torch, steps, flush):
    """The element-wise quantized operators (workloads.elementwise_case): GB/s
    of algorithmic bytes (each input and output byte once), cold (median,
    p10, p90 after a read flush; the flush's run time hides the host's
    enqueue, so this is the kernel's time) and back to back. Calls go
    straight to the C ABI with their arguments marshalled once."""
    import ctypes as C

    import workloads as W

    lib = dq.load()
    st = torch.cuda.current_stream().cuda_stream
    out = {}

    def ck(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: {rc} {lib.dqip_last_error()}")

    def i64(vals):
        return (C.c_int64 * max(1, len(vals)))(*[int(v) for v in vals])

    for kind in W.ELEMENTWISE:
        c = W.elementwise_case(kind)
        t = dq.DQ_U8 if c["type"] == "u8" else dq.DQ_I8
        tdt = torch.uint8 if c["type"] == "u8" else torch.int8
        zdt = np.uint8 if c["type"] == "u8" else np.int8
        xs = [dev_tensor(x, torch) for x in c["xs"]]
        sc = [dev_tensor(np.array([v], np.float32), torch) for v in c["scales"]]
        zp = [dev_tensor(np.array([v], zdt), torch) for v in c["zps"]]
        P = lambda tt: tt.data_ptr()  # noqa: E731
        keep = []
        if kind in ("add", "add_rowvec", "mul", "mul_integer"):
            A, B = xs
            shape = np.broadcast_shapes(tuple(A.shape), tuple(B.shape))
            sa, sb = i64(A.shape), i64(B.shape)
            keep += [sa, sb]
            if kind == "mul_integer":
                Y = torch.empty(shape, dtype=torch.int32, device="cuda")
                args = (P(A), A.dim(), sa, P(zp[0]), P(B), B.dim(), sb, P(zp[1]), t, P(Y), st)
                call = lib.dq_mul_integer
                nbytes = A.numel() + B.numel() + 4 * Y.numel()
            else:
                Y = torch.empty(shape, dtype=tdt, device="cuda")
                args = (P(A), A.dim(), sa, P(sc[0]), P(zp[0]), P(B), B.dim(), sb, P(sc[1]), P(zp[1]),
                        P(sc[2]), P(zp[2]), t, P(Y), st)
                call = lib.qlinear_mul if kind == "mul" else lib.qlinear_add
                nbytes = A.numel() + B.numel() + Y.numel()
            desc = f"{c['type']} {tuple(A.shape)} with {tuple(B.shape)}"
        elif kind in ("sigmoid", "leaky_relu"):
            X = xs[0]
            Y = torch.empty_like(X)
            if kind == "sigmoid":
                call = lib.qlinear_sigmoid
                args = (P(X), X.numel(), P(sc[0]), P(zp[0]), P(sc[1]), P(zp[1]), t, P(Y), st)
            else:
                call = lib.qlinear_leaky_relu
                args = (P(X), X.numel(), P(sc[0]), P(zp[0]), P(sc[1]), P(zp[1]), float(c["alpha"]), t,
                        P(Y), st)
            nbytes = 2 * X.numel()
            desc = f"{c['type']} {X.numel()} codes"
        elif kind.startswith(("sum_", "mean_")):
            X = xs[0]
            axes = (C.c_int32 * len(c["axes"]))(*c["axes"])
            shp = i64(X.shape)
            keep += [axes, shp]
            nout = X.numel()
            for a in c["axes"]:
                nout //= X.shape[a]
            if kind.startswith("sum_"):
                Y = torch.empty(nout, dtype=torch.int32, device="cuda")
                call = lib.dq_reduce_sum_integer
                args = (P(X), t, X.dim(), shp, axes, len(c["axes"]), P(Y), st)
                nbytes = X.numel() + 4 * nout
            else:
                Y = torch.empty(nout, dtype=tdt, device="cuda")
                call = lib.qlinear_reduce_mean
                args = (P(X), t, X.dim(), shp, axes, len(c["axes"]), P(sc[0]), P(zp[0]), P(sc[1]),
                        P(zp[1]), P(Y), st)
                nbytes = X.numel() + nout
            desc = f"{c['type']} {tuple(X.shape)} over axes {c['axes']}"
        else:  # concat
            ax = c["axis"]
            shape = list(xs[0].shape)
            shape[ax] = sum(int(x.shape[ax]) for x in xs)
            Y = torch.empty(shape, dtype=tdt, device="cuda")
            n = len(xs)
            xa = (C.c_void_p * n)(*[P(x) for x in xs])
            sha = i64([v for x in xs for v in x.shape])
            sca = (C.c_void_p * n)(*[P(v) for v in sc[:n]])
            zpa = (C.c_void_p * n)(*[P(v) for v in zp[:n]])
            keep += [xa, sha, sca, zpa]
            call = lib.qlinear_concat
            args = (n, C.cast(xa, C.c_void_p), C.cast(sha, C.c_void_p), xs[0].dim(), ax,
                    C.cast(sca, C.c_void_p), C.cast(zpa, C.c_void_p), P(sc[n]), P(zp[n]), t, P(Y), st)
            nbytes = 2 * Y.numel()
            desc = f"{c['type']} {n} x {tuple(xs[0].shape)} along axis {ax}"
        fn = lambda call=call, args=args, kind=kind: ck(call(*args), kind)  # noqa: E731
        rec = _bw_record(nbytes, *time_cold_warm(fn, torch, steps, flush))
        rec["workload"] = desc
        rec["bytes_per_call"] = int(nbytes)
        out[kind] = rec
        log(f"bench: elementwise {kind}: {rec}")
        del xs, sc, zp, Y, keep
    out["timing"] = ("cold: median (p10, p90) of calls each after a 512 MiB read flush; warm: back to "
                     "back on one buffer set (host-bound below ~15 us)")
    return out


def bench_qconv_general(dq, torch, steps, flush):
    """The general 2-D QLinearConv (implicit GEMM) on ResNet-shaped layers at
    a batch of 8: uint8 x (zero point 128), int8 w per-channel scales, int32
    bias, uint8 y. TOP/s of 2 N M oH oW (C / group) kH kW, cold and back to
    back; a depthwise layer runs the direct kernel (GB/s there)."""
    import workloads as W

    out = {}
    for name, (N, C, H, Wd, M, k, st, pad, grp) in W.QCONV_LAYERS.items():
        c = W.qconv_layer_case(name)
        ctx = dq.dq_qconv_init(C, H, Wd, M, k, k, dq.DQ_U8, dq.DQ_I8, dq.DQ_U8, strides=(st, st),
                               pads=(pad, pad, pad, pad), group=grp)
        try:
            oh, ow = dq.dq_qconv_output_shape(ctx)
            dq.dq_qconv_set_w(ctx, dev_tensor(c["w"], torch), dev_tensor(c["w_scale"], torch), None,
                              dev_tensor(c["bias"], torch))
            x = dev_tensor(c["x"], torch)
            y = torch.empty((N, M, oh, ow), dtype=torch.uint8, device="cuda")
            xs = dev_tensor(np.array([c["x_scale"]], np.float32), torch)
            ys = dev_tensor(np.array([c["y_scale"]], np.float32), torch)
            z = dev_tensor(np.array([128], np.uint8), torch)
            fn = lambda: dq.dq_qconv_forward(ctx, x, xs, z, ys, z, y)  # noqa: E731
            cold, warm = time_cold_warm(fn, torch, steps, flush)
            ops = 2.0 * N * M * oh * ow * (C // grp) * k * k
            nbytes = x.numel() + y.numel() + c["w"].size
            out[name] = {"us_cold": round(cold[0] * 1e3, 2), "us_cold_p10": round(cold[1] * 1e3, 2),
                         "us_cold_p90": round(cold[2] * 1e3, 2), "us_warm": round(warm * 1e3, 2),
                         "TOPS_cold": round(ops / (cold[0] / 1e3) / 1e12, 1),
                         "TOPS_warm": round(ops / (warm / 1e3) / 1e12, 1),
                         "GBps_cold": round(nbytes / (cold[0] / 1e3) / 1e9, 1),
                         "kernel": dq.dq_qconv_info(ctx)}
            log(f"bench: qconv {name}: {out[name]}")
        finally:
            dq.dq_qconv_release(ctx)
    return out


def bench_lstm(dq, torch, steps, flush):
    """DynamicQuantizeLSTM on the gate-projection workload (seq 128, batch 32,
    input 512, hidden 512, per-column int8 W and R), forward and
    bidirectional: one forward call runs the whole sequence (the input
    projection and 128 steps). us per sequence cold and back to back, tokens
    (seq x batch) per second, and the TOP/s of the two products,
    2 seq batch (input + hidden) 4 hidden per direction."""
    import workloads as W

    out = {}
    for direction in ("forward", "bidirectional"):
        c = W.lstm_case(direction=direction)
        seq, batch, nin = c["X"].shape
        h = c["hidden"]
        dirs = 2 if direction == "bidirectional" else 1
        ctx = dq.dq_lstm_init(seq, batch, nin, h, direction, dq.DQ_I8, dq.DQ_I8)
        try:
            t = lambda a: None if a is None else dev_tensor(a, torch)  # noqa: E731
            dq.dq_lstm_set_weights(ctx, t(c["W"]), t(c["W_scale"]), t(c["W_zp"]), t(c["R"]),
                                   t(c["R_scale"]), t(c["R_zp"]), t(c["B"]), t(c["P"]))
            X, h0, c0 = t(c["X"]), t(c["initial_h"]), t(c["initial_c"])
            Y = torch.empty((seq, dirs, batch, h), device="cuda")
            Yh = torch.empty((dirs, batch, h), device="cuda")
            Yc = torch.empty((dirs, batch, h), device="cuda")
            fn = lambda: dq.dq_lstm_forward(ctx, X, None, h0, c0, Y, Yh, Yc)  # noqa: E731
            cold, warm = time_cold_warm(fn, torch, steps, flush)
            ops = 2.0 * seq * batch * (nin + h) * 4 * h * dirs
            out[direction] = {"us_cold": round(cold[0] * 1e3, 1), "us_cold_p10": round(cold[1] * 1e3, 1),
                              "us_cold_p90": round(cold[2] * 1e3, 1), "us_warm": round(warm * 1e3, 1),
                              "us_per_step_warm": round(warm * 1e3 / seq, 2),
                              "tokens_per_s_warm": round(seq * batch / (warm / 1e3)),
                              "TOPS_warm": round(ops / (warm / 1e3) / 1e12, 2),
                              "kernel": dq.dq_lstm_info(ctx)}
            log(f"bench: lstm {direction}: {out[direction]}")
        finally:
            dq.dq_lstm_release(ctx)
    return out


def bench_dqip_case(dq, torch, case, steps, warmup, flush):
    """Back-to-back forwards (warm: a recurrence keeps its weights cache-
    resident), their per-phase kernel times, and single forwards after a
    cache flush (cold: median, p10, p90)."""
    d = Dqip(dq, torch, case)
    try:
        ms, ph = d.timed(torch, steps, warmup)
        cold, _ = time_cold_warm(d.forward, torch, steps, flush)
    finally:
        d.release()
    return {"workload": case["name"], "us_per_forward": round(ms * 1e3, 2),
            "us_cold": round(cold[0] * 1e3, 2), "us_cold_p10": round(cold[1] * 1e3, 2),
            "us_cold_p90": round(cold[2] * 1e3, 2),
            "TOPS": round(d.ops / (ms / 1e3) / 1e12, 2),
            "phase_us": {"quant_a": round(ph[0] * 1e3, 2), "quant_b": round(ph[1] * 1e3, 2),
                         "gemm": round(ph[2] * 1e3, 2)},
            "gemm_TOPS": round(d.ops / (ph[2] / 1e3) / 1e12, 2) if ph[2] > 0 else None}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _cpu_threads():
    """Threads for the all-core oracle leg: the host's CPUs this process may
    use, capped by OMP_NUM_THREADS (the share a GPU job is given)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else n


def _oracle_rows(case, rows, threads):
    """The oracle (unchanged, single-threaded C) over `rows`, split into
    `threads` contiguous slices run at once from a thread pool (each call
    releases the interpreter lock while in C; output rows are independent,
    so the results are the same as one call's)."""
    import concurrent.futures as cf

    import oracle

    if threads == 1:
        oracle.dqip_forward(case, rows=rows)
        return
    parts = [p for p in np.array_split(rows, threads) if p.size]
    with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(lambda p: oracle.dqip_forward(case, rows=p), parts))


def cpu_baseline(case, budget_s=12.0, others=True):
    """The oracle as it is (plain C, one output row after another) timed on
    this host's cores on a bounded sample of rows of the same workload,
    scaled to TOP/s of the whole inner product: once on one thread, once
    with the rows split over every available thread. With `others`, the
    oracle's single-thread time for the other configurations too (bounded
    samples, each stated)."""
    import oracle
    import workloads as W

    N, K = case["N"], case["K"]
    t0 = time.perf_counter()
    oracle.dqip_forward(case, rows=np.arange(2))
    t_probe = (time.perf_counter() - t0) / 2
    rows1 = int(max(2, min(512, budget_s / 2 / max(t_probe, 1e-4))))
    t0 = time.perf_counter()
    _oracle_rows(case, np.arange(rows1), 1)
    dt1 = time.perf_counter() - t0
    threads = _cpu_threads()
    rowsN = int(min(case["M"], rows1 * threads))
    t0 = time.perf_counter()
    _oracle_rows(case, np.arange(rowsN), threads)
    dtN = time.perf_counter() - t0
    v1 = 2.0 * rows1 * N * K / dt1 / 1e12
    vN = 2.0 * rowsN * N * K / dtN / 1e12
    rec = {"value": round(vN, 6), "unit": "TOP/s", "cores": threads, "kind": "oracle",
           "sample": (f"{rowsN} of {case['M']} rows of the same 4096^3 workload split over {threads} "
                      f"threads ({dtN:.1f} s); single thread: {rows1} rows in {dt1:.1f} s. Each call: "
                      f"row quantization of its rows, the whole B's column sums, the rows' integer "
                      f"sums and epilogue"),
           "value_1_thread": round(v1, 6), "cpu_model": _cpu_model(), "nproc": os.cpu_count()}
    if not others:
        return rec
    extra = {}
    # c1: the whole 64x64x128 forward, median of 3
    c1 = W.dqip_small()
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.dqip_forward(c1)
        ts.append(time.perf_counter() - t0)
    extra["dqip_64x64x128"] = {"us_per_forward": round(float(np.median(ts)) * 1e6, 1)}
    # c2: QuantizeLinear + DequantizeLinear over the whole [64,256,56,56] tensor
    q = W.qdq_per_axis(seed=1)
    t0 = time.perf_counter()
    yq = oracle.quantize_linear(q["x"], q["scale"], q["zp"], axis=1)
    tq = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.dequantize_linear(yq, q["scale"], q["zp"], axis=1)
    td = time.perf_counter() - t0
    nb = 5 * q["x"].size
    extra["qdq_64x256x56x56"] = {"quantize_GBps": round(nb / tq / 1e9, 3),
                                 "dequantize_GBps": round(nb / td / 1e9, 3)}
    # c4: the input projection on 256 of its 4096 rows, the recurrent step whole
    c4 = W.dqip_lstm(recurrent=False)
    t0 = time.perf_counter()
    oracle.dqip_forward(c4, rows=np.arange(256))
    t4 = time.perf_counter() - t0
    c4r = W.dqip_lstm(recurrent=True)
    t0 = time.perf_counter()
    oracle.dqip_forward(c4r)
    t4r = time.perf_counter() - t0
    extra["lstm_input_4096x2048x512"] = {"TOPS": round(2.0 * 256 * c4["N"] * c4["K"] / t4 / 1e12, 6),
                                         "sample": "256 of 4096 rows"}
    extra["lstm_recurrent_32x2048x512"] = {"us_per_forward": round(t4r * 1e6, 1)}
    # c5b: the 1x1 QLinearConv on one of the eight images
    c = W.qconv1x1()
    x1 = np.ascontiguousarray(c["x"][:1])
    C_, HW = x1.shape[1], x1.shape[2] * x1.shape[3]
    t0 = time.perf_counter()
    oracle.qlinear_conv(x1.reshape(1, C_, HW, 1), c["x_scale"], int(c["x_zp"]), c["w"].reshape(-1, C_),
                        c["w_scale"], np.zeros(c["w"].shape[0], np.int32), c["y_scale"], int(c["y_zp"]),
                        bias=c["bias"], y_type="u8")
    t5 = time.perf_counter() - t0
    nb5 = (2 * C_ * HW + c["w"].size) * 8  # whole-batch bytes, time scaled from one image
    extra["qlinearconv_1x1"] = {"GBps": round(nb5 / (8 * t5) / 1e9, 3), "sample": "image 0 of 8"}
    rec["other_configs_1_thread"] = extra
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline only: no secondary configs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", metavar="PATH", help="also write every secondary record in full to PATH")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scales the HBM traffic counters)")
    ap.add_argument("--only", choices=["headline", "qdq", "qconv1x1", "lstm_input", "lstm_recurrent",
                                       "dqip_8192", "mitf", "dqmm", "qgemm", "elementwise", "qconv_general",
                                       "lstm", "probes"],
                    help="run one workload only (for profiler runs); prints a short record, not the line")
    ap.add_argument("--write-counters", nargs="+", metavar="ARG",
                    help="no GPU: COPY_FETCH_CSV COPY_WRITE_CSV then specs "
                         "label=kernel=fetch_csv=write_csv=algorithmic_bytes=sources")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("CSV", "KERNEL_SUBSTRING"),
                    help="no GPU: mean of each counter per dispatch of the matching kernels")
    args = ap.parse_args()
    if args.write_counters:
        write_counters(args.write_counters[0], args.write_counters[1], args.write_counters[2:])
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path, so --gpus "
              f"{args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_quantized_gemm_amd as dq
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    dq.load()
    if args.only:
        run_only(args.only, dq, torch, W, args.steps)
        return

    log("bench: generating the 4096^3 workload")
    case = W.dqip_large()
    d = Dqip(dq, torch, case)
    info = dq.dqip_info(d.h)
    log(f"bench: {info}")
    ms, phases = d.timed(torch, args.steps, args.warmup)
    d.release()
    value = d.ops / (ms / 1e3) / 1e12
    gemm_ms = phases[2]
    achieved = d.ops / (gemm_ms / 1e3) / 1e12
    log(f"bench: {ms * 1e3:.1f} us/forward = {value:.1f} TOPS; gemm {gemm_ms * 1e3:.1f} us = "
        f"{achieved:.1f} TOPS; quant_a {phases[0] * 1e3:.1f} us; host enqueue {d.enqueue_us:.1f} us/forward")
    tr = traffic_record("gemm_i8")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                "traffic": None if tr is None else tr["bytes_per_launch"],
                "kernel": "gemm_i8 (int8 MFMA, fused dequant/bias/ReLU/bf16 epilogue)",
                "scope": ("the GEMM kernel alone (its own launch duration); `value` is the whole "
                          "forward, row quantization included"),
                "avg_launch_us": round(gemm_ms * 1e3, 2),
                "ops_per_launch": d.ops}
    log("bench: achievable rates (MFMA-only loop, plain copy)")
    ach = achievable(dq, torch)
    log(f"bench: {ach}")

    secondary = {"dqip_4096_phases_us": {"quant_a": round(phases[0] * 1e3, 2),
                                         "gemm": round(gemm_ms * 1e3, 2),
                                         "host_enqueue": round(d.enqueue_us, 2)},
                 "quant_a_GBps": (round((case["M"] * case["K"] * 3) / (phases[0] / 1e3) / 1e9, 1)
                                  if phases[0] > 0 else None)}
    if not args.quick:
        steps2 = max(10, args.steps // 2)
        log("bench: QuantizeLinear / DequantizeLinear [64,256,56,56]")
        secondary["qdq"] = bench_qdq(dq, torch, steps2)
        log(f"bench: {secondary['qdq']}")
        log("bench: QLinearConv 1x1 [8,256,56,56]")
        secondary["qlinearconv_1x1"] = bench_qconv(dq, torch, steps2)
        log(f"bench: {secondary['qlinearconv_1x1']}")
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        for name, mk in (("dqip_64x64x128", W.dqip_small),
                         ("lstm_input_4096x2048x512", lambda: W.dqip_lstm(recurrent=False)),
                         ("lstm_recurrent_32x2048x512", lambda: W.dqip_lstm(recurrent=True)),
                         ("dqip_8192_dynamic_b", W.dqip_dynamic_b)):
            log(f"bench: {name}")
            secondary[name] = bench_dqip_case(dq, torch, mk(), steps2, 3, flush)
            log(f"bench: {secondary[name]}")
        for kind, name in (("mitf", "matmul_integer_to_float_4096"),
                           ("dqmm", "dynamic_quantize_matmul_4096"),
                           ("qgemm", "qgemm_u8_4096")):
            log(f"bench: {name}")
            secondary[name] = bench_qgemm(dq, torch, kind, steps2, flush)
            log(f"bench: {secondary[name]}")
        log("bench: element-wise quantized operators")
        secondary["elementwise"] = bench_elementwise(dq, torch, steps2, flush)
        log("bench: general QLinearConv")
        secondary["qlinearconv_general"] = bench_qconv_general(dq, torch, steps2, flush)
        log("bench: DynamicQuantizeLSTM")
        secondary["dynamic_quantize_lstm"] = bench_lstm(dq, torch, steps2, flush)
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(case, others=not args.quick)
        log(f"bench: {cpu}")

    # the metric's second half and the context of the first, also inside
    # `roofline` (a record every reader of the line keeps whole)
    roofline["achievable"] = {k: v for k, v in ach.items() if k != "how"}
    roofline["achievable"]["gemm_frac_of_mfma_loop_random"] = round(
        roofline["achieved"] / ach["mfma_loop_TOPS_random_operands"], 3)
    qdq = None
    if "qdq" in secondary:
        qq, dd = secondary["qdq"]["quantize"], secondary["qdq"]["dequantize"]
        qdq = {"workload": "QuantizeLinear / DequantizeLinear per channel (axis 1), x fp32 [64,256,56,56] <-> "
                           "int8, 256.9 MB moved per call",
               "quantize_GBps_cold": qq["GBps_cold"], "quantize_frac_cold": qq["frac_cold"],
               "dequantize_GBps_cold": dd["GBps_cold"], "dequantize_frac_cold": dd["frac_cold"],
               "quantize_us_cold": qq["us_cold"], "dequantize_us_cold": dd["us_cold"],
               "quantize_GBps_stream": qq.get("GBps_stream"), "dequantize_GBps_stream": dd.get("GBps_stream"),
               "peak_GBps": HBM_PEAK_GBS}
        roofline["qdq"] = {"bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                           "quantize": {"achieved": qq["GBps_cold"], "frac": qq["frac_cold"],
                                        "us": qq["us_cold"]},
                           "dequantize": {"achieved": dd["GBps_cold"], "frac": dd["frac_cold"],
                                          "us": dd["us_cold"]},
                           "timing": "cold: after a 512 MiB read flush; 256.9 MB a call"}
    line = {
        "metric": "dyn-quant GEMM TOPS (% int8 MFMA peak) + Quantize/DequantizeLinear GB/s",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "dynamic quantized inner product M=N=K=4096: bf16 A ~N(0,1) with "
                               "1% x20 outliers, constant int8 B with per-column scales, fp32 "
                               "bias, ReLU, bf16 C",
                   "M": 4096, "N": 4096, "K": 4096, "pct_int8_peak": round(100 * value / INT8_PEAK_TOPS, 2)},
        "qdq": qdq,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": {k: compact(v) for k, v in secondary.items()},
        "info": info,
    }
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"secondary": secondary, "cpu_baseline": cpu, "achievable": ach}, f, indent=1)
    print(json.dumps(line), flush=True)


def run_only(which, dq, torch, W, steps):
    """One workload alone, `steps` calls after three warm-up calls (profiler
    runs: every dispatch of the run is that workload's)."""
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    if which == "headline":
        d = Dqip(dq, torch, W.dqip_large())
        ms, ph = d.timed(torch, steps, 3)
        d.release()
        rec = {"us_per_forward": round(ms * 1e3, 2), "phase_us": [round(x * 1e3, 2) for x in ph]}
    elif which == "qdq":
        rec = bench_qdq(dq, torch, steps)
    elif which == "qconv1x1":
        rec = bench_qconv(dq, torch, steps)
    elif which in ("lstm_input", "lstm_recurrent"):
        rec = bench_dqip_case(dq, torch, W.dqip_lstm(recurrent=which == "lstm_recurrent"), steps, 3, flush)
    elif which == "dqip_8192":
        rec = bench_dqip_case(dq, torch, W.dqip_dynamic_b(), steps, 3, flush)
    elif which in ("mitf", "dqmm", "qgemm"):
        rec = bench_qgemm(dq, torch, which, steps, flush)
    elif which == "elementwise":
        rec = bench_elementwise(dq, torch, steps, flush)
    elif which == "qconv_general":
        rec = bench_qconv_general(dq, torch, steps, flush)
    elif which == "lstm":
        rec = bench_lstm(dq, torch, steps, flush)
    else:
        rec = achievable(dq, torch, reps=steps)
    print(json.dumps({"only": which, "record": rec}), flush=True)


_KEEP = ("us_cold", "us_per_forward", "us_warm", "TOPS", "TOPS_cold", "TOPS_warm", "GBps_cold",
         "frac_cold", "GBps_stream", "frac_stream", "gemm_TOPS", "phase_us", "us_per_step_warm",
         "tokens_per_s_warm", "quant_a", "gemm", "host_enqueue")


def compact(v):
    """The few figures of a secondary record that the JSON line keeps (the
    whole record is on stderr, and in --detail's file)."""
    if not isinstance(v, dict):
        return v
    if any(k in v for k in _KEEP):
        return {k: v[k] for k in _KEEP if k in v}
    return {k: compact(x) for k, x in v.items() if isinstance(x, dict)}


if __name__ == "__main__":
    main()
