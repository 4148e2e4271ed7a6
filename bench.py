#!/usr/bin/env python3
"""Benchmark of the MI355X Gated DeltaNet path; prints ONE JSON line.

Headline workload: batched decode, B=64, Hk=16, Hv=32, D=128, bf16 operands,
float32 state, 100 chained decode steps updating the state in place (fresh
operands per step, already resident in HBM).  One benchmark "step" is one
such 100-token chain; ``value`` is the state traffic of the chain
(2 * 4 * B * Hv * D * D bytes per decode step: one read and one write of every
state row) divided by its time, in GB/s.

Also measured (object "scan"): the prefill scan B=1 T=4096 (bf16, token-major)
and the head-major scan B=16 T=1024 (f16), in tokens/s and algorithmic
TFLOP/s (7 * D * D flops per head-token) against the FP32 vector peak
(157.3 TFLOP/s): the block form (the default at D = 128) runs its products on
the matrix cores ("bound": "mfma"; with bf16/f16 operands over bf16 parts of
the f32 state, field "products"), so that fraction can pass 1; the matrix work
it actually issues is reported against the 2.5 PFLOP/s bf16 peak in
"matrix_cores" (from the committed counter summary).  The exact-products mode
is timed beside the default.

``roofline`` is for the decode kernel: algorithmic bytes per launch over its
average launch time (HIP events on the launch stream over the timed region),
against MI355X's 8 TB/s; ``traffic`` comes from the committed rocprofv3
FETCH_SIZE/WRITE_SIZE summary when it was taken on the current kernel source.
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the same
workload on this host.  ``gate_producer`` and ``conv_producer`` time the two
producers next to the recurrence (HBM-bound, algorithmic GB/s).
``shader_clock`` is the clock the chip sustains under a vector-ALU load and the
unpacked FP32 rate reached there (one and eight waves per SIMD), beside the
2.4 GHz at which the FP32 peak is quoted; ``decode_b1`` is the single decode
step, bound by launch latency.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN decode state GB/s + scan tokens/s, % of MI355X HBM/FP32 roofline"
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3  # FP32 vector and dense FP32 matrix peak alike
DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_kernel_b64_counters.txt")
SCAN_COUNTERS = os.path.join(ROOT, "profiles", "scan_kernels_instruction_counters.txt")
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak
# the kernels one default gdn_scan call launches, per scan workload
SCAN_KERNELS = {3: ("rows_la_kernel<2, 2, 128>", "prep_kernel<2, 2, 128, true, true>",
                    "gated_norm_kernel<2, 128>"),
                4: ("state_kernel<1, 2, 128>", "prep_kernel<1, 1, 128, false, false>")}
# sources the kernels are built from: their counters are stale once these change
_CSRC = os.path.join(ROOT, "linear_attention_recurrence_recurrent_amd", "csrc")
DECODE_SRC = [os.path.join(_CSRC, f) for f in ("gdn_decode.hip", "gdn_device.h")]
SCAN_SRC = [os.path.join(_CSRC, f) for f in ("gdn_chunk.hip", "gdn_scan.hip", "gdn_device.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def settle(fn, torch, min_ms):
    """Untimed: call fn until min_ms of wall time has passed.  The GPU's clocks
    ramp up over the first ~100 ms of sustained load (the first kernel timed
    in a fresh process runs up to ~20% slow), so every measurement below
    starts from the sustained clock state a long-running job sees."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def kernel_source_hash(files=None) -> str:
    h = hashlib.sha256()
    for f in files or DECODE_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def scan_matrix_figures(idx, ms):
    """Matrix-core work of one default scan call, from the committed rocprofv3
    counter summary (flops of the kernels' MFMA instructions per dispatch, the
    main kernel's matrix-core busy fraction) over this run's live call time.
    None when the summary is missing or was taken on another kernel source."""
    if not os.path.exists(SCAN_COUNTERS):
        return None
    kv = {}
    for line in open(SCAN_COUNTERS):
        m = re.match(r"^(scan_source_sha256|matrix\.\S.*?):\s*(.*)$", line.strip())
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("scan_source_sha256") != kernel_source_hash(SCAN_SRC):
        return None
    tot = {"bf16": 0.0, "f16": 0.0, "f32": 0.0}
    busy = None
    for i, kern in enumerate(SCAN_KERNELS[idx]):
        fields = dict(f.split("=", 1) for f in kv.get("matrix." + kern, "").split())
        if not fields:
            return None
        for t in tot:
            tot[t] += float(fields[t + "_flop"])
        if i == 0:
            busy = float(fields["busy"])
    sec = ms * 1e-3
    half = (tot["bf16"] + tot["f16"]) / sec / 1e12
    return {"main_kernel": SCAN_KERNELS[idx][0],
            "bf16_f16_tflops_issued": round(half, 1), "bf16_peak_tflops": BF16_PEAK_TFLOPS,
            "frac_of_bf16_peak": round(half / BF16_PEAK_TFLOPS, 4),
            "f32_mfma_tflops_issued": round(tot["f32"] / sec / 1e12, 2),
            "main_kernel_matrix_busy": busy,
            "source": "profiles/scan_kernels_instruction_counters.txt"}


def matrix_lines(paths):
    """Machine-readable per-kernel lines of the matrix-core counters (MOPS of
    512 flops each; busy = SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles of
    the dispatch, GRBM_GUI_ACTIVE summing the 8 XCDs, 1024 SIMDs)."""
    import csv
    acc = {}
    for path in paths:
        per = {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                key = (row["Dispatch_Id"], _short_kernel(row["Kernel_Name"]))
                d = per.setdefault(key, {})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        for (_, k), d in per.items():
            for c, v in d.items():
                acc.setdefault(k, {}).setdefault(c, []).append(v)
    print("scan_source_sha256: %s" % kernel_source_hash(SCAN_SRC))
    for k, cs in sorted(acc.items()):
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        need = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
        if not all(n in avg for n in need):
            continue
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * avg["GRBM_GUI_ACTIVE"] / 8)
        print("matrix.%s: bf16_flop=%.6g f16_flop=%.6g f32_flop=%.6g busy=%.4f" % (
            k, 512 * avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"], 512 * avg["SQ_INSTS_VALU_MFMA_MOPS_F16"],
            512 * avg["SQ_INSTS_VALU_MFMA_MOPS_F32"], busy))


def read_counters():
    """HBM bytes per decode launch from the committed rocprofv3 summary, or None
    when the summary is missing or was taken on another kernel source."""
    if not os.path.exists(DECODE_COUNTERS):
        return None
    kv = {}
    for line in open(DECODE_COUNTERS):
        m = re.match(r"^\s*([a-z_0-9]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Launcher:
    """Pre-marshalled C-ABI call (no per-call Python validation in the timed loop)."""

    def __init__(self, fn_name, desc, tensors, stream, extra=()):
        from linear_attention_recurrence_recurrent_amd import _native
        self.fn = getattr(_native.lib(), fn_name)
        self.desc = desc
        self.args = [ctypes.byref(desc)] + [
            None if t is None else ctypes.c_void_p(t.data_ptr()) for t in tensors
        ] + list(extra) + [ctypes.c_void_p(stream)]

    def __call__(self):
        rc = self.fn(*self.args)
        if rc:
            from linear_attention_recurrence_recurrent_amd import _native
            raise RuntimeError("launch rejected: %s" % _native.last_error())


def shader_clock(torch, args):
    """The shader clock the chip sustains under a vector-ALU load (the FP32
    peak is quoted at 2.4 GHz): the library's clock reference kernel
    (include/gdn_calib.h) with one wave per SIMD and with eight, each after the
    settle period.  The clock is the waves' shader cycles over their ticks of
    the constant 100 MHz counter; that counter's rate is checked against the
    HIP events around the same launch.  The FMAs issued per second are the
    unpacked FP32 rate the vector units reach there."""
    from linear_attention_recurrence_recurrent_amd import _native
    L = _native.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, waves, iters in (("one_wave_per_simd", 1024, 40000),
                               ("eight_waves_per_simd", 8192, 8000)):
        out = torch.zeros(4 * waves, dtype=torch.int64, device=dev)

        def call():
            rc = L.gdn_calib_clock(waves, iters, ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream))
            if rc:
                raise RuntimeError("clock kernel rejected: %s" % _native.last_error())
        settle(call, torch, args.settle_ms)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        o = out.view(waves, 4).cpu().double()
        ghz = float(o[:, 0].sum() / o[:, 1].sum()) * 0.1
        res[name + "_ghz"] = round(ghz, 3)
        res[name + "_us"] = round(us, 1)
        # eight FMAs per round on each of 64 lanes: the unpacked FP32 rate achieved
        res[name + "_fma_tflops"] = round(waves * iters * 8 * 64 * 2 / (us * 1e-6) / 1e12, 1)
        if name == "one_wave_per_simd":
            res["realtime_counter_mhz"] = round(float(o[:, 1].max()) / us, 1)
        log("shader clock, %s: %.3f GHz over %.0f us" % (name.replace("_", " "), ghz, us))
    return res


def streaming_ceiling(torch, nbytes, args):
    """The HBM rate an in-place state update can reach here: the library's
    streaming reference kernels (include/gdn_calib.h) rewrite a buffer of the
    decode state's size in place (read + write, one multiply-add per element)
    or copy it, each call on the next of four such buffers, so the working set
    (4x the state) exceeds the 256 MB Infinity Cache.  Every access variant is
    timed; the fastest read-modify-write is the ceiling."""
    from linear_attention_recurrence_recurrent_amd import _native
    L = _native.lib()
    dev = torch.device("cuda:0")
    nbuf = 4
    bufs = [torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(0.5)
            for _ in range(nbuf)]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    ptr = [ctypes.c_void_p(b.data_ptr()) for b in bufs]

    def timed(fn, reps=24):
        settle(lambda: [fn(i) for i in range(nbuf)], torch, args.settle_ms / 8)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def call(op, v, a, b):
        rc = L.gdn_calib_stream(op, v, ptr[a], ptr[b], nbytes, sp)
        if rc:
            raise RuntimeError(_native.last_error())

    rmw, copy = {}, {}
    for v in range(_native.GDN_CALIB_VARIANTS):
        name = L.gdn_calib_variant_name(v).decode()
        rmw[name] = 2 * nbytes / timed(lambda i: call(_native.GDN_CALIB_RMW, v, i % nbuf,
                                                      i % nbuf)) / 1e9
        copy[name] = 2 * nbytes / timed(lambda i: call(_native.GDN_CALIB_COPY, v, i % nbuf,
                                                       (i + 1) % nbuf)) / 1e9
    torch_copy = 2 * nbytes / timed(lambda i: bufs[(i + 1) % nbuf].copy_(bufs[i % nbuf])) / 1e9
    del bufs
    best_rmw = max(rmw, key=rmw.get)
    best_copy = max(copy, key=copy.get)
    log("streaming ceiling at %d MB per buffer, %d buffers in turn: in-place %.1f GB/s (%s), "
        "copy %.1f GB/s (%s), torch copy %.1f GB/s" % (nbytes >> 20, nbuf, rmw[best_rmw],
                                                        best_rmw, copy[best_copy], best_copy,
                                                        torch_copy))
    return {"rmw_gbs": round(rmw[best_rmw], 1), "rmw_variant": best_rmw,
            "copy_gbs": round(copy[best_copy], 1), "copy_variant": best_copy,
            "torch_copy_gbs": round(torch_copy, 1), "buffer_bytes": nbytes, "buffers": nbuf,
            "working_set_bytes": nbuf * nbytes,
            "rmw_all_gbs": {k: round(x, 1) for k, x in rmw.items()}}


def bench_decode(args, torch):
    import linear_attention_recurrence_recurrent_amd as gdn
    from linear_attention_recurrence_recurrent_amd import synth
    wl = synth.WORKLOADS[2]
    log("decode: drawing operands (B=%d, %d steps)" % (wl.B, wl.steps))
    ops = synth.make(wl)
    steps = synth.step_slices(ops, head_major=False)
    dev = torch.device("cuda:0")
    d_steps = [{n: t.to(dev) for n, t in st.items()} for st in steps]
    w = ops["w"].to(dev)
    state = ops["s0"].to(dev).clone()
    ys = [torch.empty(st["v"].shape, dtype=torch.float32, device=dev) for st in d_steps]
    stream = torch.cuda.current_stream(dev)
    desc = gdn._desc(wl.B, 1, wl.Hk, wl.Hv, wl.Dk, wl.Dv, False, 2, 2, True, True, 1e-6, 1e-6)
    calls = [Launcher("gdn_recurrent_step", desc,
                      [st["q"], st["k"], st["v"], st["log_decay"], st["beta"], state, st["z"], w,
                       y, state], stream.cuda_stream) for st, y in zip(d_steps, ys)]

    def chain():
        for c in calls:
            c()

    for _ in range(args.warmup):
        chain()
    settle(chain, torch, args.settle_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        chain()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    launches = args.steps * wl.steps
    state_bytes = 2 * 4 * wl.B * wl.Hv * wl.Dv * wl.Dk
    es = 2  # bf16
    io_bytes = (2 * wl.B * wl.Hk * wl.Dk * es + 2 * wl.B * wl.Hv * wl.Dv * es
                + 2 * wl.B * wl.Hv * es + wl.Dv * es + wl.B * wl.Hv * wl.Dv * 4)
    launch_s = ms * 1e-3 / launches
    ms_per_chain = ms / args.steps
    value = state_bytes * wl.steps / (ms_per_chain * 1e-3) / 1e9
    achieved = state_bytes / launch_s / 1e9
    traffic = read_counters()
    ceiling = streaming_ceiling(torch, state_bytes // 2, args)
    # template arguments: operand and gate dtype, D, lanes per row, rows per
    # lane, waves, the state stores' cache policy (18 = nt | sc1: from 128 MiB
    # of state the stores are written through at device scope)
    kernel = "decode_kernel<bf16,bf16,128,16,2,16,18>"
    res = dict(ms_per_step=ms_per_chain, value=value, launch_us=launch_s * 1e6,
               roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic, "kernel": kernel,
                         "algorithmic_bytes_per_launch": state_bytes,
                         "operand_io_bytes_per_launch": io_bytes,
                         "avg_launch_us": round(launch_s * 1e6, 3),
                         "ceiling": ceiling,
                         "frac_of_rmw_ceiling": round(achieved / ceiling["rmw_gbs"], 4)})
    log("decode: %.3f ms per 100-step chain, %.2f us per launch, state %.1f GB/s = %.1f%% of "
        "8 TB/s, %.1f%% of the in-place streaming ceiling (%.1f GB/s)" %
        (ms_per_chain, launch_s * 1e6, achieved, 100 * achieved / HBM_PEAK_GBS,
         100 * achieved / ceiling["rmw_gbs"], ceiling["rmw_gbs"]))

    # the same chain with the state double-buffered (each step reads one buffer
    # and writes the other, s_out of a step is s0 of the next): the same bytes,
    # no read and write of the same lines within a launch
    state_b = torch.empty_like(state)
    calls_db = [Launcher("gdn_recurrent_step", desc,
                         [st["q"], st["k"], st["v"], st["log_decay"], st["beta"],
                          state if i % 2 == 0 else state_b, st["z"], w, y,
                          state_b if i % 2 == 0 else state], stream.cuda_stream)
                for i, (st, y) in enumerate(zip(d_steps, ys))]

    def chain_db():
        for c in calls_db:
            c()

    settle(chain_db, torch, args.settle_ms / 4)
    e0.record(stream)
    for _ in range(args.steps):
        chain_db()
    e1.record(stream)
    torch.cuda.synchronize()
    db_us = e0.elapsed_time(e1) * 1e3 / launches
    del state_b
    res["double_buffered"] = {"us_per_step": round(db_us, 2),
                              "state_gbs": round(state_bytes / (db_us * 1e-6) / 1e9, 1)}
    log("decode double-buffered: %.1f us per launch, state %.1f GB/s" %
        (db_us, state_bytes / (db_us * 1e-6) / 1e9))

    # ablation: the literal three-pass step on the same chain (3 reads + 1 write of S)
    calls3 = [Launcher("gdn_recurrent_step_three_pass", desc,
                       [st["q"], st["k"], st["v"], st["log_decay"], st["beta"], state, st["z"], w,
                        y, state], stream.cuda_stream) for st, y in zip(d_steps, ys)]
    def chain3():
        for c in calls3:
            c()

    settle(chain3, torch, args.settle_ms / 4)
    reps3 = max(1, args.steps // 4)
    e0.record(stream)
    for _ in range(reps3):
        for c in calls3:
            c()
    e1.record(stream)
    torch.cuda.synchronize()
    ms3 = e0.elapsed_time(e1) / reps3
    step3_us = ms3 * 1e3 / wl.steps
    res["ablation"] = {
        "three_pass_us_per_step": round(step3_us, 2),
        "three_pass_state_bytes_per_step": 2 * state_bytes,
        "three_pass_gbs": round(2 * state_bytes / (step3_us * 1e-6) / 1e9, 1),
        "fused_us_per_step": round(launch_s * 1e6, 2),
        "fusion_speedup": round(step3_us / (launch_s * 1e6), 3)}
    log("decode three-pass: %.1f us per step (fusion speedup %.2fx)" %
        (step3_us, step3_us / (launch_s * 1e6)))
    return res, ops


def bench_decode_single(args, torch):
    """The single decode step at B=1 (Hk16 Hv32 D128, bf16): its 4 MiB state fits
    in the caches, so this measures launch latency more than HBM."""
    import linear_attention_recurrence_recurrent_amd as gdn
    from linear_attention_recurrence_recurrent_amd import synth
    wl = synth.WORKLOADS[1]
    ops = synth.make(wl)
    dev = torch.device("cuda:0")
    d = {n: t.to(dev) for n, t in ops.items()}
    y = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    desc = gdn._desc(wl.B, 1, wl.Hk, wl.Hv, wl.Dk, wl.Dv, False, 2, 2, True, True, 1e-6, 1e-6)
    call = Launcher("gdn_recurrent_step", desc, [d["q"], d["k"], d["v"], d["log_decay"],
                                                 d["beta"], d["s0"], d["z"], d["w"], y, d["s0"]],
                    stream.cuda_stream)
    settle(call, torch, args.settle_ms / 4)
    reps = 200
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    state_bytes = 2 * 4 * wl.B * wl.Hv * wl.Dv * wl.Dk
    log("decode B=1: %.2f us per step, state %.1f GB/s" % (us, state_bytes / (us * 1e-6) / 1e9))
    return {"workload": wl.name, "us_per_step": round(us, 2), "state_bytes": state_bytes,
            "state_gbs": round(state_bytes / (us * 1e-6) / 1e9, 1)}


def bench_scan(idx, args, torch):
    import linear_attention_recurrence_recurrent_amd as gdn
    from linear_attention_recurrence_recurrent_amd import synth
    wl = synth.WORKLOADS[idx]
    log("scan %d: drawing operands (%s)" % (idx, wl.name))
    ops = synth.make(wl)
    dev = torch.device("cuda:0")
    d = {n: t.to(dev) for n, t in ops.items()}
    del ops
    y = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
    s_out = torch.empty_like(d["s0"])
    stream = torch.cuda.current_stream(dev)
    dt = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    form_arg = None if args.scan_form == "auto" else args.scan_form

    def timed_call(exact):
        desc = gdn._desc(wl.B, wl.T, wl.Hk, wl.Hv, wl.Dk, wl.Dv, wl.head_major, dt, dt, True,
                         True, 1e-6, 1e-6, form_arg, exact)
        ws_bytes = gdn.scan_workspace_bytes(desc)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)  # caller-owned
        call = Launcher("gdn_scan", desc, [d["q"], d["k"], d["v"], d["log_decay"], d["beta"],
                                           d["s0"], d["z"], d["w"], y, s_out], stream.cuda_stream,
                        extra=(ctypes.c_void_p(ws.data_ptr()), ctypes.c_uint64(ws_bytes)))
        reps = max(3, args.steps)
        for _ in range(max(1, args.warmup)):
            call()
        settle(call, torch, args.settle_ms)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed_call(False)
    flops = 7.0 * wl.B * wl.T * wl.Hv * wl.Dv * wl.Dk
    form = args.scan_form
    if form == "auto":  # the library's choice: the block form at these shapes
        form = "block"
    bound = "mfma" if form == "block" else "alu"
    tflops = flops / (ms * 1e-3) / 1e12
    tok = wl.B * wl.T / (ms * 1e-3)
    log("scan %d: %.1f us per call, %.2f M tok/s, %.1f TFLOP/s" % (idx, ms * 1e3, tok / 1e6, tflops))
    # the method's flops (7 D^2 per head-token) against the FP32 vector peak: the
    # unit the scan's target is set in; the block form runs its products on the
    # matrix cores, so this fraction can pass 1 (the matrix work actually issued
    # is in "matrix_cores", against the bf16 peak)
    res = {"workload": wl.name, "us_per_call": round(ms * 1e3, 2), "tokens_per_s": round(tok, 1),
           "algorithmic_tflops": round(tflops, 2),
           "fp32_vector_peak_tflops": FP32_PEAK_TFLOPS,
           "frac_of_fp32_vector_peak": round(tflops / FP32_PEAK_TFLOPS, 4), "bound": bound,
           "form": form, "algorithmic_flops_per_call": flops}
    if form == "block" and wl.dtype in ("bf16", "f16"):
        res["products"] = ("f32 state; its products on the bf16 matrix cores over two bf16 parts "
                           "rounded to nearest (each term within 2^-16 of the f32 product; f16 q "
                           "and k split exactly in two)")
        ms_x = timed_call(True)
        log("scan %d exact products: %.1f us per call" % (idx, ms_x * 1e3))
        res["exact_products"] = {"us_per_call": round(ms_x * 1e3, 2),
                                 "algorithmic_tflops": round(flops / (ms_x * 1e-3) / 1e12, 2),
                                 "products": "three exact bf16 parts of the state: exact f32 "
                                             "products"}
    else:
        res["products"] = "f32"
    res["matrix_cores"] = scan_matrix_figures(idx, ms)
    return res


HEAD_DIM_SHAPES = [
    # (name, B, T, Hk, Hv, dtype, head_major): the two scan workloads' shapes at other head dims
    ("prefill_b1_t4096_bf16", 1, 4096, 16, 32, "bf16", False),
    ("head_major_b16_t1024_f16", 16, 1024, 16, 32, "f16", True),
]
# and with f32 operands at head dim 256 (the block form's f32 path with q and k from global memory)
F32_256_SHAPES = [
    ("prefill_b1_t4096_f32", 1, 4096, 16, 32, "f32", False),
    ("head_major_b16_t1024_f32", 16, 1024, 16, 32, "f32", True),
]
DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def bench_head_dims(args, torch):
    """Both time loops of the scan at head dims 32, 64 and 256 on the shapes of
    the two scan workloads (synthetic operands, the workloads' recipe), and at
    256 with f32 operands too."""
    import linear_attention_recurrence_recurrent_amd as gdn
    from linear_attention_recurrence_recurrent_amd import synth
    dev = torch.device("cuda:0")
    out = []
    cases = [(D, sh) for D in (32, 64, 256) for sh in HEAD_DIM_SHAPES]
    cases += [(256, sh) for sh in F32_256_SHAPES]
    for D, (name, B, T, Hk, Hv, dt, hm) in cases:
        ops = synth.random_operands(B, T, Hk, Hv, D, D, dtype=dt, head_major=hm, seed=D)
        d = {n: t.to(dev) for n, t in ops.items()}
        y = torch.empty(d["v"].shape, dtype=torch.float32, device=dev)
        s_out = torch.empty_like(d["s0"])
        row = {"shape": name, "D": D, "dtype": dt}
        flops = 7.0 * B * T * Hv * D * D
        for form in ("per_token", "block"):
            desc = gdn._desc(B, T, Hk, Hv, D, D, hm, DT_CODE[dt], DT_CODE[dt], True, True,
                             1e-6, 1e-6, form, False)
            ws = torch.empty(max(gdn.scan_workspace_bytes(desc), 1), dtype=torch.uint8,
                             device=dev)

            def call():
                gdn.scan(d["q"], d["k"], d["v"], d["log_decay"], d["beta"], d["s0"], d["z"],
                         d["w"], head_major=hm, form=form, out=y, state_out=s_out,
                         workspace=ws)
            for _ in range(max(1, args.warmup)):
                call()
            settle(call, torch, args.settle_ms)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(3, args.steps)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            row[form] = {"us_per_call": round(us, 1),
                         "frac_of_fp32_vector_peak": round(flops / us / 1e6 / FP32_PEAK_TFLOPS, 4)}
            log("D=%d %s %s: %.1f us" % (D, name, form, us))
        row["speedup"] = round(row["per_token"]["us_per_call"] / row["block"]["us_per_call"], 2)
        out.append(row)
        del d, y, s_out
    return out


def bench_gates(args, torch):
    """Gate producer on the head-major scan's gate count (B*T*Hv = 16*1024*32), f16."""
    from linear_attention_recurrence_recurrent_amd import _native
    n = 16 * 1024 * 32
    g = torch.Generator(device="cpu").manual_seed(5)
    a = torch.randn(n, generator=g).to(torch.float16).cuda()
    b = torch.randn(n, generator=g).to(torch.float16).cuda()
    ld = torch.empty_like(a)
    be = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    L = _native.lib()
    args_c = (n, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), 1, 0.01,
              ctypes.c_void_p(ld.data_ptr()), ctypes.c_void_p(be.data_ptr()), 1,
              ctypes.c_void_p(stream.cuda_stream))
    for _ in range(3):
        assert L.gdn_gates(*args_c) == 0
    settle(lambda: L.gdn_gates(*args_c), torch, args.settle_ms / 4)
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        L.gdn_gates(*args_c)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = 4 * 2 * n
    log("gates: %.2f us per launch for %d elements" % (us, n))
    return {"elements": n, "us_per_launch": round(us, 2), "bytes_per_launch": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "dtype": "f16"}


def bench_conv(args, torch):
    """Conv + silu producer (W=4, bf16) on the q/k/v channels of the scan's heads:
    C = 2*Hk*D + Hv*D = 8192.  Prefill: B=1, T=4096, no context.  Decode: B=64,
    T=1 with its [B, C, 3] context updated in place.  HBM-bound: algorithmic
    bytes = x read + y written + carried context read and written + weights."""
    from linear_attention_recurrence_recurrent_amd import _native
    L = _native.lib()
    C, W, es = 2 * 16 * 128 + 32 * 128, 4, 2
    g = torch.Generator(device="cpu").manual_seed(7)
    out = {}
    for name, B, T, with_state in (("prefill_b1_t4096_c8192_w4_bf16", 1, 4096, False),
                                   ("decode_b64_t1_c8192_w4_bf16", 64, 1, True)):
        x = torch.randn((B, T, C), generator=g).to(torch.bfloat16).cuda()
        w = (torch.randn((C, W), generator=g) * 0.5).to(torch.bfloat16).cuda()
        y = torch.empty_like(x)
        st = torch.randn((B, C, W - 1), generator=g).to(torch.bfloat16).cuda() if with_state \
            else None
        stream = torch.cuda.current_stream()
        vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        args_c = (B, T, C, W, 2, 1, vp(x), vp(w), None, vp(st), vp(y), vp(st),
                  ctypes.c_void_p(stream.cuda_stream))
        for _ in range(3):
            assert L.gdn_conv_silu(*args_c) == 0
        settle(lambda: L.gdn_conv_silu(*args_c), torch, args.settle_ms / 4)
        reps = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            L.gdn_conv_silu(*args_c)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = 2 * B * T * C * es + C * W * es + (2 * B * C * (W - 1) * es if with_state else 0)
        gbs = nbytes / (us * 1e-6) / 1e9
        log("conv %s: %.2f us per launch, %.1f GB/s" % (name, us, gbs))
        out[name] = {"us_per_launch": round(us, 2), "algorithmic_bytes_per_launch": nbytes,
                     "gbs": round(gbs, 1), "peak_gbs": HBM_PEAK_GBS,
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
                     "tokens_per_s": round(B * T / (us * 1e-6), 1)}
    return out


def cpu_baseline(ops, args):
    """The float64 oracle on the whole decode chain (100 chained steps of all 64
    sequences == the scan over 100 tokens), repeated until about ``cpu_seconds``
    of wall time have passed."""
    import numpy as np
    from oracle import gdn_oracle as orc
    f64 = {k: np.ascontiguousarray(v.double().numpy()) for k, v in ops.items()}
    threads = orc.default_threads()
    orc._load()  # build/load outside the timed region
    T = f64["q"].shape[1]
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.scan(**f64, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= args.cpu_seconds or reps >= 1000:
            break
    B, Hv, D = ops["s0"].shape[0], ops["s0"].shape[1], ops["s0"].shape[2]
    gbs = 2 * 4 * B * Hv * D * D * T * reps / dt / 1e9
    log("cpu oracle: %d x %d tokens x B=%d in %.2f s on %d threads: %.3f GB/s" %
        (reps, T, B, dt, threads, gbs))
    # the same chain once on a single thread
    t1 = time.perf_counter()
    orc.scan(**f64, threads=1)
    dt1 = time.perf_counter() - t1
    gbs1 = 2 * 4 * B * Hv * D * D * T / dt1 / 1e9
    log("cpu oracle, one thread: %.2f s per chain: %.3f GB/s" % (dt1, gbs1))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "float64 three-pass oracle on the whole decode chain (B=64 Hk16 Hv32 "
                      "D128, 100 chained steps), run %d times in %.1f s" % (reps, dt),
            "single_thread_value": round(gbs1, 4), "cpu_model": model}


def copy_reference(args, torch):
    """A plain copy kernel of known size: its FETCH_SIZE/WRITE_SIZE readings give the
    factor that turns those counters into bytes."""
    n = args.copy_ref_mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(max(1, args.steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_each_way": n * 4, "launches": max(1, args.steps)}))


# ------------------------------------------------------------------ profile summaries
# rocprofv3 writes CSV files (a kernel trace with one row per dispatch, or a
# counter collection with one row per dispatch and counter); these turn them
# into the short summaries kept under profiles/.

def _short_kernel(name):
    """'gdn::(anonymous namespace)::decode_kernel<2, 2, 128>(gdn::...)' -> 'decode_kernel<2, 2, 128>'."""
    name = name.replace("(anonymous namespace)", "anon")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # the parameter list starts at the first '(' outside <>
        depth += (ch == "<") - (ch == ">")
        if ch == "(" and depth == 0:
            cut = i
            break
    base = name[:cut].strip()
    depth, start = 0, 0
    for i, ch in enumerate(base):  # keep what follows the last '::' outside <>
        depth += (ch == "<") - (ch == ">")
        if depth == 0 and base.startswith("::", i):
            start = i + 2
    base = base[start:]
    return base.split(" ")[-1] if " " in base and "<" not in base else base


def _grid(row):
    if "Grid_Size" in row and row["Grid_Size"]:
        return int(float(row["Grid_Size"]))
    g = 1
    for ax in ("X", "Y", "Z"):
        v = row.get("Grid_Size_" + ax)
        if v:
            g *= int(float(v))
    return g


def trace_summary(path):
    """Per (kernel, grid size): calls, average / median / min / max duration."""
    import csv
    import statistics
    groups = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            key = (_short_kernel(row["Kernel_Name"]), _grid(row))
            us = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3
            groups.setdefault(key, []).append(us)
    total = sum(sum(v) for v in groups.values())
    print("| kernel | grid (threads) | calls | avg us | median us | min us | max us | share |")
    print("|---|---|---|---|---|---|---|---|")
    for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print("| %s | %d | %d | %.2f | %.2f | %.2f | %.2f | %.1f%% |" % (
            k, g, len(v), sum(v) / len(v), statistics.median(v), min(v), max(v),
            100 * sum(v) / total))


def counter_summary(paths):
    """Per (kernel, grid size): every counter averaged over the dispatches
    (counter values are summed over the GPU's XCDs and dimensions first)."""
    import csv
    acc = {}
    for path in paths:
        per_dispatch = {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                key = (_short_kernel(row["Kernel_Name"]), _grid(row))
                d = per_dispatch.setdefault((row["Dispatch_Id"], key), {})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(
                    row["Counter_Value"])
        for (_, key), d in per_dispatch.items():
            a = acc.setdefault(key, {})
            for c, v in d.items():
                a.setdefault(c, []).append(v)
    for (k, g), cs in sorted(acc.items()):
        print("%s grid %d:" % (k, g))
        for c, v in sorted(cs.items()):
            print("  %s %.6g per dispatch (%d dispatches)" % (c, sum(v) / len(v), len(v)))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls for this long before each measurement (clock ramp)")
    ap.add_argument("--no-scan", action="store_true", help="skip the scan sub-measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--scan-form", choices=("auto", "per_token", "block"), default="auto",
                    help="time loop of the scan (default: the library's choice per shape)")
    ap.add_argument("--scan-only", action="store_true",
                    help="only the two scan workloads (for counter collection); partial JSON")
    ap.add_argument("--head-dims", action="store_true",
                    help="only both scan forms at head dims 32, 64 and 256 on the scan shapes "
                         "(and f32 operands at 256)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this size (counter reference)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print the per-kernel, per-grid summary of a rocprofv3 kernel trace")
    ap.add_argument("--counter-summary", metavar="CSV", nargs="+",
                    help="print per-kernel averages of rocprofv3 --pmc counter CSV files")
    ap.add_argument("--matrix-lines", metavar="CSV", nargs="+",
                    help="print the per-kernel matrix-core lines bench.py reads back from "
                         "profiles/ (from the MOPS / MFMA-busy counter CSV)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.matrix_lines:
        matrix_lines(args.matrix_lines)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (each (batch, "
              "value head) pair is independent, so several GPUs would each run their share of the heads)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_ref_mib:
        copy_reference(args, torch)
        return
    import linear_attention_recurrence_recurrent_amd  # noqa: F401  (fails loudly if unbuilt)
    if args.head_dims:
        print(json.dumps({"head_dims": bench_head_dims(args, torch)}))
        return
    if args.scan_only:
        print(json.dumps({"scan": {"prefill_b1_t4096_bf16": bench_scan(3, args, torch),
                                   "head_major_b16_t1024_f16": bench_scan(4, args, torch)}}))
        return
    dec, ops = bench_decode(args, torch)
    scan = {}
    if not args.no_scan:
        scan["prefill_b1_t4096_bf16"] = bench_scan(3, args, torch)
        scan["head_major_b16_t1024_f16"] = bench_scan(4, args, torch)
    out = {
        "metric": METRIC,
        "value": round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode B64 Hk16 Hv32 D128, bf16 operands, f32 state, 100 chained "
                               "in-place steps per benchmark step",
                   "B": 64, "Hk": 16, "Hv": 32, "D": 128, "tokens_per_step": 100,
                   "parallelism": "single GPU"},
        "roofline": dec["roofline"],
        "ablation_three_pass_decode": dec["ablation"],
        "decode_double_buffered": dec["double_buffered"],
    }
    out["decode_b1"] = bench_decode_single(args, torch)
    out["shader_clock"] = shader_clock(torch, args)
    if scan:
        out["scan"] = scan
    if not args.no_scan:
        out["gate_producer"] = bench_gates(args, torch)
        out["conv_producer"] = bench_conv(args, torch)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(ops, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
