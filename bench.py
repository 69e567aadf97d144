"""Benchmark: fused butterfly rotation + INT4 quantization on one MI355X.

Workload (the headline one): n = 4096, 8192 bf16 token rows with 0.1 % x50
outlier channels (LLaMA-2-7B hidden width), 12 Givens stages with 24576
angles, bf16 Q x out, symmetric absmax INT4 codes per group of 128 with fp16
scales.  One step = one bfly_forward_quant call from the angles (the
prepare kernel makes the coefficient table in the call's workspace, then the
fused kernel runs over all 8192 rows).  Inputs are resident in HBM before the
timed region; the step cycles through 5 separate input/output buffer sets
(722 MiB) so that no step finds its rows in the 256 MB last-level cache.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

Prints ONE JSON line.  `value` is algorithmic GB/s of the whole step:
18 496 B per row (8192 in + 8192 out + 2048 codes + 64 scale bytes) plus the
96 KiB of angles, divided by the mean step time.  After the timed steps the
fused kernel runs again with its table made once (fixed angles, as at
inference), back to back, at least 200 times: a HIP event pair around those
launches on their stream gives its average launch duration
(`roofline.kernel_avg_us`), which `roofline` prices against the 8 TB/s HBM
peak.  Then 240 launches with events attached to each dispatch
(bfly_time_next_forward) give the median and spread beside it.  `traffic` comes from
rocprofv3 FETCH_SIZE / WRITE_SIZE counters recorded for the current kernel
sources (null if they changed).  `roofline.copy_context` is a plain device
copy of the same bytes (half read, half written) timed the same way, as
context only.  `cpu_baseline` times the fp64 oracle on the host's cores (all
threads; one-thread timings of three workloads beside it).

--workload picks one of the other workloads for a secondary line:
tiny_n256_fp32, weight_n4096_bf16_int2, kron_n5120_bf16_int4,
kron_n11008_bf16_int4, kron_bwd_n5120_fp32, calib_n4096_fp32_fwd_bwd,
calib_step_n4096_fp32, calib_step_weight_n4096_out4096, act_n8192_bf16_int4,
hadamard_n4096_bf16_int4, w2a16_m8192_k4096_n11008,
w2a16_m1_k4096_n11008, w2a16_m16_k4096_n11008.  --copy-probe runs a plain
device copy of known size (for calibrating the byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "butterfly+quant GB/s (% of HBM roofline), n=4096, 8192 rows bf16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X
MFMA_FP32_PEAK_TFLOPS = 157.3   # dense fp32 matrix-core peak of the MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bfly_fwd_quant_n4096_bf16_int4_traffic.txt")
NSETS = 5


# The sources the fused forward kernel is compiled from (its translation unit
# and every header it includes): the recorded counters hold while these are
# unchanged.
FUSED_KERNEL_SOURCES = ("bfly_fwd_plain.hip", "bfly_fwd_kernel.h", "bfly_common.h",
                        "bfly_internal.h")


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    for name in FUSED_KERNEL_SOURCES:
        p = os.path.join(ROOT, "learnable_butterfly_rotation_amd", "csrc", name)
        h.update(name.encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the fused kernel from the committed counter
    summary, or None if it is missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != kernel_sources_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(oracle, w, kind):
    """One pass of the oracle over a workload: fp64 forward (or Kronecker
    forward), bf16 rounding of y, the workload's quantizer."""
    if kind == "tiny":
        oracle.forward(w["x"], w["theta"])
    elif kind == "act":
        y64 = oracle.forward(w["x"], w["theta"])
        oracle.round_bf16(y64)
        oracle.quantize(y64, 4, 128, oracle.SYM)
    else:  # kron
        y64 = oracle.kron_forward(w["x"], w["theta_b"], w["mix"])
        oracle.round_bf16(y64)
        oracle.quantize(y64, 4, 128, oracle.SYM)


def _median_time(fn, passes):
    ts = []
    for _ in range(passes):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline_act(w, bytes_per_row, inputs, passes=3):
    """The oracle on the headline workload with all host threads (the
    reported baseline), plus one-thread timings of the tiny, headline and
    n = 5120 Kronecker workloads."""
    import oracle
    threads = oracle.num_threads()
    rows = w["x"].shape[0]
    t = _median_time(lambda: _oracle_pass(oracle, w, "act"), passes)
    one = {}
    try:
        oracle.set_num_threads(1)
        for name, wl, kind, bpr in (
                ("tiny_n256_fp32", inputs.tiny_fp32(), "tiny", 256 * 8),
                ("act_n4096_bf16_int4", w, "act", bytes_per_row),
                ("kron_n5120_bf16_int4", inputs.kron_int4(rows=2048), "kron",
                 10240 + 10240 + 2560 + 80)):
            r = wl["x"].shape[0]
            t1 = _median_time(lambda: _oracle_pass(oracle, wl, kind), 3 if kind == "tiny" else 1)
            one[name] = {"rows": r, "s": round(t1, 4), "rows_per_s": round(r / t1),
                         "GBs": round(r * bpr / t1 / 1e9, 5)}
    finally:
        oracle.set_num_threads(threads)
    return {"value": rows * bytes_per_row / t / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "all %d rows of the workload (fp64 forward, bf16 rounding, INT4 quantization),"
                      " median of %d passes: %.3f s per pass, %.0f rows/s" % (rows, passes, t, rows / t),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "one_thread": one}


# ---------------------------------------------------------------------------
# the headline workload
# ---------------------------------------------------------------------------

KERNEL_TIMED_LAUNCHES = 240   # event-timed launches of the fused kernel, whatever --steps is


def warm_up(torch, fn, steps, min_seconds=0.3):
    """Run `steps` untimed steps, then keep going until `min_seconds` have
    passed, so the timed steps start at steady clocks.  Returns the seconds
    spent."""
    t0 = time.perf_counter()
    i = 0
    while i < steps or time.perf_counter() - t0 < min_seconds:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def copy_context(torch, stream, nbytes, reps=200, sets=5):
    """GB/s of a plain device copy moving `nbytes` (half read, half written)
    per call, rotating buffer pairs so no copy finds its source in cache."""
    n = nbytes // 8  # fp32 elements per buffer
    bufs = [(torch.ones(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(sets)]
    for i in range(20):
        bufs[i % sets][1].copy_(bufs[i % sets][0])
    torch.cuda.synchronize()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev[0].record(stream)
    for i in range(reps):
        bufs[i % sets][1].copy_(bufs[i % sets][0])
    ev[1].record(stream)
    torch.cuda.synchronize()
    s = ev[0].elapsed_time(ev[1]) / 1e3 / reps
    del bufs
    return 8 * n / s / 1e9


def bench_act(args, torch, B, inputs):
    w = inputs.act_int4()
    x, th = w["x"], w["theta"]
    rows, n = x.shape
    group, bits = 128, 4
    bytes_per_row = 2 * n + 2 * n + n * bits // 8 + 2 * (n // group)     # 18 496
    step_bytes = rows * bytes_per_row + th.nbytes
    kernel_bytes = rows * bytes_per_row

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    theta = to_dev(th, torch)
    tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    sets = []
    xd = to_dev(x, torch)
    for k in range(NSETS):
        sets.append({
            "x": xd if k == 0 else xd.clone(),
            "y": torch.empty((rows, n), dtype=torch.bfloat16, device="cuda"),
            "codes": torch.empty((rows, n * bits // 8), dtype=torch.uint8, device="cuda"),
            "scales": torch.empty((rows, n // group), dtype=torch.float16, device="cuda"),
        })
    lib = B.lib()
    ptrs = [(s["x"].data_ptr(), s["y"].data_ptr(), s["codes"].data_ptr(), s["scales"].data_ptr())
            for s in sets]
    th_p, tab_p, tab_n = theta.data_ptr(), tab.data_ptr(), tab.numel()

    def launch(i, ev=None, from_angles=True):
        px, py, pc, ps = ptrs[i % NSETS]
        st = 0
        if ev is not None:  # events on the forward kernel's own dispatch
            st |= lib.bfly_time_next_forward(ev[0].cuda_event, ev[1].cuda_event)
        if from_angles:  # the call prepares the table into the workspace, then runs the kernel
            st |= lib.bfly_forward_quant(px, B.BFLY_BF16, py, B.BFLY_BF16, pc, ps, None, rows, n,
                                         th_p, None, bits, group, B.BFLY_SYM_ABSMAX, tab_p, tab_n,
                                         sh)
        else:  # the table bfly_prepare made once
            st |= lib.bfly_forward_quant(px, B.BFLY_BF16, py, B.BFLY_BF16, pc, ps, None, rows, n,
                                         None, tab_p, bits, group, B.BFLY_SYM_ABSMAX, None, 0, sh)
        if st:
            raise RuntimeError("libbfly call failed with status %d" % st)

    def step(i):
        # the whole path, angles in: one bfly_forward_quant call (the prepare
        # kernel, then the fused kernel)
        launch(i)

    def fixed(i):
        launch(i, from_angles=False)

    # 1. the timed steps (the headline value)
    warm_s = warm_up(torch, step, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_step / 1e3) / 1e9

    # 2. the fused kernel with the table made once (fixed angles, as at
    # inference), back to back: its average launch duration is the HIP event
    # pair around the timed launches on their stream, divided by their count
    # (at least 200, whatever --steps is).  This is the roofline's time.
    st = lib.bfly_prepare(th_p, n, tab_p, tab_n, sh)
    if st:
        raise RuntimeError("bfly_prepare failed with status %d" % st)
    nfixed = max(args.steps, 200)
    warm_up(torch, fixed, 20, min_seconds=0.1)
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(nfixed):
        fixed(i)
    region[1].record(stream)
    torch.cuda.synchronize()
    us_fixed = (time.perf_counter() - t0) * 1e6 / nfixed
    kern_avg_s = region[0].elapsed_time(region[1]) / 1e3 / nfixed

    # 3. each kernel's own duration: HIP events attached to its dispatch
    # (bfly_time_next_forward), KERNEL_TIMED_LAUNCHES launches rotating the
    # buffer sets, median and spread (reported beside the average; on some
    # boxes these read up to 10 % above the kernel trace while the average
    # agrees with it).  Recording each event once creates it.
    def kernel_times(from_angles):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(KERNEL_TIMED_LAUNCHES)]
        for e in evs:
            e[0].record(stream)
            e[1].record(stream)
        torch.cuda.synchronize()
        for i, e in enumerate(evs):
            launch(i, e, from_angles)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in evs])

    # the kernel as it runs back to back with its table made once: the same
    # kernel as in the step (the prepare launch ahead of it in a step only
    # moves the dispatch's start stamp)
    kern_ms = kernel_times(False)
    kern_med_s = float(np.median(kern_ms)) / 1e3
    achieved = kernel_bytes / kern_avg_s / 1e9
    copy_gbs = copy_context(torch, stream, kernel_bytes)
    traffic = recorded_traffic()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w["name"] + ": 8192 rows x n=4096, bf16 in, bf16 Q x out, "
                               "symmetric absmax INT4 codes per group of 128, fp16 scales; "
                               "a step = one bfly_forward_quant call from the angles (the "
                               "prepare kernel, then the fused kernel)",
                   "rows": rows, "n": n, "bits": bits, "group": group,
                   "bytes_per_step": step_bytes, "rows_per_s": round(rows / (ms_step / 1e3)),
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "table_made_once_us_per_launch": round(us_fixed, 3),
                   "table_made_once_GBs": round(kernel_bytes / (us_fixed / 1e6) / 1e9, 2),
                   "table_made_once_launches": nfixed,
                   "buffer_sets": NSETS, "warmup_s": round(warm_s, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "fwd_kernel<12,1,2,bf16,bf16 out,int4 g128> (bfly_forward_quant)",
                     "timed_launches": nfixed,
                     "kernel_avg_us": round(kern_avg_s * 1e6, 3),
                     "attached_events": {
                         "launches": len(kern_ms),
                         "median_us": round(kern_med_s * 1e6, 3),
                         "p10_us": round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
                         "p90_us": round(float(np.percentile(kern_ms, 90)) * 1e3, 3)},
                     "algorithmic_bytes_per_launch": kernel_bytes,
                     "copy_context": {"GBs": round(copy_gbs, 2),
                                      "kernel_frac_of_copy": round(achieved / copy_gbs, 4),
                                      "what": "torch device copy of the same bytes (half read, half "
                                              "written), 5 rotating buffer pairs, 200 copies "
                                              "between one event pair; context only"}},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_act(w, bytes_per_row, inputs)
    return out


# ---------------------------------------------------------------------------
# secondary workloads (reported on one line each, not the headline)
# ---------------------------------------------------------------------------

def time_loop(torch, fn, steps, warmup):
    warm_up(torch, fn, warmup)
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def bench_secondary(args, torch, B, inputs):
    name = args.workload
    res = {"workload": name}
    if name == "tiny_n256_fp32":
        w = inputs.tiny_fp32()
        x, y, th = to_dev(w["x"], torch), torch.empty((64, 256), device="cuda"), to_dev(w["theta"], torch)
        t = time_loop(torch, lambda i: B.bfly_forward(x, y, theta=th), args.steps, args.warmup)
        res.update(us_per_step=t * 1e6, bytes=64 * 256 * 8)
    elif name == "weight_n4096_bf16_int2":
        w = inputs.weight_int2()
        th = to_dev(w["theta"], torch)
        tab = torch.empty(B.bfly_coeff_bytes(4096), dtype=torch.uint8, device="cuda")
        sets = []  # 3 sets of both matrices (765 MB): no step finds its rows in cache
        for _ in range(3):
            mats = []
            for k in ("w1", "w2"):
                xw = to_dev(w[k], torch)
                r = xw.shape[0]
                mats.append((xw, torch.empty_like(xw), torch.empty((r, 1024), dtype=torch.uint8, device="cuda"),
                             torch.empty((r, 32), dtype=torch.float16, device="cuda"),
                             torch.empty((r, 32), dtype=torch.float16, device="cuda")))
            sets.append(mats)

        def fn(i):
            B.bfly_prepare(th, 4096, tab)
            for xw, yw, c, s, z in sets[i % 3]:
                B.bfly_forward_quant(xw, yw, c, s, z, coeffs=tab, bits=2, group=128, mode=1)
        t = time_loop(torch, fn, args.steps, args.warmup)
        rows = 4096 + 11008
        b = rows * (8192 + 8192 + 1024 + 128)
        res.update(us_per_step=t * 1e6, bytes=b, GBs=b / t / 1e9, rows_per_s=rows / t)
        # The same step with both matrices stored one after the other in one
        # allocation (rows are independent, so one call over the 15104 rows
        # gives the same outputs): one launch's start-up instead of two.
        del sets
        one = []
        for _ in range(3):
            xw = to_dev(np.concatenate([w["w1"], w["w2"]], axis=0), torch)
            one.append((xw, torch.empty_like(xw), torch.empty((rows, 1024), dtype=torch.uint8, device="cuda"),
                        torch.empty((rows, 32), dtype=torch.float16, device="cuda"),
                        torch.empty((rows, 32), dtype=torch.float16, device="cuda")))

        def fn_one(i):
            B.bfly_prepare(th, 4096, tab)
            xw, yw, c, s, z = one[i % 3]
            B.bfly_forward_quant(xw, yw, c, s, z, coeffs=tab, bits=2, group=128, mode=1)
        t1 = time_loop(torch, fn_one, args.steps, args.warmup)
        res.update(stacked_one_call_us_per_step=t1 * 1e6, stacked_one_call_GBs=b / t1 / 1e9)
    elif name == "kron_n5120_bf16_int4":
        w = inputs.kron_int4()
        th, mix = to_dev(w["theta_b"], torch), to_dev(w["mix"], torch)
        rows = w["x"].shape[0]
        sets = []  # 4 sets (720 MB): no step finds its rows in cache
        for _ in range(4):
            x = to_dev(w["x"], torch)
            sets.append((x, torch.empty_like(x), torch.empty((rows, 2560), dtype=torch.uint8, device="cuda"),
                         torch.empty((rows, 40), dtype=torch.float16, device="cuda")))
        tab = torch.empty(B.bfly_coeff_bytes(1024), dtype=torch.uint8, device="cuda")

        def fn(i):
            x, y, c, s = sets[i % 4]
            B.bfly_prepare(th, 1024, tab)
            B.bfly_kron_forward(x, y, mix, c, s, coeffs_b=tab, bits=4, group=128)
        t = time_loop(torch, fn, args.steps, args.warmup)
        b = rows * (10240 + 10240 + 2560 + 80)
        res.update(us_per_step=t * 1e6, bytes=b, GBs=b / t / 1e9, rows_per_s=rows / t)
    elif name == "hadamard_n4096_bf16_int4":
        # The headline batch through H_4096 (table from bfly_prepare_hadamard,
        # made once: a fixed transform) against the learned rotation through
        # the same fused kernel, its table also made once (inference after
        # calibration), and the learned step that prepares every time.
        w = inputs.act_int4()
        rows, n = w["x"].shape
        th = to_dev(w["theta"], torch)
        had = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
        lrn = torch.empty_like(had)
        B.bfly_prepare_hadamard(n, had)
        B.bfly_prepare(th, n, lrn)
        sets = []
        xd = to_dev(w["x"], torch)
        for k in range(NSETS):
            sets.append((xd if k == 0 else xd.clone(), torch.empty_like(xd),
                         torch.empty((rows, n // 2), dtype=torch.uint8, device="cuda"),
                         torch.empty((rows, n // 128), dtype=torch.float16, device="cuda")))

        def run(tab, prep):
            def fn(i):
                x, y, c, s = sets[i % NSETS]
                if prep:
                    B.bfly_prepare(th, n, tab)
                B.bfly_forward_quant(x, y, c, s, coeffs=tab, bits=4, group=128, mode=0)
            return fn
        b = rows * (2 * n + 2 * n + n // 2 + 2 * (n // 128))
        t_h = time_loop(torch, run(had, False), args.steps, args.warmup)
        t_l = time_loop(torch, run(lrn, False), args.steps, args.warmup)
        t_lp = time_loop(torch, run(lrn, True), args.steps, args.warmup)
        res.update(us_per_step=t_h * 1e6, bytes=b, GBs=b / t_h / 1e9, rows_per_s=rows / t_h,
                   learned_fixed_us_per_step=t_l * 1e6, learned_prepared_us_per_step=t_lp * 1e6,
                   learned_fixed_over_hadamard=t_l / t_h, learned_prepared_over_hadamard=t_lp / t_h)
    elif name == "w2a16_m8192_k4096_n11008":
        # The consumer of the quantized weights: y = (Q x)(W Q^T)^T for the
        # headline batch (8192 x 4096 bf16, rotated by the library) against
        # the 11008 x 4096 weight rotated and quantized to asym INT2 g128 by
        # the library; bf16 out.  One step = one bfly_quant_matmul.
        w = inputs.act_int4()
        ww = inputs.weight_int2()
        rows, k = w["x"].shape
        n_out = ww["w2"].shape[0]
        a = torch.empty((rows, k), dtype=torch.bfloat16, device="cuda")
        B.bfly_forward(to_dev(w["x"], torch), a, theta=to_dev(w["theta"], torch))
        w2 = to_dev(ww["w2"], torch)
        codes = torch.empty((n_out, k // 4), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n_out, k // 128), dtype=torch.float16, device="cuda")
        zr = torch.empty_like(sc)
        B.bfly_forward_quant(w2, None, codes, sc, zr, theta=to_dev(ww["theta"], torch), bits=2,
                             group=128, mode=B.BFLY_ASYM_MINMAX)
        del w2
        y = torch.empty((rows, n_out), dtype=torch.bfloat16, device="cuda")
        stream = torch.cuda.current_stream()

        def fn(i, ev=None):
            if ev is not None:
                ev[0].record(stream)
            B.bfly_quant_matmul(a, codes, sc, zr, y, bits=2, group=128, mode=B.BFLY_ASYM_MINMAX)
            if ev is not None:
                ev[1].record(stream)
        warm_up(torch, fn, args.warmup)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i, evs[i])
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / args.steps
        kern_s = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) / 1e3
        flops = 2.0 * rows * k * n_out
        hbm = rows * k * 2 + codes.numel() + 4 * sc.numel() + rows * n_out * 2
        res.update(us_per_step=t * 1e6, kernel_avg_us=kern_s * 1e6, flops=flops,
                   TFLOPs=flops / kern_s / 1e12, mfma_bf16_peak_TFLOPs=MFMA_BF16_PEAK_TFLOPS,
                   frac_of_mfma_peak=flops / kern_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                   hbm_bytes=hbm, GBs_hbm=hbm / kern_s / 1e9)
    elif name == "kron_n11008_bf16_int4":
        # O43 (x) B256 on 8192 bf16 rows, sym INT4 g128: the mix pass into an
        # fp32 workspace, then the fused butterfly + quantizer on the segments.
        w = inputs.kron_wide_int4()
        th, mix = to_dev(w["theta_b"], torch), to_dev(w["mix"], torch)
        rows, n, m, nb = w["rows"], w["n"], w["m"], w["nb"]
        sets = []  # 3 sets (700 MB) so no step finds its rows in cache
        for _ in range(3):
            x = to_dev(w["x"], torch)
            sets.append((x, torch.empty_like(x), torch.empty((rows, n // 2), dtype=torch.uint8, device="cuda"),
                         torch.empty((rows, n // 128), dtype=torch.float16, device="cuda")))
        ws = torch.empty(B.bfly_kron_forward_wide_workspace_bytes(rows, m, nb), dtype=torch.uint8,
                         device="cuda")
        tab = torch.empty(B.bfly_coeff_bytes(nb), dtype=torch.uint8, device="cuda")

        def fn(i):
            x, y, c, s = sets[i % 3]
            B.bfly_prepare(th, nb, tab)
            B.bfly_kron_forward_wide(x, y, mix, ws, c, s, coeffs_b=tab, bits=4, group=128)
        t = time_loop(torch, fn, args.steps, args.warmup)
        b = rows * (2 * n + 2 * n + n // 2 + 2 * (n // 128))
        res.update(us_per_step=t * 1e6, bytes=b, GBs=b / t / 1e9, rows_per_s=rows / t,
                   fp32_intermediate_bytes=rows * n * 8)
    elif name in ("w2a16_m1_k4096_n11008", "w2a16_m16_k4096_n11008"):
        # Decode-time W2A16: 1 or 16 activation rows against the 11008 x 4096
        # asym INT2 g128 weight (rotated and quantized by the library): the
        # product is bound by reading the codes, scales and zero points once.
        rows = 1 if name == "w2a16_m1_k4096_n11008" else 16
        ww = inputs.weight_int2()
        k, n_out = 4096, ww["w2"].shape[0]
        gen = torch.Generator(device="cuda").manual_seed(7)
        a = torch.randn((rows, k), device="cuda", generator=gen).to(torch.bfloat16)
        w2 = to_dev(ww["w2"], torch)
        sets = []  # 16 weight copies (210 MB): no launch finds its codes in cache
        codes = torch.empty((n_out, k // 4), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n_out, k // 128), dtype=torch.float16, device="cuda")
        zr = torch.empty_like(sc)
        B.bfly_forward_quant(w2, None, codes, sc, zr, theta=to_dev(ww["theta"], torch), bits=2,
                             group=128, mode=B.BFLY_ASYM_MINMAX)
        for _ in range(16):
            sets.append((codes.clone(), sc.clone(), zr.clone()))
        del w2
        y = torch.empty((rows, n_out), dtype=torch.bfloat16, device="cuda")
        stream = torch.cuda.current_stream()

        def fn(i, ev=None):
            c, s_, z = sets[i % 16]
            if ev is not None:
                ev[0].record(stream)
            B.bfly_quant_matmul(a, c, s_, z, y, bits=2, group=128, mode=B.BFLY_ASYM_MINMAX)
            if ev is not None:
                ev[1].record(stream)
        warm_up(torch, fn, args.warmup)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i, evs[i])
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / args.steps
        kern_s = float(np.median([e[0].elapsed_time(e[1]) for e in evs])) / 1e3
        hbm = codes.numel() + 4 * sc.numel() + rows * k * 2 + rows * n_out * 2
        res.update(us_per_step=t * 1e6, kernel_median_us=kern_s * 1e6, hbm_bytes=hbm,
                   GBs=hbm / kern_s / 1e9, flops=2.0 * rows * k * n_out)
    elif name == "kron_bwd_n5120_fp32":
        # Gradients of the composite O5 (x) B1024 on 32768 fp32 rows (x, G
        # drawn on the GPU from a seeded generator): dX and dtheta_b.
        w = inputs.kron_int4()
        rows, m, nb = 32768, 5, 1024
        gen = torch.Generator(device="cuda").manual_seed(5)
        X = torch.randn((rows, m * nb), device="cuda", generator=gen)
        G = torch.randn((rows, m * nb), device="cuda", generator=gen)
        dX = torch.empty_like(X)
        dth = torch.empty((10, 512), device="cuda")
        th, mix = to_dev(w["theta_b"], torch), to_dev(w["mix"], torch)
        ws = torch.empty(B.bfly_kron_backward_workspace_bytes(rows, m, nb), dtype=torch.uint8,
                         device="cuda")
        t = time_loop(torch, lambda i: B.bfly_kron_backward(X, G, dX, dth, mix, ws, theta_b=th),
                      args.steps, args.warmup)
        b = rows * m * nb * 12  # x and G read, dX written once
        res.update(us_per_step=t * 1e6, bytes=b, GBs=b / t / 1e9, rows_per_s=rows / t)
    elif name == "calib_step_n4096_fp32":
        # One calibration step (loss, dL/dY, backward, Adam) on the 262144
        # calibration rows of n = 4096 (128 samples x 2048 tokens).
        c = inputs.CalibFP32()
        X = torch.empty((c.rows, c.n), device="cuda")
        for r0, xb, _ in c.blocks(threads=16):
            X[r0:r0 + xb.shape[0]].copy_(torch.from_numpy(xb))
        th = to_dev(c.theta, torch)
        m, v = torch.zeros_like(th), torch.zeros_like(th)
        loss = torch.zeros(3, device="cuda")
        ws = torch.empty(B.bfly_calib_workspace_bytes(c.rows, c.n), dtype=torch.uint8, device="cuda")
        cfg = B.bfly_calib_config(4, 128, 16, 0.05, 1e-3, 0.9, 0.999, 1e-8)
        t = time_loop(torch, lambda i: B.bfly_calib_step(X, th, m, v, i + 1, cfg, loss, ws),
                      args.steps, args.warmup)
        passes = c.rows * c.n * 4 * 4  # X and Y (forward), Y (histogram), X (backward)
        res.update(us_per_step=t * 1e6, rows_per_s=c.rows / t, bytes_moved=passes,
                   GBs_moved=passes / t / 1e9, loss=[float(z) for z in loss.cpu()])
    elif name == "act_n8192_bf16_int4":
        # n = 8192 (two passes: the halves' 12 stages into an fp32 workspace,
        # then stage 12 with the bf16 output and the INT4 g128 quantizer) on
        # 4096 bf16 rows with outlier channels: the headline's bytes at twice
        # the width.  One step = one bfly_forward_quant call from the angles.
        rng = np.random.default_rng(7)
        n, rows = 8192, 4096
        th = to_dev(inputs.angles(rng, n), torch)
        cols = inputs.outlier_columns(rng, n)
        xh = inputs.activations(rng, rows, n, cols, "bf16")
        sets = []
        for _ in range(NSETS):
            x = to_dev(xh, torch)
            sets.append((x, torch.empty_like(x), torch.empty((rows, n // 2), dtype=torch.uint8, device="cuda"),
                         torch.empty((rows, n // 128), dtype=torch.float16, device="cuda")))
        ws = torch.empty(B.bfly_forward_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")

        def fn(i):
            x, y, c, sc = sets[i % NSETS]
            B.bfly_forward_quant(x, y, c, sc, theta=th, bits=4, group=128, mode=0, workspace=ws)
        t = time_loop(torch, fn, args.steps, args.warmup)
        b = rows * (2 * n + 2 * n + n // 2 + 2 * (n // 128))
        res.update(us_per_step=t * 1e6, bytes=b, GBs=b / t / 1e9, rows_per_s=rows / t,
                   fp32_intermediate_bytes=rows * n * 8)
    elif name == "calib_step_weight_n4096_out4096":
        # One layer-output calibration step on the 262144 calibration rows of
        # n = 4096 against the 4096 x 4096 weight of the weight workload (a
        # LLaMA-2-7B attention projection's shape), asym INT2 g128 (W2A16):
        # forward of X and of W's rows, the two fp32 products on the matrix
        # cores, the uniformity term, one backward, Adam.
        c = inputs.CalibFP32()
        X = torch.empty((c.rows, c.n), device="cuda")
        for r0, xb, _ in c.blocks(threads=16):
            X[r0:r0 + xb.shape[0]].copy_(torch.from_numpy(xb))
        ww = inputs.weight_int2()
        W = to_dev(ww["w1"], torch)
        out = W.shape[0]
        th = to_dev(c.theta, torch)
        m, v = torch.zeros_like(th), torch.zeros_like(th)
        loss = torch.zeros(3, device="cuda")
        ws = torch.empty(B.bfly_calib_step_weight_workspace_bytes(c.rows, out, c.n),
                         dtype=torch.uint8, device="cuda")
        cfg = B.bfly_calib_weight_config(2, 128, B.BFLY_ASYM_MINMAX, 16, 0.05, 1e-3, 0.9, 0.999,
                                         1e-8)
        t = time_loop(torch, lambda i: B.bfly_calib_step_weight(X, W, th, m, v, i + 1, cfg, loss,
                                                                 ws), args.steps, args.warmup)
        flops = 4.0 * c.rows * out * c.n  # R = Xr E^T and G = R E, 2 flops per multiply-add
        res.update(us_per_step=t * 1e6, rows_per_s=c.rows / t, out=out, product_flops=flops,
                   product_TFLOPs_at_step=flops / t / 1e12,
                   mfma_fp32_peak_TFLOPs=MFMA_FP32_PEAK_TFLOPS,
                   frac_of_fp32_mfma_peak_at_step=flops / t / 1e12 / MFMA_FP32_PEAK_TFLOPS,
                   loss=[float(z) for z in loss.cpu()])
    elif name == "calib_n4096_fp32_fwd_bwd":
        c = inputs.CalibFP32()
        X = torch.empty((c.rows, c.n), device="cuda")
        G = torch.empty((c.rows, c.n), device="cuda")
        for r0, xb, gb in c.blocks(threads=16):
            X[r0:r0 + xb.shape[0]].copy_(torch.from_numpy(xb))
            G[r0:r0 + gb.shape[0]].copy_(torch.from_numpy(gb))
        Y, dX = torch.empty_like(X), torch.empty_like(X)
        dth = torch.empty((12, 2048), device="cuda")
        th = to_dev(c.theta, torch)
        ws = torch.empty(B.bfly_backward_workspace_bytes(c.rows, c.n), dtype=torch.uint8, device="cuda")
        t = time_loop(torch, lambda i: B.bfly_backward(X, G, Y, dX, dth, ws, theta=th),
                      args.steps, args.warmup)
        b = c.rows * c.n * 16
        res.update(us_per_step=t * 1e6, bytes=b, GBs=b / t / 1e9, rows_per_s=c.rows / t)
        if not args.no_cpu_baseline:
            # the oracle's forward + backward (Y, dX, dtheta) on the first
            # block of rows with all host threads, median of 3: a bounded
            # sample of the workload, scaled to its rows
            import oracle
            xb = X[:4096].cpu().numpy()
            gb = G[:4096].cpu().numpy()
            thh = c.theta
            tc = _median_time(lambda: oracle.backward(xb, gb, thh), 3)
            res["cpu_baseline"] = {
                "kind": "oracle", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
                "nproc": os.cpu_count(), "sample_rows": 4096, "s_per_sample": round(tc, 3),
                "rows_per_s": round(4096 / tc), "GBs": round(4096 * c.n * 16 / tc / 1e9, 4),
                "full_workload_s_estimate": round(tc * c.rows / 4096, 1)}
    else:
        raise SystemExit("unknown workload %s" % name)
    if "GBs" in res:
        res["pct_of_hbm_peak"] = 100 * res["GBs"] / HBM_PEAK_GBS
    return res


def copy_probe(torch, steps):
    """A plain device-to-device copy of 256 MiB, for calibrating counters."""
    a = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": a.numel() * 4, "copy_probe_bytes_written": a.numel() * 4,
                      "launches": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="act_n4096_bf16_int4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (--gpus 1): the rotation is row-parallel, and "
              "runs on several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    import learnable_butterfly_rotation_amd as B
    from learnable_butterfly_rotation_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()
    if args.copy_probe:
        copy_probe(torch, args.steps)
        return
    if args.workload == "act_n4096_bf16_int4":
        print(json.dumps(bench_act(args, torch, B, inputs)))
    else:
        print(json.dumps(bench_secondary(args, torch, B, inputs)))


if __name__ == "__main__":
    main()
