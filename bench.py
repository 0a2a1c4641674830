#!/usr/bin/env python3
"""Benchmark of the register-tiled GEMM library on one MI355X.

One step = one call of the hot path on one batch of synthetic input: the fp32 register-tiled
GEMM C = A @ B at M = N = K = 4096 (row-major, U[-1,1], alpha = 1, beta = 0), inputs
resident in HBM before the timed region. The same JSON line also carries the bf16 and fp16
MFMA paths at 8192^3 (A row-major, B column-major, N(0,1) rounded to the 16-bit type) and the
kernel ladder (naive -> LDS-tiled -> register-tiled -> MFMA), each timed the same way.

    python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--settle-ms 200] [--no-ladder] [--no-cpu]

Timing: untimed launches for --settle-ms of wall time (the clock ramps up over the first 20-50
large launches after idle; reported as clock_settle), W untimed warm-up steps, then the timed
region: K back-to-back steps between two
torch.cuda.synchronize() calls (wall clock -> ms_per_step and value; one HIP event pair
around the region -> back_to_back_ms_per_launch). A second pass of K launches puts a HIP
event pair around every launch on the stream the library launches on (the caller's current
stream) -> the average kernel duration used for the roofline figure, which is what the
rocprofv3 kernel trace reports per dispatch. The CPU baseline times the fp64 oracle as it stands
on a bounded row sample of the same workload, and a blocked multithreaded fp32 CPU GEMM
(cpu_baseline/) on the whole workload.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of FP32-vector / bf16-MFMA peak at M=N=K=4096/8192"


def _parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed launches before each timed region")
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="before each headline leg's warmup, untimed launches for at least this "
                        "long: after idle the GPU needs about 20 fp32 4096^3 or 50 bf16 8192^3 "
                        "launches to reach its steady clock (reported as clock_settle; 0 skips)")
    p.add_argument("--no-ladder", action="store_true", help="skip the naive/LDS rungs")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-bf16", action="store_true", help="skip the bf16 and fp16 8192^3 legs")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--only", choices=["f32_4096", "bf16_8192", "f16_8192", "f32_ragged",
                                      "f32_tall", "f32_256", "bf16_few", "copy"],
                   help="profiler mode: run just this workload's kernel (warmup + steps) and "
                        "print one summary line; 'copy' runs a plain 1 GiB device copy used to "
                        "calibrate the HBM byte counters")
    p.add_argument("--algo", type=int, default=0,
                   help="with --only: kernel ladder rung (the regtile_algo_f32 / _bf16 value; "
                        "0 = the default entry point)")
    return p.parse_args()


def _kernel_times(torch, fn, steps, warmup):
    """(wall ms per step, per-launch kernel ms from event pairs around each launch on the
    current stream, which is the stream every launch here goes to)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, [s.elapsed_time(e) for s, e in zip(starts, ends)]


def _time(torch, fn, steps, warmup):
    """(wall ms per step, mean per-launch kernel ms from event pairs, fastest launch ms)."""
    wall_ms, kern = _kernel_times(torch, fn, steps, warmup)
    return wall_ms, float(np.mean(kern)), float(np.min(kern))


def _settle(torch, fn, settle_ms):
    """Untimed launches for at least `settle_ms` of wall time (synchronising every 10 launches),
    so that a timed region that follows sees the steady clock. Returns {"ms", "launches"}."""
    n, t0 = 0, time.perf_counter()
    while settle_ms > 0 and (time.perf_counter() - t0) * 1e3 < settle_ms:
        fn()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "launches": n}


def _time_steps(torch, fn, steps, warmup):
    """The timed region of a leg: `steps` back-to-back launches bracketed by synchronisations
    (no per-launch events in between). Returns (wall ms per step, event ms per step from one
    event pair around the region), then a second pass with an event pair around every launch
    for the per-launch kernel duration: (mean, fastest) ms."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    region_ms = e0.elapsed_time(e1) / steps
    _, kern = _kernel_times(torch, fn, steps, 0)
    return wall_ms, region_ms, float(np.mean(kern)), float(np.min(kern))


def _steady_median(torch, step, with_region=False):
    """Median kernel time (ms) of 30 event-timed launches after warming up for at least 50
    launches and 100 ms (small problems ramp the clock slowly). With `with_region`, also the
    time per launch of 30 back-to-back launches inside one event pair (for kernels of tens of
    microseconds the per-launch event pair adds a few microseconds of its own)."""
    t_end, n = time.perf_counter() + 0.1, 0
    while n < 50 or time.perf_counter() < t_end:
        step()
        n += 1
        if n % 50 == 0:
            torch.cuda.synchronize()
    _, kern = _kernel_times(torch, step, 30, 0)
    if not with_region:
        return float(np.median(kern))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(30):
        step()
    e1.record()
    torch.cuda.synchronize()
    return float(np.median(kern)), e0.elapsed_time(e1) / 30


def _graph_ms_per_launch(torch, raw, call, rt, launches=20, replays=25):
    """Time per launch of `launches` identical calls captured in one HIP graph and replayed
    `replays` times inside one event pair (after warm-up replays). The library launches on the
    stream it is given and makes no allocation or synchronisation, so the calls capture as
    they are; the graph removes the host's per-launch cost, which dominates kernels of a few
    microseconds."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(launches):
            st = raw(*call[:-1], cap)
            if st:
                raise rt.RegtileError(st, rt.strerror(st))
    for _ in range(10):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * launches)
    del graph
    return ms


def _kernel_info(rt):
    """Resources of the kernel launched last, as the HIP runtime reports them."""
    try:
        return rt.last_kernel_info()
    except rt.RegtileError:
        return None


def _configs(torch, gi, rt, acc, dev, stream, with_16bit, with_cpu):
    """Every configuration through the default entry points: at least 50 warm-up launches and
    100 ms, then 30 timed launches; TFLOP/s from the median event time, and the fraction of the
    peak that bounds it. Then one more launch from the original C, compared in full with the
    fp64 oracle (max |err| / bound), and with `with_cpu` the oracle's and the blocked CPU GEMM's
    times on the same workload."""
    res = {}
    names = ["f32_256", "f32_4096", "f32_ragged", "f32_tall", "f32_8192"] + (["bf16_8192"] if with_16bit else [])
    for wname in names:
        wc = gi.WORKLOADS[wname]
        ic = gi.workload_inputs(wc)
        if wc.dtype == "f32":
            A = torch.from_numpy(ic.A).to(dev)
            B = torch.from_numpy(ic.B).to(dev)
            raw, ldb, peak = rt.gemm_f32_raw, wc.N, acc.PEAK_FP32_VECTOR_TFLOPS
        else:
            A = torch.from_numpy(ic.A.view(np.int16)).to(dev)
            B = torch.from_numpy(ic.B.view(np.int16)).to(dev)
            raw, ldb, peak = rt.gemm_bf16_raw, wc.K, acc.PEAK_BF16_MFMA_TFLOPS
        C = (torch.from_numpy(ic.C).to(dev) if ic.C is not None
             else torch.empty((wc.M, wc.N), dtype=torch.float32, device=dev))
        call = (wc.M, wc.N, wc.K, wc.alpha, A.data_ptr(), wc.K, B.data_ptr(), ldb, wc.beta,
                C.data_ptr(), wc.N, stream)

        def step(call=call, raw=raw):
            st = raw(*call)
            if st:
                raise rt.RegtileError(st, rt.strerror(st))

        step()
        kname = rt.last_kernel()
        info = _kernel_info(rt)
        med, region = _steady_median(torch, step, with_region=True)
        tf = wc.flop / (med * 1e-3) / 1e12
        tf_b2b = wc.flop / (region * 1e-3) / 1e12
        res[wname] = {"shape": [wc.M, wc.N, wc.K], "kernel": kname, "kernel_ms_median": round(med, 4),
                      "TFLOP/s": round(tf, 3), "peak": peak, "frac": round(tf / peak, 4),
                      "basis": "median of 30 launches, each timed by its own HIP event pair",
                      "back_to_back_ms_per_launch": round(region, 4),
                      "TFLOP/s_back_to_back": round(tf_b2b, 3), "frac_back_to_back": round(tf_b2b / peak, 4),
                      "kernel_resources": info, "counters": _sq_record(kname), "traffic": _traffic(kname)}
        if med < 0.1:  # launch-bound: also as launches replayed from a captured HIP graph
            gms = _graph_ms_per_launch(torch, raw, call, rt)
            tf_g = wc.flop / (gms * 1e-3) / 1e12
            res[wname].update({"graph_ms_per_launch": round(gms, 4), "TFLOP/s_graph": round(tf_g, 3),
                               "frac_graph": round(tf_g / peak, 4),
                               "graph_basis": "20 launches captured in one HIP graph, 25 replays in one event pair"})
        if with_cpu and wname != "f32_8192":  # the five configurations; 8192^3 fp32 is extra
            if ic.C is not None:
                C.copy_(torch.from_numpy(ic.C).to(dev))
            step()
            torch.cuda.synchronize()
            res[wname].update(_cpu_and_check(ic, C.cpu().numpy()))
        del A, B, C
    return res


def _cpu_and_check(inp, got):
    """The fp64 oracle on the whole workload (timed: the oracle CPU baseline), the GPU result's
    worst |err| / bound against it, and the blocked fp32 CPU GEMM on the same workload (16-bit
    operands widened to fp32 first, outside its timing)."""
    import cpu_baseline
    import gemm_inputs as gi
    import oracle

    t0 = time.perf_counter()
    ref, mag = oracle.gemm_inputs(inp)
    t_oracle = time.perf_counter() - t0
    ok, worst = oracle.check(got, ref, mag)
    del ref, mag
    if inp.dtype == "f32":
        A32, B32 = inp.A, inp.B
    else:
        def widen(bits):
            if inp.dtype == "bf16":
                return gi.bf16_bits_to_f32(bits)
            return np.ascontiguousarray(bits).view(np.float16).astype(np.float32)

        A32 = widen(inp.A)
        B32 = np.ascontiguousarray(widen(inp.B).T)  # N x K storage of column-major B -> K x N
    t0 = time.perf_counter()
    cpu_baseline.sgemm(A32, B32)
    t_blocked = time.perf_counter() - t0
    flop = 2.0 * inp.M * inp.N * inp.K
    return {"err_over_bound": round(worst, 4), "parity_ok": bool(ok),
            "cpu_oracle": {"seconds": round(t_oracle, 3), "TFLOP/s": round(flop / t_oracle / 1e12, 5),
                           "cores": oracle.num_threads(), "sample": "whole workload"},
            "cpu_blocked": {"seconds": round(t_blocked, 3), "TFLOP/s": round(flop / t_blocked / 1e12, 4),
                            "cores": cpu_baseline.num_threads(),
                            "sample": "whole workload" + ("" if inp.dtype == "f32" else
                                                          f", {inp.dtype} operands widened to fp32")}}


def _sources_digest(files):
    """Digest of the named kernel sources (register_tiled_matrix_amd/csrc)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "register_tiled_matrix_amd", "csrc")
    for name in files:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_name):
    """HBM bytes per launch of `kernel_name` from the committed rocprofv3 --pmc summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by its reading for a plain copy of known size),
    or None when absent or when the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get("kernels", {}).get(kernel_name)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    try:
        if rec.get("sources_digest") != _sources_digest(rec["sources"]):
            return None
    except (OSError, KeyError):
        return None
    return rec.get("hbm_bytes_per_launch")


def _sq_record(kernel_name):
    """LDS bank-conflict rate and wave-state shares of `kernel_name` from the committed
    rocprofv3 --pmc summary (profiles/sq_counters_bench_kernels.json), or None when absent or
    when the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "sq_counters_bench_kernels.json")
    try:
        with open(path) as f:
            rec = json.load(f).get("kernels", {}).get(kernel_name)
        if not rec or rec.get("sources_digest") != _sources_digest(rec["sources"]):
            return None
    except (OSError, ValueError, KeyError):
        return None
    return {k: rec[k] for k in ("lds_bank_conflict_rate", "valu_active_share", "waiting_share") if k in rec}


def _cpu_baseline(inp, target_s):
    """The fp64 oracle, as it stands, on the first R rows of the workload (R sized so the
    sample takes about target_s seconds); rate in TFLOP/s of the same 2*R*N*K flop count."""
    import oracle

    def run_rows(r):
        t0 = time.perf_counter()
        oracle.gemm(inp.A[:r], inp.B, None, alpha=inp.alpha, beta=0.0)
        return time.perf_counter() - t0

    r = 16
    dt = run_rows(r)
    while dt < 0.5 and r < inp.M:
        r = min(inp.M, r * 4)
        dt = run_rows(r)
    rate = r / dt
    rows = int(min(inp.M, max(r, rate * target_s)))
    if rows != r:
        dt = run_rows(rows)
    flop = 2.0 * rows * inp.N * inp.K
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {inp.M}x{inp.N}x{inp.K} fp32 workload "
                      f"({rows}x{inp.N}x{inp.K} fp64 multiply-adds, {dt:.1f} s)",
            "seconds": dt,
            "host_cpu": _cpu_model(),
            "host_cores_available": len(os.sched_getaffinity(0))}


def _cpu_blocked(inp):
    """The blocked multithreaded fp32 CPU GEMM on the whole workload (best of two runs)."""
    import cpu_baseline

    best = None
    for _ in range(2):
        t0 = time.perf_counter()
        cpu_baseline.sgemm(inp.A, inp.B)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    flop = 2.0 * inp.M * inp.N * inp.K
    return {"value": flop / best / 1e12, "unit": "TFLOP/s", "cores": cpu_baseline.num_threads(),
            "kind": "blocked fp32 (8x16 register micro-kernel, AVX2/FMA, OpenMP)",
            "sample": f"the whole {inp.M}x{inp.N}x{inp.K} fp32 workload, best of 2 ({best:.2f} s)",
            "seconds": best}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _only(args, torch, gi, rt, dev):
    """Run one workload's kernel alone (for rocprofv3 runs)."""
    if args.only == "copy":
        n = 1 << 28  # 2^28 floats = 1 GiB each way
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        wms, kms, _ = _time(torch, lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"only": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "kernel_ms_mean": kms}), flush=True)
        return 0
    w = gi.WORKLOADS[args.only]
    inp = gi.workload_inputs(w)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if w.dtype == "f32":
        A = torch.from_numpy(inp.A).to(dev)
        B = torch.from_numpy(inp.B).to(dev)
        fn = rt.gemm_f32_raw if args.algo == 0 else (
            lambda *a: rt.regtile_gemm_f32_algo(args.algo, *a))
    else:
        A = torch.from_numpy(inp.A.view(np.int16)).to(dev)
        B = torch.from_numpy(inp.B.view(np.int16)).to(dev)
        raw, algo_fn = ((rt.gemm_bf16_raw, rt.regtile_gemm_bf16_algo) if w.dtype == "bf16"
                        else (rt.gemm_f16_raw, rt.regtile_gemm_f16_algo))
        fn = raw if args.algo == 0 else (lambda *a: algo_fn(args.algo, *a))
    C = (torch.from_numpy(inp.C).to(dev) if inp.C is not None
         else torch.empty((w.M, w.N), dtype=torch.float32, device=dev))
    call = (w.M, w.N, w.K, w.alpha, A.data_ptr(), inp.lda, B.data_ptr(), inp.ldb, w.beta,
            C.data_ptr(), w.N, stream)

    def step():
        st = fn(*call)
        if st:
            raise rt.RegtileError(st, rt.strerror(st))

    wms, kms, kmin = _time(torch, step, args.steps, args.warmup)
    print(json.dumps({"only": args.only, "kernel": rt.last_kernel(), "kernel_resources": _kernel_info(rt),
                      "kernel_ms_mean": kms,
                      "kernel_ms_min": kmin, "TFLOP/s": w.flop / (kms * 1e-3) / 1e12}),
          flush=True)
    return 0


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import gemm_inputs as gi
    import register_tiled_matrix_amd as rt
    from register_tiled_matrix_amd import accounting as acc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    rt.load()  # raises RegtileLibraryMissing when the HIP library is not built
    dev = torch.device("cuda:0")
    if args.only:
        return _only(args, torch, gi, rt, dev)

    # ---- headline: fp32 register-tiled 4096^3 ----------------------------------------------
    w = gi.WORKLOADS["f32_4096"]
    inp = gi.workload_inputs(w)
    A = torch.from_numpy(inp.A).to(dev)
    B = torch.from_numpy(inp.B).to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    f32_args = (w.M, w.N, w.K, 1.0, A.data_ptr(), w.K, B.data_ptr(), w.N, 0.0, C.data_ptr(), w.N,
                stream)

    def step_f32():
        st = rt.gemm_f32_raw(*f32_args)
        if st:
            raise rt.RegtileError(st, rt.strerror(st))

    step_f32()
    kernel_name = rt.last_kernel()
    kernel_info = _kernel_info(rt)
    torch.cuda.synchronize()
    settle = _settle(torch, step_f32, args.settle_ms)
    wall_ms, region_ms, kern_ms, kern_min = _time_steps(torch, step_f32, args.steps, args.warmup)
    flop = w.flop
    value = flop / (wall_ms * 1e-3) / 1e12
    achieved = flop / (kern_ms * 1e-3) / 1e12
    work = acc.GemmWork(w.M, w.N, w.K, 4)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settle,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "f32_4096: fp32 GEMM M=N=K=4096, A and B row-major, "
                               "U[-1,1] seed 1002, alpha=1, beta=0",
                   "M": w.M, "N": w.N, "K": w.K, "kernel": kernel_name},
        "percent_of_fp32_vector_peak": round(100 * value / acc.PEAK_FP32_VECTOR_TFLOPS, 2),
        "roofline": {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": acc.PEAK_FP32_VECTOR_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / acc.PEAK_FP32_VECTOR_TFLOPS, 4),
            "frac_basis": "achieved = flop per launch / mean per-launch HIP event duration on the launch stream",
            "achieved_wall": round(value, 3),
            "frac_wall": round(value / acc.PEAK_FP32_VECTOR_TFLOPS, 4),
            "traffic": _traffic(kernel_name),
            "algorithmic_hbm_bytes": work.hbm_bytes,
            "kernel": kernel_name,
            "kernel_ms_mean": round(kern_ms, 4),
            "kernel_ms_min": round(kern_min, 4),
            "flop_per_launch": flop,
            "back_to_back_ms_per_launch": round(region_ms, 4),
            "kernel_resources": kernel_info,
            "counters": _sq_record(kernel_name),
        },
    }

    # ---- bf16 and fp16 MFMA 8192^3 ------------------------------------------------------------
    def leg_16b(wname, raw, algo_fn, label):
        wb = gi.WORKLOADS[wname]
        ib = gi.workload_inputs(wb)
        Ab = torch.from_numpy(ib.A.view(np.int16)).to(dev)
        Bb = torch.from_numpy(ib.B.view(np.int16)).to(dev)
        Cb = torch.empty((wb.M, wb.N), dtype=torch.float32, device=dev)
        bf_args = (wb.M, wb.N, wb.K, 1.0, Ab.data_ptr(), wb.K, Bb.data_ptr(), wb.K, 0.0,
                   Cb.data_ptr(), wb.N, stream)

        def step_16():
            st = raw(*bf_args)
            if st:
                raise rt.RegtileError(st, rt.strerror(st))

        step_16()
        kname = rt.last_kernel()
        kinfo = _kernel_info(rt)
        settle16 = _settle(torch, step_16, args.settle_ms)
        wms, rms, kms, kmin = _time_steps(torch, step_16, args.steps, args.warmup)
        v = wb.flop / (wms * 1e-3) / 1e12
        a = wb.flop / (kms * 1e-3) / 1e12
        res = {
            "value": round(v, 2), "unit": "TFLOP/s", "ms_per_step": round(wms, 4),
            "clock_settle": settle16,
            "dtype": f"{label} in, f32 accumulate",
            "workload": f"{wname}: {wb.description}, seed {wb.seed}, alpha=1, beta=0",
            "percent_of_mfma_peak": round(100 * v / acc.PEAK_BF16_MFMA_TFLOPS, 2),
            "roofline": {"bound": "mfma", "achieved": round(a, 2), "peak": acc.PEAK_BF16_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(a / acc.PEAK_BF16_MFMA_TFLOPS, 4),
                         "frac_basis": "achieved = flop per launch / mean per-launch HIP event duration",
                         "achieved_wall": round(v, 2), "frac_wall": round(v / acc.PEAK_BF16_MFMA_TFLOPS, 4),
                         "kernel_resources": kinfo, "counters": _sq_record(kname),
                         "traffic": _traffic(kname),
                         "algorithmic_hbm_bytes": acc.GemmWork(wb.M, wb.N, wb.K, 2).hbm_bytes,
                         "kernel": kname, "kernel_ms_mean": round(kms, 4),
                         "kernel_ms_min": round(kmin, 4), "flop_per_launch": wb.flop,
                         "back_to_back_ms_per_launch": round(rms, 4)},
        }

        # the same tiles and pipeline on 16x16x32 MFMA fragments (the fragment-shape rung)
        def step_16x16():
            st = algo_fn(rt.ALGO_BF16_MFMA_16X16, *bf_args)
            if st:
                raise rt.RegtileError(st, rt.strerror(st))

        step_16x16()
        k16 = rt.last_kernel()
        _, kms16, _ = _time(torch, step_16x16, args.steps, args.warmup)
        res["mfma_16x16x32"] = {"kernel": k16, "kernel_ms_mean": round(kms16, 4),
                                "TFLOP/s": round(wb.flop / (kms16 * 1e-3) / 1e12, 2)}
        del Ab, Bb, Cb
        return res

    if not args.no_bf16:
        out["bf16_8192"] = leg_16b("bf16_8192", rt.gemm_bf16_raw, rt.regtile_gemm_bf16_algo, "bf16")
        out["f16_8192"] = leg_16b("f16_8192", rt.gemm_f16_raw, rt.regtile_gemm_f16_algo, "fp16")

    # ---- operand layouts (BLAS transpose flags over row-major storage) ----------------------
    if not args.no_ladder:
        lay = {}
        for wname, ex in (("f32_4096", rt.regtile_gemm_f32_ex), ("bf16_8192", rt.regtile_gemm_bf16_ex)):
            wl = gi.WORKLOADS[wname]
            il = gi.workload_inputs(wl)
            if wl.dtype == "f32":
                Am = torch.from_numpy(il.A).to(dev)
                Bm = torch.from_numpy(il.B).to(dev)
            else:
                Am = torch.from_numpy(il.A.view(np.int16)).to(dev)
                Bm = torch.from_numpy(il.B.view(np.int16)).to(dev)
            Cm = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
            for ta in (0, 1):
                for tb in (0, 1):
                    # the same values in the requested storage (square problems: the transposed
                    # copy has the same leading dimension)
                    A_ = Am.t().contiguous() if ta else Am
                    B_ = Bm if (tb == 1) == (wl.dtype != "f32") else Bm.t().contiguous()
                    call = (0, ta, tb, wl.M, wl.N, wl.K, 1.0, A_.data_ptr(), wl.K, B_.data_ptr(),
                            wl.K, 0.0, Cm.data_ptr(), wl.N, stream)

                    def step_l(call=call, ex=ex):
                        st = ex(*call)
                        if st:
                            raise rt.RegtileError(st, rt.strerror(st))

                    step_l()
                    kms = _steady_median(torch, step_l)
                    code = ("n", "t")[ta] + ("n", "t")[tb]
                    lay[f"{wname}_{code}"] = {"kernel": rt.last_kernel(), "kernel_ms": round(kms, 4),
                                              "TFLOP/s": round(wl.flop / (kms * 1e-3) / 1e12, 2)}
                    del A_, B_
            del Am, Bm, Cm
        out["layouts"] = lay

    # ---- a bf16 problem of few output tiles: split-K inside the workgroup against the
    # LDS-DMA kernel (64 tiles of 128x128 for 256 CUs) --------------------------------------
    if not args.no_ladder and not args.no_bf16:
        wf = gi.WORKLOADS["bf16_few"]
        M_, N_, K_ = wf.M, wf.N, wf.K
        ift = gi.workload_inputs(wf)
        Af = torch.from_numpy(ift.A.view(np.int16)).to(dev)
        Bf = torch.from_numpy(ift.B.view(np.int16)).to(dev)  # stored N x K
        Cf = torch.empty((M_, N_), dtype=torch.float32, device=dev)
        few = {"shape": [M_, N_, K_]}
        for algo, label in ((rt.ALGO_BF16_AUTO, "default"), (rt.ALGO_BF16_MFMA, "lds_dma_kernel")):
            def step_f(algo=algo):
                st = rt.regtile_gemm_bf16_algo(algo, M_, N_, K_, 1.0, Af.data_ptr(), K_, Bf.data_ptr(), K_, 0.0,
                                               Cf.data_ptr(), N_, stream)
                if st:
                    raise rt.RegtileError(st, rt.strerror(st))

            step_f()
            kms = _steady_median(torch, step_f)
            few[label] = {"kernel": rt.last_kernel(), "kernel_ms": round(kms, 4),
                          "TFLOP/s": round(2.0 * M_ * N_ * K_ / (kms * 1e-3) / 1e12, 2)}
        out["bf16_few_tiles"] = few
        del Af, Bf, Cf

    # ---- the ladder on the headline workload ------------------------------------------------
    if not args.no_ladder:
        ladder = {}
        for algo, label in ((rt.ALGO_F32_NAIVE, "naive"), (rt.ALGO_F32_LDS, "lds_32x32"),
                            (rt.ALGO_F32_REGTILE, "regtile_8x16")):
            def step(algo=algo):
                st = rt.regtile_gemm_f32_algo(algo, *f32_args)
                if st:
                    raise rt.RegtileError(st, rt.strerror(st))
            if algo == rt.ALGO_F32_REGTILE:
                kms = _steady_median(torch, step)
            else:  # 9-31 ms per launch: three launches after one
                _, kms, _ = _time(torch, step, 3, 1)
            ladder[label] = {"kernel": rt.last_kernel(), "kernel_ms": round(kms, 4),
                             "TFLOP/s": round(flop / (kms * 1e-3) / 1e12, 3)}
        if "bf16_8192" in out:
            ladder["mfma_bf16_8192"] = {"kernel": out["bf16_8192"]["roofline"]["kernel"],
                                        "kernel_ms": out["bf16_8192"]["roofline"]["kernel_ms_mean"],
                                        "TFLOP/s": out["bf16_8192"]["roofline"]["achieved"]}
            ladder["mfma16_bf16_8192"] = {
                "kernel": out["bf16_8192"]["mfma_16x16x32"]["kernel"],
                "kernel_ms": out["bf16_8192"]["mfma_16x16x32"]["kernel_ms_mean"],
                "TFLOP/s": out["bf16_8192"]["mfma_16x16x32"]["TFLOP/s"]}
            ladder["mfma_f16_8192"] = {"kernel": out["f16_8192"]["roofline"]["kernel"],
                                       "kernel_ms": out["f16_8192"]["roofline"]["kernel_ms_mean"],
                                       "TFLOP/s": out["f16_8192"]["roofline"]["achieved"]}
        out["ladder"] = ladder

    # ---- every configuration, median of 30 launches ------------------------------------------
    out["configs"] = _configs(torch, gi, rt, acc, dev, stream, not args.no_bf16, not args.no_cpu)

    # ---- CPU baseline: the oracle on a bounded sample --------------------------------------
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(inp, args.cpu_seconds)
        out["cpu_blocked_gemm"] = _cpu_blocked(inp)
    else:
        out["cpu_baseline"] = None

    out["device"] = torch.cuda.get_device_name(dev)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
