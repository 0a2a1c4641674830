"""Micro-tile / occupancy sweep of the fp32 register-tiled kernel.

The trade the pages put at the centre of register tiling ("寄存器Tiling跨架构解析" sections 2.4,
6.2 and 7.1-7.4; "Understanding Register Tiling", the accounting of registers against reuse):
a bigger TM x TN micro-tile reads LDS less per FMA but holds more registers, so fewer waves
fit a SIMD, and past the register file the compiler spills. Every variant is the same kernel
source built with other compile-time values (F32_TM, F32_TN, F32_BK, F32_WAVES_PER_EU and the
LDS stage count F32_STAGES), so the sweep measures the trade itself. The one-output-per-thread ablation is the LDS rung of the
ladder (algorithm 2).

    python -m register_tiled_matrix_amd.tune build            # CPU: compile every variant
    python -m register_tiled_matrix_amd.tune run  > sweep.jsonl   # GPU: time every variant
    python -m register_tiled_matrix_amd.tune report sweep.jsonl  # markdown summary
    python -m register_tiled_matrix_amd.tune ladder > ladder.jsonl   # GPU: every rung, every config
    python -m register_tiled_matrix_amd.tune datadep              # GPU: bf16 rate against input data
    python -m register_tiled_matrix_amd.tune shapes               # GPU: fp32 / bf16 on more shapes

Correctness of each variant is checked bitwise against the naive rung of the default library:
every fp32 rung accumulates each output with fmaf over k in natural order, so any micro-tile
shape must reproduce it exactly.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import json
import os
import subprocess
import sys
import time

from . import build as _build

VARIANT_DIR = os.path.join(_build.BUILD_DIR, "variants")

# name -> (TM, TN, BK, waves per SIMD requested, LDS stages)
VARIANTS = {}
for _bk in (8, 16, 32):
    for _w in (2, 3, 4):
        VARIANTS[f"8x8_bk{_bk}_w{_w}"] = (8, 8, _bk, _w, 2)
    for _w in (1, 2):
        VARIANTS[f"8x16_bk{_bk}_w{_w}"] = (8, 16, _bk, _w, 2)
for _bk in (8, 16):
    for _w in (1, 2):
        VARIANTS[f"16x8_bk{_bk}_w{_w}"] = (16, 8, _bk, _w, 2)
for _bk in (16, 32):
    for _w in (2, 4, 8):
        VARIANTS[f"4x4_bk{_bk}_w{_w}"] = (4, 4, _bk, _w, 2)
VARIANTS["8x16_bk16_w4"] = (8, 16, 16, 4, 2)  # past the register file: the spill cliff
# LDS stages: one (two barriers per slab) and three, beside the default two
for _tm, _tn, _bk, _w in ((8, 16, 16, 2), (8, 16, 8, 2), (16, 8, 16, 2), (8, 8, 16, 2), (8, 8, 8, 4),
                          (4, 4, 32, 4)):
    for _st in (1, 3):
        VARIANTS[f"{_tm}x{_tn}_bk{_bk}_w{_w}_s{_st}"] = (_tm, _tn, _bk, _w, _st)

F32_SRC = "gemm_f32_regtile.hip"


def _variant_flags(tm, tn, bk, w, st):
    return [f"-DF32_TM={tm}", f"-DF32_TN={tn}", f"-DF32_BK={bk}", f"-DF32_WAVES_PER_EU={w}",
            f"-DF32_STAGES={st}"]


def build_variant(name: str) -> dict:
    """Compile the fp32 kernel with the variant's values and link it with the default objects
    of every other translation unit (from the in-tree build)."""
    out = os.path.join(VARIANT_DIR, name)
    os.makedirs(out, exist_ok=True)
    obj, log = _build._compile(F32_SRC, _variant_flags(*VARIANTS[name]), out)
    others = [os.path.join(_build.BUILD_DIR, s + ".o") for s in _build.SOURCES if s != F32_SRC]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the default library first (missing {missing[0]})")
    lib = os.path.join(out, "libregtile.so")
    r = subprocess.run([_build._hipcc(), f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", obj,
                        *others, "-o", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {name}:\n{r.stderr[-3000:]}")
    with open(os.path.join(out, "resource_usage.txt"), "w") as f:
        f.write(_build._resource_report([log]))
    return variant_resources(name)


def variant_resources(name: str) -> dict:
    """VGPRs, scratch, occupancy and LDS of the variant's fully aligned interior kernel."""
    res = _build.resource_usage(os.path.join(VARIANT_DIR, name))
    key = [k for k in res if "SquareCfgELb0ELb0ELb0ELb1ELb1ELb1EE" in k]
    r = res[key[0]] if key else {}
    return {"vgprs": r.get("VGPRs"), "agprs": r.get("AGPRs"), "scratch_bytes": r.get("ScratchSize [bytes/lane]"),
            "waves_per_simd": r.get("Occupancy [waves/SIMD]"), "lds_bytes": r.get("LDS Size [bytes/block]")}


def cmd_build(args) -> int:
    if not os.path.exists(_build.LIB):
        _build.build(verbose=True)
    names = args.variants.split(",") if args.variants else list(VARIANTS)
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for name, r in zip(names, ex.map(build_variant, names)):
            print(json.dumps({"variant": name, **r}), flush=True)
    return 0


def cmd_run(args) -> int:
    import numpy as np
    import torch

    import gemm_inputs as gi
    import register_tiled_matrix_amd as rt

    if not torch.cuda.is_available():
        print("tune run needs a GPU", file=sys.stderr)
        return 2
    rt.load()
    names = args.variants.split(",") if args.variants else [
        n for n in VARIANTS if os.path.exists(os.path.join(VARIANT_DIR, n, "libregtile.so"))]
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn, steps, warmup):
        # untimed launches for settle_ms of wall time first: after a kernel change or idle the
        # clock takes 20-50 large launches to reach its steady value, so without this the
        # variants timed first would run at a lower clock than the later ones
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        return float(np.mean(ms)), float(np.min(ms))

    for wl in args.workloads.split(","):
        w = gi.WORKLOADS[wl]
        inp = gi.workload_inputs(w)
        A = torch.from_numpy(inp.A).cuda()
        B = torch.from_numpy(inp.B).cuda()
        C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        ref = torch.empty_like(C)
        call = (w.M, w.N, w.K, 1.0, A.data_ptr(), inp.lda, B.data_ptr(), inp.ldb, 0.0)
        assert rt.regtile_gemm_f32_algo(rt.ALGO_F32_NAIVE, *call, ref.data_ptr(), w.N, stream) == 0
        torch.cuda.synchronize()
        rungs = [("ladder:naive", rt.ALGO_F32_NAIVE), ("ladder:lds_1x1", rt.ALGO_F32_LDS),
                 ("ladder:regtile_default", rt.ALGO_F32_REGTILE), ("ladder:regtile_small", rt.ALGO_F32_REGTILE_SMALL),
                 ("ladder:splitk", rt.ALGO_F32_SPLITK)]
        for label, algo in ([] if args.no_rungs else rungs):
            def fn(algo=algo):
                st = rt.regtile_gemm_f32_algo(algo, *call, C.data_ptr(), w.N, stream)
                if st:
                    raise rt.RegtileError(st, rt.strerror(st))
            fn()
            torch.cuda.synchronize()
            exact = bool(torch.equal(C, ref)) if algo != rt.ALGO_F32_SPLITK else None
            steps = 3 if algo in (rt.ALGO_F32_NAIVE, rt.ALGO_F32_LDS) else args.steps
            mean, mn = timed(fn, steps, 1)
            print(json.dumps({"workload": wl, "variant": label, "kernel": rt.last_kernel(),
                              "bitwise_equal_naive": exact, "ms_mean": round(mean, 4), "ms_min": round(mn, 4),
                              "tflops": round(w.flop / (mean * 1e-3) / 1e12, 2)}), flush=True)
        for name in names:
            lib = ctypes.CDLL(os.path.join(VARIANT_DIR, name, "libregtile.so"))
            f = lib.regtile_gemm_f32_algo
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                               ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            lib.regtile_last_kernel.restype = ctypes.c_char_p
            args_v = (rt.ALGO_F32_REGTILE, *call, C.data_ptr(), w.N, stream)

            def fn(f=f, args_v=args_v):
                st = f(*args_v)
                if st:
                    raise RuntimeError(f"variant call failed: {st}")
            C.fill_(float("nan"))
            fn()
            torch.cuda.synchronize()
            exact = bool(torch.equal(C, ref))
            mean, mn = timed(fn, args.steps, args.warmup)
            print(json.dumps({"workload": wl, "variant": name, "kernel": lib.regtile_last_kernel().decode(),
                              "bitwise_equal_naive": exact, "ms_mean": round(mean, 4), "ms_min": round(mn, 4),
                              "tflops": round(w.flop / (mean * 1e-3) / 1e12, 2), **variant_resources(name)}),
                  flush=True)
        del A, B, C, ref
    return 0


# every rung of the ladder, per element type: (label, algorithm value, kernel-name prefix in
# the compiler's resource report)
F32_RUNGS = [("naive", 1, "naive_kernelIfLb0ELb0E"), ("lds_32x32", 2, "f32_lds_kernel"),
             ("regtile_8x16", 3, "SquareCfgELb0ELb0E"), ("regtile_small_4x4", 5, "SmallCfgELb0ELb0E"),
             ("splitk", 4, {"splitk8_64x128": "SplitCfgILi8ELi8ELi16ELi8E", "splitk8_64x96": "SplitCfgILi8ELi8ELi12E",
                            "splitk8_64x64": "SplitCfgILi8ELi8ELi8ELi16E", "splitk4_64x64": "SplitCfgILi4ELi8ELi8ELi16E",
                            "splitk8_32x32": "SplitCfgILi8ELi4ELi4ELi16E"})]
R16_RUNGS = [("naive", 1, "naive_kernelI{T}Lb0ELb1E"), ("mfma_32x32x16", 2, "ELi32ELi1ELi1ELb{F}E"),
             ("mfma_16x16x32", 3, "ELi16ELi1ELi0ELb{F}E")]


def _rung_prefix(prefix, kernel_name: str) -> str:
    """A rung's mangled-name prefix; a dict maps a substring of the launched kernel's label
    to the prefix of that kernel (rungs that pick between kernel shapes)."""
    if isinstance(prefix, dict):
        return next(v for k, v in prefix.items() if k in kernel_name)
    return prefix


def _kernel_resources(prefix: str) -> dict:
    """Largest VGPR count, occupancy and LDS among the in-tree kernels whose mangled name
    contains `prefix` (all vector/edge variants of one rung)."""
    res = _build.resource_usage()
    hits = [r for k, r in res.items() if prefix in k]
    if not hits:
        return {}
    r = max(hits, key=lambda r: r.get("VGPRs", 0) + r.get("AGPRs", 0))
    return {"vgprs": r.get("VGPRs"), "agprs": r.get("AGPRs"), "scratch_bytes": r.get("ScratchSize [bytes/lane]"),
            "waves_per_simd": r.get("Occupancy [waves/SIMD]"), "lds_bytes": r.get("LDS Size [bytes/block]")}


def cmd_ladder(args) -> int:
    """Every rung on every workload: TFLOP/s plus the compiler's VGPRs / occupancy / LDS."""
    import numpy as np
    import torch

    import gemm_inputs as gi
    import register_tiled_matrix_amd as rt

    if not torch.cuda.is_available():
        print("tune ladder needs a GPU", file=sys.stderr)
        return 2
    rt.load()
    stream = torch.cuda.current_stream().cuda_stream
    for wl in args.workloads.split(","):
        w = gi.WORKLOADS[wl]
        inp = gi.workload_inputs(w)
        if w.dtype == "f32":
            A = torch.from_numpy(inp.A).cuda()
            B = torch.from_numpy(inp.B).cuda()
            rungs, fn = F32_RUNGS, rt.regtile_gemm_f32_algo
        else:
            A = torch.from_numpy(inp.A.view(np.int16)).cuda()
            B = torch.from_numpy(inp.B.view(np.int16)).cuda()
            T, F = ("DF16_", "1") if w.dtype == "f16" else ("t", "0")
            rungs = [(l, a, p.format(T=T, F=F)) for l, a, p in R16_RUNGS]
            fn = rt.regtile_gemm_bf16_algo if w.dtype == "bf16" else rt.regtile_gemm_f16_algo
        C = (torch.from_numpy(inp.C).cuda() if inp.C is not None
             else torch.empty((w.M, w.N), dtype=torch.float32, device="cuda"))
        for label, algo, prefix in rungs:
            call = (algo, w.M, w.N, w.K, w.alpha, A.data_ptr(), inp.lda, B.data_ptr(), inp.ldb, w.beta,
                    C.data_ptr(), w.N, stream)
            slow = label in ("naive", "lds_32x32") and w.flop > 1e11
            steps = 3 if slow else args.steps
            for _ in range(1 if slow else args.warmup):
                assert fn(*call) == 0
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record()
                fn(*call)
                b.record()
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            print(json.dumps({"workload": wl, "rung": label, "kernel": rt.last_kernel(),
                              "ms_median": round(ms, 4), "tflops": round(w.flop / (ms * 1e-3) / 1e12, 3),
                              **_kernel_resources(_rung_prefix(prefix, rt.last_kernel()))}), flush=True)
        del A, B, C
    return 0


def cmd_datadep(args) -> int:
    """bf16 8192^3 through the default entry point with four input data sets, interleaved: the
    clock, and so the rate, depends on how much the matrix unit's operands toggle."""
    import numpy as np
    import torch

    import gemm_inputs as gi
    import register_tiled_matrix_amd as rt

    if not torch.cuda.is_available():
        print("tune datadep needs a GPU", file=sys.stderr)
        return 2
    rt.load()
    stream = torch.cuda.current_stream().cuda_stream
    w = gi.WORKLOADS["bf16_8192"]
    inp = gi.workload_inputs(w)
    rng = np.random.Generator(np.random.PCG64(2024))

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()

    def ints():
        return gi.f32_to_bf16_bits(rng.integers(-2, 3, size=(w.M, w.K)).astype(np.float32))

    ones = np.full((w.M, w.K), 0x3F80, np.uint16)
    same = dev(ones)
    a_dev = dev(inp.A)
    sets = {"N(0,1) rounded to bf16 (the bench workload)": (a_dev, dev(inp.B)),
            "N(0,1), A and B one 128 MB buffer": (a_dev, a_dev),
            "integers in [-2, 2]": (dev(ints()), dev(ints())),
            "all ones": (dev(ones), dev(ones)),
            "all zeros": (dev(np.zeros_like(ones)), dev(np.zeros_like(ones))),
            "all ones, A and B one 128 MB buffer": (same, same)}
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

    def launcher(A, B):
        call = (w.M, w.N, w.K, 1.0, A.data_ptr(), w.K, B.data_ptr(), w.K, 0.0, C.data_ptr(), w.N, stream)
        return lambda: rt.gemm_bf16_raw(*call)

    fns = {k: launcher(*v) for k, v in sets.items()}
    first = next(iter(fns.values()))
    for _ in range(args.warmup):
        assert first() == 0
    times = {k: [] for k in fns}
    for _ in range(args.rounds):
        for k, fn in fns.items():
            for _ in range(10):
                assert fn() == 0
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            times[k] += [a.elapsed_time(b) for a, b in ev]
    print(f"kernel `{rt.last_kernel()}`; median of {args.rounds} interleaved rounds of {args.steps} launches "
          f"after {args.warmup} warm-up launches", flush=True)
    print("| A, B data | median ms | TFLOP/s |\n|---|---|---|")
    for k, ts in times.items():
        ms = float(np.median(ts))
        print(f"| {k} | {ms:.4f} | {w.flop / (ms * 1e-3) / 1e12:.0f} |", flush=True)
    return 0


SHAPES_F32 = [(4096, 4096, 4096), (8192, 8192, 8192), (1000, 1500, 777), (16384, 128, 4096), (256, 256, 256),
              (2048, 2048, 2048), (4096, 2048, 4096), (3072, 3072, 3072), (1024, 1024, 8192), (3000, 2000, 512),
              (8190, 8190, 1023), (512, 4096, 4096)]
SHAPES_16 = [(8192, 8192, 8192), (8000, 8000, 8192), (6000, 6000, 6000), (4096, 4096, 4096), (4000, 4000, 4000),
             (2048, 4096, 4096), (2048, 2048, 8192), (1536, 1536, 8192), (1024, 1024, 16384), (512, 512, 8192),
             (2048, 512, 4096), (1024, 8192, 8192), (3000, 5000, 2000),
             (8190, 8190, 8190)]


def cmd_shapes(args) -> int:
    """fp32 and bf16 through the default entry points (row-major A; B row-major for fp32,
    column-major for bf16) on shapes beyond the five workloads: kernel chosen, median time."""
    import numpy as np
    import torch

    import register_tiled_matrix_amd as rt

    if not torch.cuda.is_available():
        print("tune shapes needs a GPU", file=sys.stderr)
        return 2
    rt.load()
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda").manual_seed(0)
    print("| dtype | M x N x K | kernel | median ms | TFLOP/s | % of peak |\n|---|---|---|---|---|---|")
    for dtype, shapes in (("f32", SHAPES_F32), ("bf16", SHAPES_16)):
        for M, N, K in shapes:
            if dtype == "f32":
                A = torch.rand(M, K, device="cuda", generator=g) * 2 - 1
                B = torch.rand(K, N, device="cuda", generator=g) * 2 - 1
                call = (M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0)
                fn, peak = rt.gemm_f32_raw, 157.3
            else:
                A = torch.randn(M, K, device="cuda", generator=g).bfloat16()
                B = torch.randn(N, K, device="cuda", generator=g).bfloat16()  # column-major K x N
                call = (M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), K, 0.0)
                fn, peak = rt.gemm_bf16_raw, 2516.6
            C = torch.empty(M, N, device="cuda")
            launch = lambda: fn(*call, C.data_ptr(), N, stream)
            for _ in range(args.warmup):
                assert launch() == 0
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                a.record()
                launch()
                b.record()
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            print(f"| {dtype} | {M} x {N} x {K} | `{rt.last_kernel()}` | {ms:.4f} | {tf:.1f} | {100 * tf / peak:.1f} |",
                  flush=True)
            del A, B, C
    return 0


def _ladder_report(rows, src) -> str:
    out = ["# Kernel ladder on every configuration", "",
           "Command (repository root, one MI355X):", "", "```",
           f"python -m register_tiled_matrix_amd.tune ladder > {src}",
           f"python -m register_tiled_matrix_amd.tune report {src}", "```", "",
           "Median of 30 timed launches after 50 warm-up launches (3 timed after 1 for the naive "
           "and LDS rungs on the large problems), operands resident on the device. VGPRs / "
           "occupancy / LDS: the compiler's resource report for the kernel the rung launched "
           "(largest of its vector / edge variants).", "",
           "| workload | rung | kernel | median ms | TFLOP/s | VGPRs | AGPRs | waves/SIMD | LDS bytes |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['workload']} | {r['rung']} | `{r['kernel']}` | {r['ms_median']} | {r['tflops']} | "
                   f"{r.get('vgprs', '-')} | {r.get('agprs', '-')} | {r.get('waves_per_simd', '-')} | "
                   f"{r.get('lds_bytes', '-')} |")
    return "\n".join(out) + "\n"


def _workload_mn(wl: str):
    """(M, N) of a named workload, or (0, 0) when unknown."""
    try:
        import gemm_inputs as gi
        w = gi.WORKLOADS[wl]
        return w.M, w.N
    except (ImportError, KeyError):
        return 0, 0


def cmd_report(args) -> int:
    rows = [json.loads(l) for l in open(args.jsonl) if l.strip().startswith("{")]
    src = os.path.relpath(os.path.abspath(args.jsonl), _build.ROOT)
    if rows and "rung" in rows[0]:
        text = _ladder_report(rows, src)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        else:
            sys.stdout.write(text)
        return 0
    out = ["# fp32 micro-tile / occupancy sweep", "",
           "Commands (repository root; the variants are built on the CPU first):", "", "```",
           "python -m register_tiled_matrix_amd.tune build",
           "python -m register_tiled_matrix_amd.tune run --workloads "
           f"{','.join(dict.fromkeys(r['workload'] for r in rows))} > {src}",
           f"python -m register_tiled_matrix_amd.tune report {src}", "```", "",
           "Each variant is the same kernel source with other compile-time values: micro-tile TM x TN "
           "per lane (workgroup tile 16TM x 16TN, 256 threads), slab depth BK, the number of LDS stages "
           "(2: double-buffered; 1: one stage, two barriers per slab; 3: a slab is stored two slabs "
           "ahead of its stage's last reader), and the waves per SIMD requested from the compiler "
           "(`amdgpu_waves_per_eu`). `tiles` is the workload's workgroup count. VGPRs, scratch and "
           "occupancy are the "
           "compiler's own report. `exact` = output bitwise equal to the naive rung (fmaf over k in "
           "natural order). LDS floats read per FMA = (TM + TN) / (TM TN). Each variant is timed "
           "after 150 ms of untimed launches (so that every variant runs at the steady clock) and 3 "
           "warm-up launches: mean of 20 launches, each timed by its own HIP event pair.", ""]
    for wl in dict.fromkeys(r["workload"] for r in rows):
        out += [f"## {wl}", "", "| variant | TM x TN | BK | stages | tiles | VGPRs | scratch B/lane | "
                "waves/SIMD | LDS B | LDS floats/FMA | exact | mean ms | TFLOP/s |",
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        wm, wn = _workload_mn(wl)
        for r in sorted((r for r in rows if r["workload"] == wl), key=lambda r: -r["tflops"]):
            name = r["variant"]
            if name in VARIANTS:
                tm, tn, bk, _, st = VARIANTS[name]
                shape, bks, lf = f"{tm}x{tn}", str(bk), f"{(tm + tn) / (tm * tn):.3f}"
                sts = str(st)
                tiles = str(-(-wm // (16 * tm)) * -(-wn // (16 * tn))) if wm else "-"
            else:
                shape, bks, lf = ("1x1", "32", "2.000") if "lds" in name else ("-", "-", "-")
                sts, tiles = "-", "-"
            out.append(f"| {name} (`{r['kernel']}`) | {shape} | {bks} | {sts} | {tiles} | {r.get('vgprs', '-')} | "
                       f"{r.get('scratch_bytes', '-')} | {r.get('waves_per_simd', '-')} | {r.get('lds_bytes', '-')} | "
                       f"{lf} | {r['bitwise_equal_naive']} | {r['ms_mean']} | {r['tflops']} |")
        out.append("")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)
    return 0


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = p.add_subparsers(dest="cmd", required=True)
    b = sub.add_parser("build")
    b.add_argument("--variants", default="")
    r = sub.add_parser("run")
    r.add_argument("--variants", default="")
    r.add_argument("--workloads", default="f32_4096,f32_tall")
    r.add_argument("--steps", type=int, default=20)
    r.add_argument("--warmup", type=int, default=3)
    r.add_argument("--settle-ms", type=float, default=150.0,
                   help="untimed launches for this long before each variant's warm-up")
    r.add_argument("--no-rungs", action="store_true",
                   help="time only the variants (for counter runs, where the default library's "
                        "kernels would share the variants' names)")
    lad = sub.add_parser("ladder")
    lad.add_argument("--workloads", default="f32_256,f32_4096,f32_ragged,f32_tall,bf16_8192,f16_8192")
    lad.add_argument("--steps", type=int, default=30)
    lad.add_argument("--warmup", type=int, default=50)
    sh = sub.add_parser("shapes", help="fp32 and bf16 default entry points on more shapes")
    sh.add_argument("--steps", type=int, default=20)
    sh.add_argument("--warmup", type=int, default=40)
    dd = sub.add_parser("datadep", help="bf16 8192^3 rate against the operands' data")
    dd.add_argument("--steps", type=int, default=20)
    dd.add_argument("--rounds", type=int, default=4)
    dd.add_argument("--warmup", type=int, default=80)
    rep = sub.add_parser("report")
    rep.add_argument("jsonl")
    rep.add_argument("--out", default="")
    args = p.parse_args(argv)
    root = _build.ROOT
    if root not in sys.path:
        sys.path.insert(0, root)
    t0 = time.time()
    rc = {"build": cmd_build, "run": cmd_run, "ladder": cmd_ladder, "report": cmd_report,
          "datadep": cmd_datadep, "shapes": cmd_shapes}[args.cmd](args)
    print(f"# {args.cmd} done in {time.time() - t0:.1f} s", file=sys.stderr)
    return rc


if __name__ == "__main__":
    sys.exit(main())
