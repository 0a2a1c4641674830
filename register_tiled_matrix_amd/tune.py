"""Micro-tile / occupancy sweep of the fp32 register-tiled kernel.

The trade the pages put at the centre of register tiling ("寄存器Tiling跨架构解析" sections 2.4,
6.2 and 7.1-7.4; "Understanding Register Tiling", the accounting of registers against reuse):
a bigger TM x TN micro-tile reads LDS less per FMA but holds more registers, so fewer waves
fit a SIMD, and past the register file the compiler spills. Every variant is the same kernel
source built with other compile-time values (F32_TM, F32_TN, F32_BK, F32_WAVES_PER_EU), so the
sweep measures the trade itself. The one-output-per-thread ablation is the LDS rung of the
ladder (algorithm 2).

    python -m register_tiled_matrix_amd.tune build            # CPU: compile every variant
    python -m register_tiled_matrix_amd.tune run  > sweep.jsonl   # GPU: time every variant
    python -m register_tiled_matrix_amd.tune report sweep.jsonl  # markdown summary

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

# name -> (TM, TN, BK, waves per SIMD requested)
VARIANTS = {}
for _bk in (8, 16, 32):
    for _w in (2, 3, 4):
        VARIANTS[f"8x8_bk{_bk}_w{_w}"] = (8, 8, _bk, _w)
    for _w in (1, 2):
        VARIANTS[f"8x16_bk{_bk}_w{_w}"] = (8, 16, _bk, _w)
for _bk in (8, 16):
    for _w in (1, 2):
        VARIANTS[f"16x8_bk{_bk}_w{_w}"] = (16, 8, _bk, _w)
for _bk in (16, 32):
    for _w in (2, 4, 8):
        VARIANTS[f"4x4_bk{_bk}_w{_w}"] = (4, 4, _bk, _w)
VARIANTS["8x16_bk16_w4"] = (8, 16, 16, 4)  # past the register file: the spill cliff

F32_SRC = "gemm_f32_regtile.hip"


def _variant_flags(tm, tn, bk, w):
    return [f"-DF32_TM={tm}", f"-DF32_TN={tn}", f"-DF32_BK={bk}", f"-DF32_WAVES_PER_EU={w}"]


def build_variant(name: str) -> dict:
    """Compile the fp32 kernel with the variant's values and link it with the default objects
    of every other translation unit (from the in-tree build)."""
    tm, tn, bk, w = VARIANTS[name]
    out = os.path.join(VARIANT_DIR, name)
    os.makedirs(out, exist_ok=True)
    obj, log = _build._compile(F32_SRC, _variant_flags(tm, tn, bk, w), out)
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


def cmd_report(args) -> int:
    rows = [json.loads(l) for l in open(args.jsonl) if l.strip().startswith("{")]
    out = ["# fp32 micro-tile / occupancy sweep", "",
           "Commands (repository root; the variants are built on the CPU first):", "", "```",
           "python -m register_tiled_matrix_amd.tune build",
           "python -m register_tiled_matrix_amd.tune run --workloads f32_4096,f32_tall > gpurun_out/sweep.jsonl",
           "python -m register_tiled_matrix_amd.tune report gpurun_out/sweep.jsonl", "```", "",
           "Each variant is the same kernel source with other compile-time values: micro-tile TM x TN "
           "per lane (workgroup tile 16TM x 16TN, 256 threads), slab depth BK, and the waves per SIMD "
           "requested from the compiler (`amdgpu_waves_per_eu`). VGPRs, scratch and occupancy are the "
           "compiler's own report. `exact` = output bitwise equal to the naive rung (fmaf over k in "
           "natural order). LDS floats read per FMA = (TM + TN) / (TM TN).", ""]
    for wl in dict.fromkeys(r["workload"] for r in rows):
        out += [f"## {wl}", "", "| variant | TM x TN | BK | VGPRs | scratch B/lane | waves/SIMD | LDS B | "
                "LDS floats/FMA | exact | mean ms | TFLOP/s |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in sorted((r for r in rows if r["workload"] == wl), key=lambda r: -r["tflops"]):
            name = r["variant"]
            if name in VARIANTS:
                tm, tn, bk, _ = VARIANTS[name]
                shape, bks, lf = f"{tm}x{tn}", str(bk), f"{(tm + tn) / (tm * tn):.3f}"
            else:
                shape, bks, lf = ("1x1", "32", "2.000") if "lds" in name else ("-", "-", "-")
            out.append(f"| {name} (`{r['kernel']}`) | {shape} | {bks} | {r.get('vgprs', '-')} | "
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
    r.add_argument("--steps", type=int, default=10)
    r.add_argument("--warmup", type=int, default=3)
    r.add_argument("--no-rungs", action="store_true",
                   help="time only the variants (for counter runs, where the default library's "
                        "kernels would share the variants' names)")
    rep = sub.add_parser("report")
    rep.add_argument("jsonl")
    rep.add_argument("--out", default="")
    args = p.parse_args(argv)
    root = _build.ROOT
    if root not in sys.path:
        sys.path.insert(0, root)
    t0 = time.time()
    rc = {"build": cmd_build, "run": cmd_run, "report": cmd_report}[args.cmd](args)
    print(f"# {args.cmd} done in {time.time() - t0:.1f} s", file=sys.stderr)
    return rc


if __name__ == "__main__":
    sys.exit(main())
