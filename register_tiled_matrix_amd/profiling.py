"""rocprofv3 evidence for the benchmark's kernels: collect on the GPU, summarise on the CPU.

    python -m register_tiled_matrix_amd.profiling collect OUT/prof    # on the MI355X
    python -m register_tiled_matrix_amd.profiling summarize OUT/prof  # writes profiles/

`collect` runs each profiler pass as a child process (rocprofv3 starts the program itself;
this process never touches the GPU), one pass at a time, each under its own time limit, and
stops at the first pass that fails. The passes:

  trace_*    --kernel-trace --stats over `bench.py --only <workload>`, one workload per run
             (per-dispatch durations of that workload's kernel alone);
  pmc_*      FETCH_SIZE, then WRITE_SIZE, one counter per run, over `bench.py --only <workload>`
             for the fp32 4096^3, bf16 8192^3 and fp32 16384x128x4096 kernels and for a plain
             1 GiB device copy (the calibration: bytes moved / counter bytes);
  sq_*       LDS, VALU and MFMA instruction and cycle counters per kernel;
  state_*    where the waves' time goes (VALU / LDS / VMEM issue, waiting) per kernel;
  clock_*    the shader clock and the MFMA busy share per dispatch of the fp32 4096^3 and bf16
             8192^3 kernels in the benchmark's own launch sequence;
  clock_datadep  the shader clock and MFMA busy share of the bf16 kernel on six input data
             sets (tune datadep).

`summarize` turns the CSV files into the short tables under profiles/ and writes
profiles/pmc_traffic.json, from which bench.py reports `roofline.traffic` (HBM bytes per
launch), stamped with a digest of the kernel's sources so a changed kernel reports null.
"""
from __future__ import annotations

import csv
import collections
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "register_tiled_matrix_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

SQ_COUNTERS = ("SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_INSTS_VALU SQ_INSTS_MFMA "
               "SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES")
LADDER_COUNTERS = "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_INSTS_VALU SQ_INSTS_MFMA SQ_WAVES"
# where the waves' time goes: issuing VALU / LDS / VMEM instructions, or waiting (any counter or
# barrier), against the waves' lifetime
STATE_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM "
                  "SQ_WAVES")
COPY_BYTES = 1 << 30
# the shader clock and the MFMA pipes' busy share per dispatch, for the same bf16 kernel on
# different input data (tune datadep)
CLOCK_COUNTERS = "GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES"
CLOCK_WORKLOADS = ["f32_4096", "bf16_8192"]
CLOCK_STEPS, CLOCK_WARMUP = 20, 30
DD_STEPS, DD_ROUNDS, DD_WARMUP = 10, 2, 20
N_XCD, N_SIMD = 8, 1024

# workload -> (kernel label as regtile_last_kernel() names it, substring of the kernel's symbol,
#              sources whose digest stamps the record, algorithmic HBM bytes per launch)
KERNELS = {
    "f32_4096": ("f32_regtile_128x256x16_8x16_va_vb_vc", "f32_regtile_kernel<regtile::(anonymous namespace)::SquareCfg",
                 ["gemm_f32_regtile.hip", "regtile_internal.h"], 3 * 4096 * 4096 * 4),
    "bf16_8192": ("bf16_mfma32x32x16_dma_256x256x64_w2x2", "bf16_mfma_dma_kernel<256, 256, 64, 2, 2, 32",
                  ["gemm_bf16_mfma_dma.hip", "mfma_common.h", "tile_addressing.h", "regtile_internal.h"],
                  2 * 8192 * 8192 * 2 + 8192 * 8192 * 4),
    "f32_tall": ("f32_regtile_splitk8_64x128x8_8x16", "SplitCfg<8, 8, 16, 8, 1, 4>, false",
                 ["gemm_f32_splitk.hip", "regtile_internal.h"], (16384 * 4096 + 4096 * 128 + 16384 * 128) * 4),
    # beta != 0: C is read and written
    "f32_ragged": ("f32_regtile_splitk8_64x96x8_8x12_guard", "SplitCfg<8, 8, 12, 8, 1, 4>, true",
                   ["gemm_f32_splitk.hip", "regtile_internal.h"], (1000 * 777 + 777 * 1500 + 2 * 1000 * 1500) * 4),
}
PMC_WORKLOADS = ["f32_4096", "bf16_8192", "f32_tall", "f32_ragged", "copy"]
# one kernel trace per workload, so that each summary's statistics are that workload's alone
TRACE_WORKLOADS = ["f32_4096", "bf16_8192", "f32_tall", "f32_ragged", "bf16_few"]
TRACE_STEPS, TRACE_WARMUP = 200, 50
SQ_WORKLOADS = ["f32_4096", "bf16_8192", "f32_tall", "f32_ragged"]


def _bench_cmd(*extra):
    return ["python3", os.path.join(ROOT, "bench.py"), *extra]


def passes(out):
    """(name, rocprofv3 argv, seconds allowed) for every pass, in order."""
    p = [(f"trace_{w}", ["rocprofv3", "--kernel-trace", "--stats", "-d", os.path.join(out, f"trace_{w}"), "-o",
                         "trace", "--output-format", "csv", "--",
                         *_bench_cmd("--only", w, "--steps", str(TRACE_STEPS), "--warmup", str(TRACE_WARMUP))], 300)
         for w in TRACE_WORKLOADS]
    for w in PMC_WORKLOADS:
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            p.append((f"pmc_{c}_{w}", ["rocprofv3", "--pmc", c, "-d", os.path.join(out, f"pmc_{c}_{w}"), "-o", "pmc",
                                       "--output-format", "csv", "--",
                                       *_bench_cmd("--only", w, "--steps", "3", "--warmup", "1")], 120))
    for w in SQ_WORKLOADS:
        p.append((f"sq_{w}", ["rocprofv3", "--pmc", *SQ_COUNTERS.split(), "-d", os.path.join(out, f"sq_{w}"), "-o", "sq",
                              "--output-format", "csv", "--",
                              *_bench_cmd("--only", w, "--steps", "3", "--warmup", "1")], 120))
    for w in SQ_WORKLOADS:
        p.append((f"state_{w}", ["rocprofv3", "--pmc", *STATE_COUNTERS.split(), "-d", os.path.join(out, f"state_{w}"),
                                 "-o", "st", "--output-format", "csv", "--",
                                 *_bench_cmd("--only", w, "--steps", "3", "--warmup", "1")], 120))
    for w in CLOCK_WORKLOADS:
        p.append((f"clock_{w}", ["rocprofv3", "--kernel-trace", "--pmc", *CLOCK_COUNTERS.split(), "-d",
                                 os.path.join(out, f"clock_{w}"), "-o", "clk", "--output-format", "csv", "--",
                                 *_bench_cmd("--only", w, "--steps", str(CLOCK_STEPS), "--warmup", str(CLOCK_WARMUP))],
                  180))
    p.append(("clock_datadep", ["rocprofv3", "--kernel-trace", "--pmc", *CLOCK_COUNTERS.split(), "-d",
                                 os.path.join(out, "clock_datadep"), "-o", "clk", "--output-format", "csv", "--",
                                 "python3", "-m", "register_tiled_matrix_amd.tune", "datadep",
                                 "--steps", str(DD_STEPS), "--rounds", str(DD_ROUNDS), "--warmup", str(DD_WARMUP)], 300))
    p.append(("sq_ladder", ["rocprofv3", "--pmc", *LADDER_COUNTERS.split(), "-d", os.path.join(out, "sq_ladder"),
                            "-o", "sq", "--output-format", "csv", "--", "python3", "-m",
                            "register_tiled_matrix_amd.tune", "ladder", "--workloads", "f32_4096,bf16_8192",
                            "--steps", "2", "--warmup", "1"], 300))
    return p


def _display(argv, prof):
    """A pass's command as the profiles print it: every path relative to the repository root."""
    return " ".join(argv).replace(prof, os.path.relpath(prof, ROOT)).replace(ROOT + os.sep, "")


def collect(out, only=None) -> int:
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT)
    for name, argv, limit in passes(out):
        if only and name not in only:
            continue
        print(f"== {name}", flush=True)
        t0 = time.time()
        with open(os.path.join(out, name + ".out"), "w") as log:
            try:
                rc = subprocess.run(argv, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT,
                                    timeout=limit).returncode
            except subprocess.TimeoutExpired:
                print(f"{name}: time limit {limit} s reached; stopping", flush=True)
                return 124
        print(f"{name}: rc={rc} in {time.time() - t0:.1f} s", flush=True)
        if rc != 0:
            return rc
    return 0


# ---- summaries ------------------------------------------------------------------------------

def _digest(files):
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _pmc(path):
    agg = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            agg[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return agg


def _mean_for(prof, dirname, prefix, sub):
    d = _pmc(os.path.join(prof, dirname, prefix + "_counter_collection.csv"))
    vals = [v for (k, _), vs in d.items() if sub in k for v in vs]
    if not vals:
        raise KeyError(f"no dispatch of '{sub}' in {dirname}")
    return sum(vals) / len(vals), len(vals)


def _cmd_block(cmds):
    return ["Commands (repository root; `cd /tmp && export TMPDIR=/tmp` first):", "", "```", *cmds, "```", ""]


LDS_PER_CU = 160 * 1024


def _resource_rows(trace_csv):
    """Per-kernel resources as the kernel trace records them for each dispatch, and the waves
    per SIMD they allow. rocprofv3's VGPR_Count on gfx950 is the descriptor's granulated
    register count times 4, half the unified (VGPR + AGPR) registers allocated in granules of 8:
    it reads 116 for a kernel of 228 VGPRs (232 allocated) and 256 for 256 VGPRs + 256 AGPRs."""
    seen = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if "regtile::" in r["Kernel_Name"] and r["Kernel_Name"] not in seen:
                seen[r["Kernel_Name"]] = r
    out = ["", "Resources per dispatch as the same trace records them (LDS bytes per workgroup, scratch "
                "bytes per lane, `VGPR_Count` as rocprofv3 reports it; allocated registers = 2 x that, "
                "see the note in `profiling.py`). Waves per SIMD = min(512 / allocated registers, "
                "workgroups per CU that fit the 160 KiB LDS x waves per workgroup / 4).", "",
           "| kernel | workgroup | LDS bytes | scratch | VGPR_Count | allocated registers | waves per SIMD |",
           "|---|---|---|---|---|---|---|"]
    for name, r in seen.items():
        lds, vg, wg = int(r["LDS_Block_Size"]), int(r["VGPR_Count"]), int(r["Workgroup_Size_X"])
        alloc = 2 * vg
        by_regs = min(8, 512 // max(alloc, 1))
        wpw = max(1, wg // 64)
        by_lds = (LDS_PER_CU // lds) * wpw / 4 if lds else 8
        waves = min(by_regs, by_lds)
        short = name.replace("void ", "").replace("regtile::(anonymous namespace)::", "").replace("regtile::", "")
        short = short.split("(int")[0]
        out.append(f"| `{short}` | {wg} | {lds} | {r['Scratch_Size']} | {vg} | {alloc} | {waves:g} |")
    return out


def summarize_trace(prof, workload, out_md):
    """Kernel trace of `bench.py --only <workload>`: the workload's kernel, its statistics over
    every dispatch (warm-up included) and over the timed launches alone (the last TRACE_STEPS),
    the roofline fraction each gives, and the same run's HIP-event mean."""
    d = os.path.join(prof, f"trace_{workload}")
    with open(os.path.join(d, "trace_kernel_stats.csv")) as f:
        rows = [r for r in csv.DictReader(f) if "regtile::" in r["Name"]]
    durs = collections.defaultdict(list)
    with open(os.path.join(d, "trace_kernel_trace.csv")) as f:
        recs = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    for r in recs:
        durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    only = None
    with open(os.path.join(prof, f"trace_{workload}.out")) as f:
        for line in f:
            if line.startswith("{") and '"only"' in line:
                only = json.loads(line)
    import gemm_inputs as gi
    from . import accounting as acc

    w = gi.WORKLOADS[workload]
    peak = acc.PEAK_FP32_VECTOR_TFLOPS if w.dtype == "f32" else acc.PEAK_BF16_MFMA_TFLOPS
    argv = [a for n, a, _ in passes(prof) if n == f"trace_{workload}"][0]
    lines = [f"# Kernel trace: {workload} ({w.description}), rocprofv3 --kernel-trace --stats", ""]
    lines += _cmd_block([_display(argv, prof)])
    lines += [f"The run makes {TRACE_WARMUP} warm-up launches, then {TRACE_STEPS} timed launches, each with a HIP "
              f"event pair (the bench's per-launch timing). Algorithmic work {w.flop:.4g} flop per launch; "
              f"peak {peak} TFLOP/s.", "",
              "| kernel | calls | average (us) | min (us) | max (us) | timed launches: mean (us) | median (us) | "
              "TFLOP/s (timed mean) | frac |", "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        ds = durs.get(r["Name"], [])
        timed = ds[-TRACE_STEPS:]
        mean_t = statistics.mean(timed) if timed else float("nan")
        tf = w.flop / (mean_t * 1e-6) / 1e12 if timed else float("nan")
        lines.append(f"| `{_short_kernel(r['Name'])[:140]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {mean_t:.1f} | "
                     f"{statistics.median(timed) if timed else float('nan'):.1f} | {tf:.1f} | {tf / peak:.4f} |")
    if only:
        lines += ["", f"The same run's HIP-event mean over the timed launches: {only['kernel_ms_mean'] * 1e3:.1f} us "
                      f"({only['TFLOP/s']:.1f} TFLOP/s, frac {only['TFLOP/s'] / peak:.4f}); kernel `{only['kernel']}`; "
                      f"resources {json.dumps(only.get('kernel_resources'))}."]
    lines += _resource_rows(os.path.join(d, "trace_kernel_trace.csv"))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_traffic(prof, out_json, out_md):
    cf, _ = _mean_for(prof, "pmc_FETCH_SIZE_copy", "pmc", "copyBuffer")
    cw, _ = _mean_for(prof, "pmc_WRITE_SIZE_copy", "pmc", "copyBuffer")
    fs, ws = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    res = {"about": "HBM-side bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, "
                    "KiB per dispatch), each scaled by the reading of the same counter for a plain 1 GiB "
                    "device copy (copy bytes / counter bytes).",
           "calibration": {"kernel": "__amd_rocclr_copyBuffer", "bytes_each_way": COPY_BYTES,
                           "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw, "fetch_scale": fs, "write_scale": ws},
           "kernels": {}}
    cmds = [_display(a, prof) for n, a, _ in passes(prof) if n.startswith("pmc_")]
    md = ["# HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)", ""] + _cmd_block(cmds)
    md += [f"Calibration: a 1 GiB copy reads FETCH_SIZE = {cf:.0f} KiB and WRITE_SIZE = {cw:.0f} KiB, so fetch "
           f"counts are scaled by {fs:.3f} and write counts by {ws:.3f}.", "",
           "| workload | kernel | FETCH_SIZE KiB (mean of dispatches) | WRITE_SIZE KiB | HBM bytes per launch "
           "(scaled) | algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|"]
    for w, (label, sub, sources, alg) in KERNELS.items():
        f, nf = _mean_for(prof, f"pmc_FETCH_SIZE_{w}", "pmc", sub)
        wr, nw = _mean_for(prof, f"pmc_WRITE_SIZE_{w}", "pmc", sub)
        tb = f * 1024 * fs + wr * 1024 * ws
        res["kernels"][label] = {"workload": w, "sources": sources, "sources_digest": _digest(sources),
                                 "FETCH_SIZE_KiB": f, "WRITE_SIZE_KiB": wr, "hbm_bytes_per_launch": int(tb),
                                 "algorithmic_bytes": alg, "dispatches": [nf, nw]}
        md.append(f"| {w} | `{label}` | {f:.0f} | {wr:.0f} | {tb / 1e6:.1f} MB | {alg / 1e6:.1f} MB | {tb / alg:.2f} |")
    md += ["", "Traffic above the algorithmic bytes is operand panels fetched again by different XCDs (each has "
               "its own L2) and re-fetched after eviction; the MALL (Infinity Cache) serves part of it."]
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")


def _kernel_means(path, sub):
    d = _pmc(path)
    vals = collections.defaultdict(list)
    for (k, c), vs in d.items():
        if sub in k:
            vals[c].extend(vs)
    return {c: sum(vs) / len(vs) for c, vs in vals.items()}


def summarize_sq(prof, out_md, out_json):
    """SQ instruction and LDS counters, and the wave-state split, per workload's kernel. The
    JSON record (stamped with a digest of the kernel's sources) gives bench.py the LDS
    bank-conflict rate and the VALU-active share of the kernel it times."""
    cmds = [_display(a, prof) for n, a, _ in passes(prof) if n.startswith("sq_") or n.startswith("state_")]
    md = ["# SQ counters: LDS instructions, bank conflicts, VALU/MFMA instructions, wave states", ""] + _cmd_block(cmds)
    md += ["Means per dispatch. The wave-state shares divide by SQ_WAVE_CYCLES (the waves' summed lifetime): "
           "`VALU-active` is SQ_ACTIVE_INST_VALU (cycles a wave spends issuing VALU instructions, MFMA "
           "included), `waiting` SQ_WAIT_ANY (cycles waiting on a counter or the barrier).", ""]
    rec = {"about": "SQ counter means per dispatch, one record per benchmarked kernel (rocprofv3 --pmc)",
           "kernels": {}}
    for w in SQ_WORKLOADS:
        label, sub, sources, _ = KERNELS[w]
        m = _kernel_means(os.path.join(prof, f"sq_{w}", "sq_counter_collection.csv"), sub)
        md += [f"## {w} (`{label}`)", ""]
        md += [f"- {c}: {m[c]:.0f}" for c in sorted(m)]
        waves = m.get("SQ_WAVES", 0)
        entry = {"workload": w, "sources": sources, "sources_digest": _digest(sources)}
        if waves:
            md.append(f"- per wave: {m['SQ_INSTS_LDS'] / waves:.0f} LDS instructions, "
                      f"{m['SQ_INSTS_VALU'] / waves:.0f} VALU instructions, "
                      f"{m.get('SQ_INSTS_MFMA', 0) / waves:.0f} MFMA instructions")
        if m.get("SQ_LDS_IDX_ACTIVE"):
            rate = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"]
            entry["lds_bank_conflict_rate"] = round(rate, 4)
            md.append(f"- bank-conflict rate SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = {100 * rate:.1f} %")
        st_path = os.path.join(prof, f"state_{w}", "st_counter_collection.csv")
        if os.path.exists(st_path):
            st = _kernel_means(st_path, sub)
            wc = st.get("SQ_WAVE_CYCLES", 0)
            if wc:
                shares = {k: st.get(c, 0) / wc for k, c in (("valu_active", "SQ_ACTIVE_INST_VALU"),
                                                             ("lds_active", "SQ_ACTIVE_INST_LDS"),
                                                             ("vmem_active", "SQ_ACTIVE_INST_VMEM"),
                                                             ("waiting", "SQ_WAIT_ANY"))}
                entry.update({f"{k}_share": round(v, 4) for k, v in shares.items()})
                md.append(f"- wave states: VALU-active {100 * shares['valu_active']:.1f} %, LDS-issue "
                          f"{100 * shares['lds_active']:.1f} %, VMEM-issue {100 * shares['vmem_active']:.1f} %, "
                          f"waiting {100 * shares['waiting']:.1f} % of SQ_WAVE_CYCLES "
                          f"({st.get('SQ_WAVES', 0):.0f} waves)")
        rec["kernels"][label] = entry
        md.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)


def _short_kernel(name):
    name = name.replace("void ", "").replace("regtile::(anonymous namespace)::", "").replace("regtile::", "")
    return name.split("(int")[0]


def summarize_ladder_sq(prof, out_md):
    """Per kernel of the ladder (fp32 rungs at 4096^3, 16-bit rungs at 8192^3), mean per
    dispatch: LDS, VALU and MFMA instructions per wave, LDS instructions per 1000 VALU, and the
    share of LDS-active cycles lost to bank conflicts."""
    d = _pmc(os.path.join(prof, "sq_ladder", "sq_counter_collection.csv"))
    per = collections.defaultdict(dict)
    for (k, c), vs in d.items():
        per[k][c] = sum(vs) / len(vs)
    cmd = [_display(a, prof) for n, a, _ in passes(prof) if n == "sq_ladder"]
    md = ["# Ladder rungs: LDS, VALU and MFMA instructions and LDS bank conflicts (rocprofv3 --pmc)", ""]
    md += _cmd_block(cmd)
    md += ["Mean per dispatch: fp32 rungs at 4096^3, 16-bit rungs at 8192^3 (every kernel the ladder launched). "
           "SQ_INSTS_VALU counts the MFMA instructions too on this counter set. The last column is "
           "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
           "| kernel | LDS instr / wave | VALU instr / wave | MFMA instr / wave | LDS per 1000 VALU | bank-conflict share |",
           "|---|---|---|---|---|---|"]
    for k, m in sorted(per.items(), key=lambda kv: _short_kernel(kv[0])):
        if "regtile" not in k:
            continue
        waves = m.get("SQ_WAVES", 0) or 1
        lds, valu, mfma = m.get("SQ_INSTS_LDS", 0) / waves, m.get("SQ_INSTS_VALU", 0) / waves, m.get("SQ_INSTS_MFMA", 0) / waves
        act = m.get("SQ_LDS_IDX_ACTIVE", 0)
        conf = f"{100 * m.get('SQ_LDS_BANK_CONFLICT', 0) / act:.1f} %" if act else "-"
        md.append(f"| `{_short_kernel(k)}` | {lds:.0f} | {valu:.0f} | {mfma:.0f} | "
                  f"{1000 * lds / valu if valu else 0:.1f} | {conf} |")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    # the same means as JSON, for the counter-invariant test (tests/test_counter_invariants.py):
    # fp32 kernels ran on f32_4096, 16-bit kernels on bf16_8192
    srcs = ["gemm_simple.hip", "gemm_f32_regtile.hip", "gemm_f32_splitk.hip", "gemm_bf16_mfma.hip",
            "gemm_bf16_mfma_dma.hip", "mfma_common.h", "tile_addressing.h", "regtile_internal.h"]
    rec = {"about": "rocprofv3 --pmc means per dispatch over the ladder run named in `command`; fp32 "
                    "kernels at 4096^3, 16-bit kernels at 8192^3 (bf16 operands)",
           "command": cmd[0], "sources": srcs, "sources_digest": _digest(srcs), "kernels": {}}
    for k, m in sorted(per.items(), key=lambda kv: _short_kernel(kv[0])):
        if "regtile" not in k:
            continue
        waves = m.get("SQ_WAVES", 0) or 1
        rec["kernels"][_short_kernel(k)] = {
            "workload": "bf16_8192" if ("bf16" in k or "unsigned short" in k) else "f32_4096",
            "waves": m.get("SQ_WAVES", 0),
            "lds_instructions_per_wave": m.get("SQ_INSTS_LDS", 0) / waves,
            "valu_instructions_per_wave": m.get("SQ_INSTS_VALU", 0) / waves,
            "mfma_instructions_per_wave": m.get("SQ_INSTS_MFMA", 0) / waves,
            "lds_bank_conflict_cycles": m.get("SQ_LDS_BANK_CONFLICT", 0),
            "lds_active_cycles": m.get("SQ_LDS_IDX_ACTIVE", 0)}
    with open(os.path.splitext(out_md)[0] + ".json", "w") as f:
        json.dump(rec, f, indent=1)


def summarize_datadep(prof, out_md):
    """Clock and MFMA busy share of the bf16 8192^3 kernel per input data set. tune datadep
    launches DD_WARMUP warm-up launches of the first set, then DD_ROUNDS rounds over the sets,
    each set 10 untimed and DD_STEPS timed launches; the dispatches are labelled in that order."""
    d = os.path.join(prof, "clock_datadep")
    rows = [r for r in csv.DictReader(open(os.path.join(d, "clk_counter_collection.csv")))
            if "bf16_mfma_dma_kernel" in r["Kernel_Name"]]
    per = collections.OrderedDict()
    for r in rows:
        per.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    dur = {}
    for r in csv.DictReader(open(os.path.join(d, "clk_kernel_trace.csv"))):
        if "bf16_mfma_dma_kernel" in r["Kernel_Name"]:
            dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    sets = []
    with open(os.path.join(prof, "clock_datadep.out")) as f:
        for line in f:
            if line.startswith("| ") and not line.startswith("| A, B data") and "---" not in line:
                sets.append(line.split("|")[1].strip())
    order = [sets[0]] * DD_WARMUP
    for _ in range(DD_ROUNDS):
        for k in sets:
            order += [k] * (10 + DD_STEPS)
    ids = sorted(per)
    if len(ids) != len(order):
        raise ValueError(f"{len(ids)} bf16 dispatches against {len(order)} expected")
    import gemm_inputs as gi

    flop = gi.WORKLOADS["bf16_8192"].flop
    stats = collections.OrderedDict((k, []) for k in sets)
    for i, k in zip(ids, order[:len(ids)]):
        c = per[i]
        cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
        t = dur[i]
        stats[k].append((t, cycles / t / 1e9, c["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cycles, flop / t / 1e12))
    argv = [a for n, a, _ in passes(prof) if n == "clock_datadep"][0]
    md = ["# bf16 8192^3: clock and MFMA busy share against the input data (rocprofv3 --pmc, GRBM and SQ cycles)", ""]
    md += _cmd_block([_display(argv, prof)])
    md += ["The same kernel and the same instruction stream on six input data sets, interleaved. Per dispatch: "
           "the duration from the kernel trace; the shader clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; the "
           "MFMA busy share = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / those cycles. Medians over the timed "
           "and untimed launches of both rounds (the counters serialise the dispatches, so durations run a "
           "little longer than in the benchmark).", "",
           "| A, B data | dispatches | duration (ms) | clock (GHz) | MFMA busy | TFLOP/s |", "|---|---|---|---|---|---|"]
    for k, v in stats.items():
        if not v:
            continue
        med = [statistics.median(x[j] for x in v) for j in range(4)]
        md.append(f"| {k} | {len(v)} | {med[0] * 1e3:.4f} | {med[1]:.2f} | {100 * med[2]:.0f} % | {med[3]:.0f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")


def summarize_clock(prof, out_md):
    """Shader clock, MFMA busy share and (fp32) SIMD cycles per wave64 FMA of the benchmarked
    fp32 4096^3 and bf16 8192^3 kernels, per dispatch of `bench.py --only <workload>` (its
    CLOCK_WARMUP warm-up launches, then CLOCK_STEPS timed ones)."""
    import gemm_inputs as gi

    md = ["# Shader clock, MFMA busy share and FMA issue rate inside the benchmarked kernels "
          "(rocprofv3 --pmc, GRBM and SQ cycles)", ""]
    md += _cmd_block([_display(a, prof) for n, a, _ in passes(prof) if n.startswith("clock_") and n != "clock_datadep"])
    md += ["Per dispatch: the duration from the kernel trace; shader cycles = GRBM_GUI_ACTIVE / 8 XCDs; "
           "clock = those cycles / the duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / those "
           "cycles; for the fp32 kernel, SIMD cycles per wave64 FMA = those cycles / (M N K / 64 lanes / 1024 "
           "SIMDs). Medians over the timed launches (the last "
           f"{CLOCK_STEPS}); the counters serialise the dispatches, so durations run a little longer than "
           "in the benchmark.", "",
           "| workload | kernel | dispatches | duration (ms) | shader cycles per XCD (M) | clock (GHz) | "
           "MFMA busy | SIMD cycles per wave64 FMA | TFLOP/s |",
           "|---|---|---|---|---|---|---|---|---|"]
    for w in CLOCK_WORKLOADS:
        d = os.path.join(prof, f"clock_{w}")
        label, sub = KERNELS[w][0], KERNELS[w][1]
        per = collections.OrderedDict()
        for r in csv.DictReader(open(os.path.join(d, "clk_counter_collection.csv"))):
            if sub in r["Kernel_Name"]:
                per.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        dur = {}
        for r in csv.DictReader(open(os.path.join(d, "clk_kernel_trace.csv"))):
            if sub in r["Kernel_Name"]:
                dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        ids = sorted(i for i in per if i in dur)[-CLOCK_STEPS:]
        wl = gi.WORKLOADS[w]
        rows = []
        for i in ids:
            cyc = per[i]["GRBM_GUI_ACTIVE"] / N_XCD
            t = dur[i]
            mfma = per[i].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / N_SIMD / cyc
            fma = cyc / (wl.M * wl.N * wl.K / 64 / N_SIMD) if wl.dtype == "f32" else None
            rows.append((t, cyc, cyc / t / 1e9, mfma, fma, wl.flop / t / 1e12))
        med = [statistics.median(r[j] for r in rows) if rows[0][j] is not None else None for j in range(6)]
        md.append(f"| {w} | `{label}` | {len(rows)} | {med[0] * 1e3:.4f} | {med[1] / 1e6:.3f} | {med[2]:.2f} | "
                  + (f"{100 * med[3]:.0f} %" if wl.dtype != "f32" else "-") + " | "
                  + (f"{med[4]:.2f}" if med[4] is not None else "-") + f" | {med[5]:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")


def summarize(prof) -> int:
    prof = os.path.abspath(prof)
    for w in TRACE_WORKLOADS:
        if os.path.exists(os.path.join(prof, f"trace_{w}", "trace_kernel_stats.csv")):
            summarize_trace(prof, w, os.path.join(PROFILES, f"kernel_trace_{w}.md"))
    if os.path.exists(os.path.join(prof, "pmc_FETCH_SIZE_copy")):
        summarize_traffic(prof, os.path.join(PROFILES, "pmc_traffic.json"),
                          os.path.join(PROFILES, "hbm_traffic_f32_4096_bf16_8192.md"))
    if os.path.exists(os.path.join(prof, "sq_f32_4096")):
        summarize_sq(prof, os.path.join(PROFILES, "sq_counters_bench_kernels.md"),
                     os.path.join(PROFILES, "sq_counters_bench_kernels.json"))
    if all(os.path.exists(os.path.join(prof, f"clock_{w}", "clk_counter_collection.csv")) for w in CLOCK_WORKLOADS):
        summarize_clock(prof, os.path.join(PROFILES, "clock_f32_4096_bf16_8192.md"))
    if os.path.exists(os.path.join(prof, "clock_datadep", "clk_counter_collection.csv")):
        summarize_datadep(prof, os.path.join(PROFILES, "clock_datadep_bf16_8192.md"))
    if os.path.exists(os.path.join(prof, "sq_ladder", "sq_counter_collection.csv")):
        summarize_ladder_sq(prof, os.path.join(PROFILES, "lds_counters_ladder_f32_4096_bf16_8192.md"))
    return 0


def main(argv=None) -> int:
    import argparse

    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("cmd", choices=["collect", "summarize", "commands"])
    p.add_argument("dir", help="directory for (collect) or of (summarize) the rocprofv3 output")
    p.add_argument("--only", default="", help="collect: comma-separated pass names")
    a = p.parse_args(argv)
    if a.cmd == "collect":
        return collect(a.dir, [s for s in a.only.split(",") if s])
    if a.cmd == "commands":
        for name, argv_, limit in passes(os.path.abspath(a.dir)):
            print(f"{name} ({limit} s): {' '.join(argv_)}")
        return 0
    return summarize(a.dir)


if __name__ == "__main__":
    sys.exit(main())
