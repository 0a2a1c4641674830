"""Builds ``libregtile.so`` (the C-ABI HIP library) in-tree for gfx950 with hipcc.

Every translation unit under ``csrc/`` is compiled for ``--offload-arch=gfx950`` with
packed-FP32 code generation switched off (``-Xclang -target-feature -Xclang
-packed-fp32-ops``), then linked into one shared library next to this file. The compiler's
per-kernel resource remarks (VGPRs, AGPRs, SGPRs, scratch, LDS, occupancy) are written to
``_build/resource_usage.txt`` at the repository root.

    python -m register_tiled_matrix_amd.build        # or build() from Python
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libregtile.so")
ARCH = "gfx950"

SOURCES = ["regtile_api.hip", "gemm_simple.hip", "gemm_f32_regtile.hip", "gemm_f32_splitk.hip",
           "gemm_bf16_mfma.hip", "gemm_bf16_mfma_dma.hip", "gemm_bf16_mfma_splitk.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, extra: list[str], obj_dir: str = BUILD_DIR) -> tuple[str, str]:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj, r.stderr


def _resource_report(logs: list[str]) -> str:
    out = []
    for log in logs:
        for line in log.splitlines():
            if "remark:" in line and ("Function Name" in line or "VGPRs" in line
                                      or "AGPRs" in line or "ScratchSize" in line
                                      or "Occupancy" in line or "LDS Size" in line
                                      or "SGPRs:" in line):
                out.append(line.split("remark: ", 1)[1])
    return "\n".join(out) + "\n"


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          out_dir: str | None = None, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libregtile.so; returns its path.

    With ``out_dir`` (used for tuning variants built with other ``-D`` values) the objects,
    the library and the resource report go there instead of the in-tree locations."""
    obj_dir = out_dir or BUILD_DIR
    lib = os.path.join(out_dir, "libregtile.so") if out_dir else LIB
    os.makedirs(obj_dir, exist_ok=True)
    extra = list(extra_flags or [])
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra, obj_dir), SOURCES))
    objs = [o for o, _ in results]
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)
    report = _resource_report([log for _, log in results])
    with open(os.path.join(obj_dir, "resource_usage.txt"), "w") as f:
        f.write(report)
    if verbose:
        print(f"built {lib}", flush=True)
    return lib


def resource_usage(build_dir: str | None = None) -> dict:
    """Parse <build_dir>/resource_usage.txt (default _build/) into {kernel: {field: value}}."""
    path = os.path.join(build_dir or BUILD_DIR, "resource_usage.txt")
    res: dict = {}
    cur = None
    with open(path) as f:
        for line in f:
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = m.group(1)
                res[cur] = {}
                continue
            m = re.search(r"^(.*?): (-?\d+)", line.strip())
            if m and cur is not None:
                res[cur][m.group(1).strip()] = int(m.group(2))
    return res


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
