"""Memory extents of the 16-bit kernels' buffer-descriptor accesses, checked on the CPU.

`extent_check.cpp` enumerates every load and store that the edge tiles of the LDS-DMA kernel
(K-contiguous "n t", M/N-major "t n", register rows "n n" / "t t"), the split-K kernel's
per-wave DMA ("sk") and the register-staged kernel's M/N-contiguous gather issue through a
buffer descriptor, computing each offset with
the functions the kernels call (csrc/tile_addressing.h). It checks that every descriptor ends
inside the caller's matrix, that no access meant for a matrix element straddles or passes a
descriptor end, that each offset addresses the element the layout assigns it, and that every
element of a tile is loaded (or stored) exactly once. A build with the earlier, looser
descriptor sizes and runs that bypass the launchers' admission rules must fail: they are the
check's own controls. No GPU is used.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "extent_check.cpp")
CSRC = os.path.join(ROOT, "register_tiled_matrix_amd", "csrc")


def _build(tmp_path_factory, *defines):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("extent") / ("extent_check" + "".join(d.lower() for d in defines))
    cmd = [gxx, "-O2", "-std=c++17", "-Wall", "-Werror", f"-I{CSRC}", *[f"-D{d}" for d in defines], SRC, "-o",
           str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return str(out)


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    return _build(tmp_path_factory)


@pytest.fixture(scope="module")
def loose_checker(tmp_path_factory):
    return _build(tmp_path_factory, "EXTENT_LOOSE")


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout


# (path, M, N, K, lda, ldb, ldc): leading dimensions are those of the stored operands (A stored
# K x M for "t n" / "t t" / gather, B stored K x N for "t n" / "n n" / gather).
TAKEN = [
    ("tn", 1000, 1504, 777, 1000, 1504, 1504),     # ragged tile edge on both operands, K tail
    ("tn", 1088, 256, 16384, 1088, 256, 256),      # last-row over-read of the earlier descriptor
    ("tn", 8192, 8192, 8192, 8192, 8192, 8192),    # the bf16 workload in this storage
    ("tn", 2048, 2048, 1024, 2056, 2048, 2048),    # 128x128 tiles, padded rows
    ("nn", 1000, 1504, 776, 776, 1504, 1504),
    ("nn", 8192, 8192, 8192, 8192, 8192, 8192),
    ("tt", 1000, 1504, 776, 1000, 776, 1504),
    ("tt", 4000, 4100, 200, 4000, 200, 4100),
    ("kc", 8192, 8192, 8192, 8192, 8192, 8192),    # A row-major, B column-major: the workload
    ("kc", 8000, 8000, 8192, 8192, 8192, 8000),
    ("kc", 6000, 6000, 6000, 6000, 6000, 6000),    # K tail
    ("kc", 1, 1, 8, 8, 8, 1),
    ("sk", 1024, 1024, 16384, 16384, 16384, 1024),  # split-K kernel: few tiles, deep K
    ("sk", 1000, 1000, 776, 776, 776, 1000),        # ragged tile edge, K tail
    ("sk", 65, 129, 72, 72, 80, 129),
    ("sk", 1, 1, 8, 8, 8, 1),
    ("gather", 4000, 4100, 200, 4000, 4100, 4100),
    ("gather", 1000, 1504, 777, 1000, 1504, 1504),
]


@pytest.mark.parametrize("case", TAKEN, ids=lambda c: "-".join(map(str, c)))
def test_descriptor_accesses_stay_inside_the_operands(checker, case):
    rc, out = _run(checker, "one", *case)
    assert rc == 0, out
    assert out.startswith("taken"), out


def test_seeded_sweep_of_edge_shapes(checker):
    # M, N, K drawn from sizes around 1, the slab depth, both tile edges and primes; every
    # arrangement a launcher takes is enumerated
    rc, out = _run(checker, "sweep", 20261202, 250)
    assert rc == 0, out
    taken = int(out.split()[2])
    assert taken > 300, out


@pytest.mark.parametrize("case", [
    ("tn", 1001, 1504, 777, 1008, 1504, 1504),     # M not a multiple of 8
    ("tn", 1000, 1500, 777, 1000, 1504, 1504),     # N not a multiple of 8
    ("nn", 1000, 1502, 776, 776, 1504, 1504),      # N not a multiple of 4
    ("tt", 1001, 1504, 776, 1004, 776, 1504),      # M not a multiple of 4
], ids=lambda c: "-".join(map(str, c)))
def test_launchers_refuse_runs_that_would_straddle(checker, case):
    # the launcher's admission rule refuses these problems ...
    rc, out = _run(checker, "one", *case)
    assert rc == 0 and out.startswith("not-taken"), out
    # ... and the enumeration shows why: a run meant for a matrix element straddles the end
    rc, out = _run(checker, "force", *case)
    assert rc == 1 and "straddles the descriptor end over a matrix element" in out, out


def test_gather_needs_whole_runs(checker):
    # column count not a multiple of 4: the staged kernel's descriptor gather would cut the
    # last run of the last row, so it takes predicated loads there instead
    rc, out = _run(checker, "one", "gather", 1001, 1502, 776, 1004, 1504, 1504)
    assert rc == 0 and out.startswith("not-taken"), out
    rc, out = _run(checker, "force", "gather", 1001, 1502, 776, 1004, 1504, 1504)
    assert rc == 1, out


@pytest.mark.parametrize("case", [
    ("tn", 1088, 256, 16384, 1088, 256, 256),
    ("tn", 1000, 1504, 777, 1000, 1504, 1504),
    ("tt", 1000, 1504, 776, 1000, 776, 1504),
], ids=lambda c: "-".join(map(str, c)))
def test_control_earlier_descriptor_sizes_read_past_the_operand(loose_checker, case):
    # K full rows from the tile's first column: the last row's columns past M (N) lie beyond
    # the operand's last element, which the check must report
    rc, out = _run(loose_checker, "one", *case)
    assert rc == 1 and "descriptor outside the matrix" in out, out
