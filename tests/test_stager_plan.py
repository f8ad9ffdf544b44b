"""The SDMA stager's copy-piece plan (csrc/sptl_plan.h), checked on the CPU.

The plan is plain host code: a small driver is built with g++ from the header and run for the
staging shapes of the workloads and for edge cases.  Properties checked:
  * the pieces of every copy cover it exactly, in order (offsets contiguous, sizes summing to
    the copy), with piece ids 0, 1, ...; every piece but the last is a multiple of 256 bytes;
  * no copy has more than kMaxPieces pieces, and none has a piece below kMinPiece / split
    bytes unless the copy itself is that small (one piece);
  * with a leading group of copies (lead > 1), each engine takes at most one of the group's
    pieces, the group takes every engine when it is large enough, and the pieces per copy
    follow the copy sizes;
  * every later copy is striped over the engines, piece p on engine p.
"""
import os
import shutil
import subprocess

import pytest

from tests.util import ROOT

CSRC = os.path.join(ROOT, "sp_transformer_linear_amd", "csrc")
MAX_PIECES = 16
MIN_PIECE = 512 * 1024
MiB = 1 << 20


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("plan") / "plan")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "stager_plan_driver.cpp"),
                    "-o", exe], check=True, timeout=120)
    return exe


def plan(driver, engines, split, lead, sizes):
    out = subprocess.run([driver, str(engines), str(split), str(lead), *map(str, sizes)], check=True,
                         capture_output=True, text=True, timeout=30).stdout
    return [tuple(int(v) for v in line.split()) for line in out.splitlines()]


def check_cover(pieces, sizes, split):
    by_copy = {}
    for copy, off, nbytes, chunk, piece, engine in pieces:
        assert chunk == copy
        by_copy.setdefault(copy, []).append((off, nbytes, piece, engine))
    assert sorted(by_copy) == list(range(len(sizes)))
    for copy, ps in by_copy.items():
        assert [p[2] for p in ps] == list(range(len(ps))), "piece ids out of order"
        assert len(ps) <= MAX_PIECES
        off = 0
        for i, (o, n, _, _) in enumerate(ps):
            assert o == off and n > 0
            if i + 1 < len(ps):
                assert n % 256 == 0
            off += n
        assert off == sizes[copy], "pieces do not cover the copy"
        if len(ps) > 1:
            assert min(n for _, n, _, _ in ps[:-1]) >= MIN_PIECE // split
    return by_copy


# staged peers (+ own slot) of the workloads: (engines, lead, sizes)
WORKLOAD_PLANS = [
    (14, 3, [8 * MiB] * 7 + [8 * MiB]),        # 8192 x 4096, tp = 8: peers 1-3 lead the first round
    (14, 1, [28 * MiB] * 3 + [28 * MiB]),      # Qwen2-like, tp = 4
    (14, 1, [64 * MiB] * 7 + [64 * MiB]),      # M-sweep top, tp = 8
    (14, 7, [8 * MiB] * 7),                    # every peer in the first round
]


@pytest.mark.parametrize("engines,lead,sizes", WORKLOAD_PLANS)
def test_workload_plans(driver, engines, lead, sizes):
    pieces = plan(driver, engines, 1, lead, sizes)
    by_copy = check_cover(pieces, sizes, 1)
    if lead > 1:
        group = [p for c in range(lead) for p in by_copy[c]]
        engines_used = [e for _, _, _, e in group]
        assert len(engines_used) == len(set(engines_used)), "an engine takes two pieces of the leading group"
        assert len(group) == engines
        counts = [len(by_copy[c]) for c in range(lead)]
        assert max(counts) - min(counts) <= 1, f"equal copies get unequal piece counts {counts}"
    for c in range(lead if lead > 1 else 0, len(sizes)):
        for off, n, piece, engine in by_copy[c]:
            assert engine == piece % engines
    if lead == 1:
        assert len(by_copy[0]) == min(MAX_PIECES, engines, sizes[0] // MIN_PIECE)


def test_leading_group_follows_sizes(driver):
    sizes = [12 * MiB, 4 * MiB, 8 * MiB, 8 * MiB]
    by_copy = check_cover(plan(driver, 12, 1, 3, sizes), sizes, 1)
    counts = [len(by_copy[c]) for c in range(3)]
    assert counts == [6, 2, 4]
    assert sorted(e for c in range(3) for _, _, _, e in by_copy[c]) == list(range(12))


@pytest.mark.parametrize("engines,split,lead,sizes", [
    (14, 1, 1, [1000]),                        # a copy smaller than a piece: one piece
    (14, 1, 3, [300, 300, 8 * MiB]),           # a tiny leading group
    (1, 1, 3, [8 * MiB, 8 * MiB]),             # one engine: no leading group
    (14, 16, 1, [4 * MiB] * 3),                # 16 pieces per chunk at most
    (3, 1, 5, [2 * MiB] * 5),                  # more leading copies than engines
    (14, 1, 0, [8 * MiB] * 2),                 # lead below 1 is taken as 1
])
def test_edge_cases(driver, engines, split, lead, sizes):
    pieces = plan(driver, engines, split, lead, sizes)
    by_copy = check_cover(pieces, sizes, split)
    assert all(0 <= e < engines for _, _, _, e in (p for ps in by_copy.values() for p in ps))
    if split == 16:
        assert all(len(ps) == MAX_PIECES for ps in by_copy.values())
