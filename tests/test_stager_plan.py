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
  * the later copies are grouped so that every engine's piece is at least 2 MiB: copies that
    large on their own are striped over the engines one after another, piece p on engine p;
    smaller ones are split together in groups like the leading group, and a short last group
    is merged into the one before, so no copy runs alone at the end.
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


def plan(driver, engines, split, lead, sizes, group=1):
    out = subprocess.run([driver, str(engines), str(split), str(lead), str(group), *map(str, sizes)], check=True,
                         capture_output=True, text=True, timeout=30).stdout.splitlines()
    assert out[0].startswith("group ")
    plan.group = int(out[0].split()[1])
    return [tuple(int(v) for v in line.split()) for line in out[1:]]


def check_group(by_copy, copies, engines):
    """The copies of one group take distinct engines, every engine when they can."""
    group = [p for c in copies for p in by_copy[c]]
    used = [e for _, _, _, e in group]
    assert len(used) == len(set(used)), f"an engine takes two pieces of the group {copies}"
    if sum(len(by_copy[c]) for c in copies) >= engines or all(len(by_copy[c]) > 1 for c in copies):
        assert len(group) == engines


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


# staged peers (+ own slot) of the workloads: (engines, lead, sizes, expected later groups)
WORKLOAD_PLANS = [
    # 8192 x 4096, tp = 8: peers 1-3 lead the first round; peers 4-7 and the own slot are split
    # together (8 MiB striped over 14 engines would give 585 KB pieces)
    (14, 3, [8 * MiB] * 7 + [8 * MiB], [[3, 4, 5, 6, 7]]),
    (14, 1, [28 * MiB] * 3 + [28 * MiB], [[0], [1], [2], [3]]),      # Qwen2-like, tp = 4
    (14, 1, [64 * MiB] * 7 + [64 * MiB], [[c] for c in range(8)]),  # M-sweep top, tp = 8
    (14, 7, [8 * MiB] * 7, []),                                     # every peer in the first round
]


@pytest.mark.parametrize("engines,lead,sizes,groups", WORKLOAD_PLANS)
def test_workload_plans(driver, engines, lead, sizes, groups):
    pieces = plan(driver, engines, 1, lead, sizes, group=0)
    by_copy = check_cover(pieces, sizes, 1)
    if lead > 1:
        check_group(by_copy, range(lead), engines)
        counts = [len(by_copy[c]) for c in range(lead)]
        assert max(counts) - min(counts) <= 1, f"equal copies get unequal piece counts {counts}"
    for g in groups:
        if len(g) == 1:  # striped alone
            for off, n, piece, engine in by_copy[g[0]]:
                assert engine == piece % engines
            assert len(by_copy[g[0]]) == min(MAX_PIECES, engines, sizes[g[0]] // MIN_PIECE)
        else:
            check_group(by_copy, g, engines)
            assert min(n for c in g for _, n, _, _ in by_copy[c][:-1]) >= 2 * MiB - 256
    # pieces are submitted group by group, in copy order
    order = [c for c, *_ in pieces]
    assert order == sorted(order)


@pytest.mark.parametrize("engines,chunk,want", [
    (14, 8 * MiB, 4), (14, 28 * MiB, 1), (14, 64 * MiB, 1), (14, 64 * 1024, 14), (1, 8 * MiB, 1), (7, 8 * MiB, 2),
])
def test_group_size_rule(driver, engines, chunk, want):
    plan(driver, engines, 1, 1, [chunk], group=0)
    assert plan.group == want


def test_explicit_groups_and_short_last_group(driver):
    sizes = [4 * MiB] * 8
    by_copy = check_cover(plan(driver, 14, 1, 1, sizes, group=3), sizes, 1)
    # groups [0, 1, 2] and [3 .. 7]: the last two copies join the group before them
    check_group(by_copy, [0, 1, 2], 14)
    check_group(by_copy, [3, 4, 5, 6, 7], 14)
    # too many to merge on 4 engines: groups [0..3], [4..7] stay apart
    by_copy = check_cover(plan(driver, 4, 1, 1, sizes, group=4), sizes, 1)
    check_group(by_copy, [0, 1, 2, 3], 4)
    check_group(by_copy, [4, 5, 6, 7], 4)
    # a last group of one that cannot merge (5 copies on 4 engines in groups of 4)
    sizes = [4 * MiB] * 5
    by_copy = check_cover(plan(driver, 4, 1, 1, sizes, group=4), sizes, 1)
    check_group(by_copy, [0, 1, 2, 3], 4)
    assert [e for _, _, _, e in by_copy[4]] == [0, 1, 2, 3]


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


def plan_links(driver, engines, per, sizes, links):
    args = [f"{n}:{l}" if l is not None else str(n) for n, l in zip(sizes, links)]
    out = subprocess.run([driver, "links", str(engines), str(per), *args], check=True, capture_output=True,
                         text=True, timeout=30).stdout.splitlines()
    assert out[0] == "group 0"
    return [tuple(int(v) for v in line.split()) for line in out[1:]]


@pytest.mark.parametrize("engines,per,sizes,links", [
    # 8192 x 4096 rows, tp = 8, two sub-chunks per rank in the interleaved order, then the own slot
    (14, 2, [4 * MiB] * 14 + [8 * MiB], [0, 1, 2, 3, 4, 5, 6] * 2 + [None]),
    (14, 1, [64 * MiB] * 7 + [64 * MiB], list(range(7)) + [None]),   # M-sweep top, one engine per peer
    (14, 4, [16 * MiB] * 6, [0, 1, 2, 0, 1, 2]),                     # tp = 4, engines 0-11
    (4, 2, [8 * MiB] * 7, list(range(7))),                            # more peers than engine pairs: shared
    (14, 2, [1000, 300 * 1024], [0, 1]),                              # copies below a piece: one piece
])
def test_link_model(driver, engines, per, sizes, links):
    pieces = plan_links(driver, engines, per, sizes, links)
    by_copy = check_cover(pieces, sizes, 1)
    for c, l in enumerate(links):
        used = [e for _, _, _, e in by_copy[c]]
        if l is None:  # no link: striped over every engine
            assert used == list(range(len(used))) and len(used) == min(engines, MAX_PIECES, max(1, sizes[c] // MIN_PIECE))
        else:  # a peer's copies only on its own engines, in order
            own = [(l * per + j) % engines for j in range(min(per, engines))]
            assert used == own[:len(used)]
            assert len(used) == min(per, engines, max(1, sizes[c] // MIN_PIECE))
    # pieces in copy order, so each engine takes a peer's copies in the order given
    order = [c for c, *_ in pieces]
    assert order == sorted(order)
    if engines >= per * (max(l for l in links if l is not None) + 1):  # disjoint engine sets
        for a in range(len(links)):
            for b in range(len(links)):
                if links[a] is not None and links[b] is not None and links[a] != links[b]:
                    assert not {e for *_, e in by_copy[a]} & {e for *_, e in by_copy[b]}


def test_trailing_copies_stay_out_of_groups(driver):
    """The own slot (the trailing copy, which no tile waits for) joins the peers' last group only
    when it adds at most a quarter of the group's bytes: at 8192 x 4096, tp = 8, peers 4-7 and the
    own slot are split together (8 MiB next to 32 MiB); with a 12 MiB own slot it follows on its
    own in 2 MiB pieces; at 32768 x 1024, tp = 4, peers 2 and 3 are split together and the own
    slot (16 MiB next to 32 MiB) follows them."""
    def run(sizes, lead):
        out = subprocess.run([driver, "14", "1", str(lead), "0:1", *map(str, sizes)], check=True,
                             capture_output=True, text=True, timeout=30).stdout.splitlines()
        pieces = [tuple(int(v) for v in line.split()) for line in out[1:]]
        assert [c for c, *_ in pieces] == sorted(c for c, *_ in pieces)
        return check_cover(pieces, sizes, 1)
    by_copy = run([8 * MiB] * 8, 3)
    check_group(by_copy, [3, 4, 5, 6, 7], 14)
    by_copy = run([8 * MiB] * 7 + [12 * MiB], 3)
    check_group(by_copy, [3, 4, 5, 6], 14)
    assert [e for _, _, _, e in by_copy[7]] == [0, 1, 2, 3, 4, 5]
    by_copy = run([16 * MiB] * 3, 1)
    check_group(by_copy, [0, 1], 14)
    assert [e for _, _, _, e in by_copy[2]] == list(range(8))
