"""The GEMM tile orders (csrc/sptl_tilemap.h), checked on the CPU.

A small driver is built with g++ from the header the kernels use.  For every shape checked:
  * plain launches: the workgroups take every tile exactly once;
  * chunk-ordered launches: the workgroups take every tile of every chunk exactly once, and
    each XCD (workgroup index mod 8) meets the chunks in processing order, so no XCD runs a
    later chunk's tile before an earlier chunk's;
  * the layout chosen for each workload: XCDs per chunk and band height.
"""
import itertools
import os
import shutil
import subprocess

import pytest

from tests.util import ROOT

CSRC = os.path.join(ROOT, "sp_transformer_linear_amd", "csrc")
CONC = 32  # workgroups an XCD runs at once: one per CU, 32 CUs per XCD


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("tilemap") / "tilemap")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "tilemap_driver.cpp"),
                    "-o", exe], check=True, timeout=120)
    return exe


def run(driver, *args):
    r = subprocess.run([driver, *map(str, args)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, f"{args}: {r.stdout} {r.stderr}"
    return r.stdout.split()


def test_plain_orders_cover_every_tile_once(driver):
    for tm, tn in itertools.product(range(1, 42, 3), range(1, 42, 4)):
        assert run(driver, "plain", tm, tn) == ["ok"]


def test_chunk_orders_cover_every_tile_once_in_chunk_order(driver):
    for tpc, tiles_n, n_chunks in itertools.product((1, 2, 3, 4, 8, 16, 32), (1, 2, 3, 5, 16, 17, 37),
                                                    (1, 2, 3, 4, 6, 8, 16)):
        for forced in (0, 1, 2, 4, 8):
            out = run(driver, "chunk", tpc, tiles_n, n_chunks, forced, CONC)
            assert out[-1] == "ok"


# (tile rows per chunk, tile columns, chunks) -> (XCDs per chunk, band height)
@pytest.mark.parametrize("tpc,tiles_n,n_chunks,forced,want", [
    (4, 16, 8, 0, (8, 2)),      # 8192 x 4096 x 4096, tp = 8: 2 x 4 blocks in each of 4 chunks
    (4, 16, 8, 2, (2, 4)),      # the same with 2 XCDs per chunk forced: a 4 x 8 block of one chunk
    (16, 37, 4, 0, (8, 4)),     # Qwen2-like: 16384 rows, N = 9472, tp = 4
    (32, 16, 8, 0, (8, 4)),     # M-sweep top: 65536 rows, tp = 8
    (32, 3, 4, 0, (8, 2)),      # Qwen3-0.6B-like shard as a gather: N = 768
    (4, 1, 8, 0, (4, 1)),       # an 8-column weight: one tile per XCD and chunk, band 1 (33 panels vs 65)
    (2, 17, 8, 0, (2, 2)),      # 512-row chunks, 17 tile columns: the band is at most the chunk's 2 rows
    (1, 3, 3, 0, (0, 4)),       # nothing divides: chunk after chunk
])
def test_workload_layouts(driver, tpc, tiles_n, n_chunks, forced, want):
    g, band, ok = run(driver, "chunk", tpc, tiles_n, n_chunks, forced, CONC)
    assert ok == "ok" and (int(g), int(band)) == want
