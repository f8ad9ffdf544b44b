"""The epilogue's workgroups-per-CU cap (csrc/sptl_epilogue_plan.h), checked on the CPU.

The register-resident epilogue launch takes an unused dynamic LDS allocation so that only
about a target number of bytes of loads is in flight per CU.  A small driver is built with g++
from the header; properties checked:
  * the default target is 192 KiB, applied to launches of at most 48 rows per CU and to none
    larger; a forced target applies at any row count;
  * the allocation is whole KiB, leaves 1 KiB per workgroup for the kernel's own LDS, fits the
    per-workgroup limit, and lets the target's workgroup count (the target over the bytes per
    workgroup, rounded) reside on a CU, and no more when the kernel's own LDS takes the whole
    margin and a KiB step separates that count from the next;
  * the 4096-column shape of the workloads: 9 inputs (the 8 partial sums and the residual)
    hold 72 KiB of loads per workgroup and get 3 workgroups per CU at 8192 and 1024 rows, and
    no cap at 16384 rows.
"""
import os
import shutil
import subprocess

import pytest

from tests.util import ROOT

CSRC = os.path.join(ROOT, "sp_transformer_linear_amd", "csrc")
KiB = 1024
LDS_CU = 160 * KiB
CUS = 256


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("epi_plan") / "epi_plan")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "epilogue_plan_driver.cpp"),
                    "-o", exe], check=True, timeout=120)
    return exe


def caps(driver, cases):
    """cases: (bytes_per_wg, rows, target, forced, lds_per_cu, lds_per_block, cus) tuples."""
    text = "".join(" ".join(str(int(v)) for v in c) + "\n" for c in cases)
    out = subprocess.run([driver], input=text, check=True, capture_output=True, text=True,
                         timeout=30).stdout.splitlines()
    assert out[-1].startswith("target ")
    caps.target, caps.rows_per_cu = (int(v) for v in out[-1].split()[1::2])
    return [int(v) for v in out[:-1]]


def bytes_per_wg(n_in, hidden):
    """Loads in flight per workgroup: every thread holds all of its vectors of every input."""
    nv = hidden // 8
    vpt = 1 if nv <= 256 else 2 if nv <= 512 else 4
    threads = (-(-nv // vpt) + 63) // 64 * 64
    return threads * vpt * n_in * 16


def resident(dyn, own, lds_cu=LDS_CU):
    return lds_cu // (dyn + own)


def test_constants(driver):
    caps(driver, [])
    assert caps.target == 192 * KiB
    assert caps.rows_per_cu == 48


def test_workload_shapes(driver):
    """8192 and 1024 rows (32 and 4 rows per CU) at 4096 columns are capped; 16384 are not."""
    b9 = bytes_per_wg(9, 4096)
    assert b9 == 72 * KiB
    got = caps(driver, [(b9, 8192, 192 * KiB, 0, LDS_CU, LDS_CU, CUS),
                        (b9, 1024, 192 * KiB, 0, LDS_CU, LDS_CU, CUS),
                        (b9, 48 * CUS, 192 * KiB, 0, LDS_CU, LDS_CU, CUS),
                        (b9, 48 * CUS + 1, 192 * KiB, 0, LDS_CU, LDS_CU, CUS),
                        (b9, 16384, 192 * KiB, 0, LDS_CU, LDS_CU, CUS)])
    assert got[0] == got[1] == got[2] == 52 * KiB
    for own in (0, 512, KiB):
        assert resident(got[0], own) == 3
    assert got[3] == got[4] == 0


def test_forced_target_any_rows(driver):
    b9 = bytes_per_wg(9, 4096)
    got = caps(driver, [(b9, 1 << 20, 64 * KiB, 1, LDS_CU, LDS_CU, CUS),
                        (b9, 1 << 20, 64 * KiB, 0, LDS_CU, LDS_CU, CUS),
                        (b9, 8, 64 * KiB, 1, LDS_CU, LDS_CU, CUS)])
    assert got[0] == got[2] > 0 and got[1] == 0
    assert resident(got[0], KiB) == 1


def test_no_cap_cases(driver):
    """No target, no CUs, a zero-byte workgroup or a cap that would not fit a workgroup: 0."""
    got = caps(driver, [(72 * KiB, 64, 0, 0, LDS_CU, LDS_CU, CUS),
                        (72 * KiB, 64, 192 * KiB, 0, LDS_CU, LDS_CU, 0),
                        (0, 64, 192 * KiB, 0, LDS_CU, LDS_CU, CUS),
                        (72 * KiB, 64, 192 * KiB, 0, 0, LDS_CU, CUS),
                        # one workgroup per CU would need 159 KiB, above a 64 KiB block limit
                        (192 * KiB, 64, 192 * KiB, 0, LDS_CU, 64 * KiB, CUS),
                        # a CU's LDS too small for even the margin
                        (KiB, 64, 192 * KiB, 0, 4 * KiB, 4 * KiB, CUS)])
    assert got == [0] * len(got)


@pytest.mark.parametrize("lds_cu,lds_block", [(LDS_CU, LDS_CU), (LDS_CU, 64 * KiB), (64 * KiB, 64 * KiB)])
def test_allocation_properties(driver, lds_cu, lds_block):
    cases = []
    for n_in in range(1, 10):
        for hidden in (512, 1024, 2048, 3584, 4096, 8192):
            b = bytes_per_wg(n_in, hidden)
            for target in (16 * KiB, 64 * KiB, 192 * KiB, 512 * KiB):
                cases.append((b, 100, target, 0, lds_cu, lds_block, CUS))
    for (b, _, target, _, lc, lb, _), dyn in zip(cases, caps(driver, cases)):
        wgs = max(1, (target + b // 2) // b)
        if dyn == 0:
            # only when the allocation would be empty or above the per-workgroup limit
            assert (lc // wgs - KiB) // KiB * KiB <= 0 or (lc // wgs - KiB) // KiB * KiB > lb - KiB
            continue
        assert dyn % KiB == 0 and dyn <= lb - KiB
        for own in (0, KiB):
            assert resident(dyn, own, lc) >= wgs, (b, target, dyn)
        # whole KiB below lds/wgs - 1 KiB: wgs + 1 no longer fit once that step is below lds/(wgs+1)
        if lc // wgs - 2 * KiB >= lc // (wgs + 1):
            assert resident(dyn, KiB, lc) == wgs, (b, target, dyn)
