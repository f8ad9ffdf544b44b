"""Row-parallel GEMM with the reduce-scatter's sends overlapped (gemm_rs_chunked) on the GPU.

The partial is computed slice by slice in send order and every peer slice is copied out by the
copy engines as soon as its rows are written ("Potential Solution" of the AReaL async-TP issue:
the reduce-scatter at the end of a sub-layer).  Checked: the partial bit for bit equal to
gemm_partial (same kernel family, one K order), every destination bit for bit equal to its slice,
and the partial against the float64 oracle.  partial and the destinations are NaN-poisoned first,
so a copy released before its slice's rows were written and visible would leave NaN behind.
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import ROOT, assert_within, bf16_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    ctx = sptl.Context(0)
    yield torch, sptl, ctx
    torch.cuda.synchronize()
    ctx.close()


def gen(seed, key, rows, cols, var=1.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)))


def run_rs(env, M, K, H, tp, rank, seed, oracle=True, in_place=(), n_chunks=None):
    torch, sptl, ctx = env
    a_b = gen(seed, (3,), M, K)
    w_b = gen(seed, (2,), K, H, 1.0 / K)
    a, w = to_dev(a_b), to_dev(w_b)
    R = M // tp
    partial = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dst = [None if q == rank else (partial[q * R:(q + 1) * R] if q in in_place else
                                   torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda"))
           for q in range(tp)]
    sptl.gemm_rs_chunked(a, w, partial, dst, rank=rank, n_chunks=n_chunks, ctx=ctx)
    ref = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(a, w, ref, ctx=ctx)
    return a_b, w_b, partial, dst, ref


def check(env, a_b, w_b, partial, dst, ref, tp, rank, oracle=True):
    torch, sptl, ctx = env
    torch.cuda.synchronize()
    ctx.check()
    M = partial.shape[0]
    R = M // tp
    assert torch.equal(partial.view(torch.int16), ref.view(torch.int16)), "partial differs from gemm_partial"
    for q in range(tp):
        if q != rank:
            assert torch.equal(dst[q].view(torch.int16), partial[q * R:(q + 1) * R].view(torch.int16)), f"dst[{q}]"
    if oracle:
        want = O.gemm_partial(a_b, w_b)
        got = O.bf16_bits_to_f64(to_bits(partial))
        assert_within(got, want, bf16_tol(want), "partial vs oracle")


@pytest.mark.parametrize("M,K,H,tp,rank,in_place", [
    (8192, 4096, 4096, 8, 0, ()),      # the page's shape: 256-row tiles, the four-wave kernel
    (2048, 768, 1024, 4, 1, ()),       # short K: the eight-wave persistent kernel
    (768, 512, 384, 2, 1, ()),         # 384-row slices: 128-row tiles, ragged columns
    (1024, 256, 512, 4, 2, (3,)),      # one destination is the slice itself (left in place)
    (600, 256, 256, 2, 0, ()),         # 300-row slices fit no chunk tile: GEMM, then the copies
])
def test_rs_matches_gemm_partial_and_oracle(env, M, K, H, tp, rank, in_place):
    print(f"gemm_rs_chunked M={M} K={K} H={H} tp={tp} rank={rank} in_place={in_place}", flush=True)
    a_b, w_b, partial, dst, ref = run_rs(env, M, K, H, tp, rank, 400 + M % 97, in_place=in_place)
    check(env, a_b, w_b, partial, dst, ref, tp, rank)


@pytest.mark.parametrize("M,K,H,tp,rank,n_chunks,order,in_place", [
    (8192, 4096, 4096, 8, 3, 32, "interleaved", ()),   # four 256-row sub-slices per slice
    (8192, 4096, 4096, 8, 3, 32, "ring", ()),
    (2048, 768, 1024, 4, 1, 8, "interleaved", ()),       # short K, two sub-slices per slice
    (2048, 512, 512, 4, 2, 16, "interleaved", (0,)),     # 128-row sub-slices; one slice left in place
    (1024, 256, 512, 4, 2, 16, "interleaved", ()),       # 64-row sub-slices fit no chunk tile: event path
])
def test_rs_sub_slices(env, M, K, H, tp, rank, n_chunks, order, in_place):
    """Sub-slices in either send order give gemm_partial's bits, every destination whole."""
    torch, sptl, ctx = env
    print(f"gemm_rs_chunked M={M} K={K} H={H} tp={tp} rank={rank} n_chunks={n_chunks} {order}", flush=True)
    ctx.set_staging(order, 0)
    try:
        a_b, w_b, partial, dst, ref = run_rs(env, M, K, H, tp, rank, 450 + n_chunks, in_place=in_place,
                                             n_chunks=n_chunks)
        check(env, a_b, w_b, partial, dst, ref, tp, rank, oracle=M <= 2048)
    finally:
        ctx.set_staging("ring", 0)


def test_rs_back_to_back(env):
    """More calls in flight than signal sets, each with fresh inputs and poisoned outputs."""
    torch, sptl, ctx = env
    runs = [run_rs(env, 2048, 1024, 1024, 4, i % 4, 500 + i) for i in range(9)]
    for i, r in enumerate(runs):
        print(f"call {i}", flush=True)
        check(env, *r, tp=4, rank=i % 4, oracle=(i < 2))


CHILD = textwrap.dedent("""
    import sys, numpy as np, torch
    sys.path.insert(0, {root!r})
    from sp_transformer_linear_amd import sptl
    M, K, H, tp = 8192, 512, 1024, 8
    R = M // tp
    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((K, H), device="cuda", generator=g) / 32).to(torch.bfloat16)
    ctx = sptl.Context(0)
    ref = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(a, w, ref, ctx=ctx)
    ok = True
    for it in range(3):
        part = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        dst = [None] + [torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(tp - 1)]
        sptl.gemm_rs_chunked(a, w, part, dst, rank=0, ctx=ctx)
        torch.cuda.synchronize()
        ok = ok and torch.equal(part.view(torch.int16), ref.view(torch.int16))
        for q in range(1, tp):
            ok = ok and torch.equal(dst[q].view(torch.int16), part[q * R:(q + 1) * R].view(torch.int16))
    try:
        ctx.check()
        report = ""
    except sptl.SptlError as e:
        report = str(e)
    ctx.close()
    print("RESULT", int(ok), repr(report))
""")


def run_child(env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], env=env, capture_output=True, text=True,
                       timeout=240)
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("RESULT")]
    assert r.returncode == 0 and line, r.stdout[-2000:] + r.stderr[-2000:]
    _, ok, report = line[0].split(" ", 2)
    return ok == "1", eval(report)  # noqa: S307 - our own child's repr of a string


def test_rs_release_every_tile_child():
    """The fallback release (every tile writes its L2 back) gives the same bits."""
    ok, report = run_child({"SPTL_RS_FLUSH": "tile"})
    assert ok and report == ""


def test_rs_share_overrun_is_reported_child():
    """With the per-XCD share under-counted by one (a test aid), each XCD's last counted tile
    releases early and the tile after it counts past the share: sptl_ctx_check reports the call
    (its copies may be stale, so only the report is checked)."""
    _, report = run_child({"SPTL_RS_SHARE_SKEW": "1"})
    assert "XCD" in report
