"""GPU parity of agmm_chunked at the limits of its paths.

- the most ranks (SPTL_MAX_TP) with the most chunks the chunk-ordered (SDMA-staged) launch
  takes (64), so every landed-flag slot and signal set row is used;
- more chunks than that launch takes, which the per-chunk event path serves;
- the most chunks a call takes (SPTL_MAX_CHUNKS), one row each;
- the most copy pieces per chunk (16), forced in a child process by striping each chunk
  more finely than the engine count;
- the interleaved order and the link model with the most ranks, and the reduce-scatter with the
  most sub-slices.

Each case checks the gathered rows bit for bit against the concatenated shards and y against
the float64 oracle (fp32 tolerance: 1e-3 * ||oracle row||_2 / sqrt(N) + 1e-5).
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import ROOT, assert_within, fp32_tol, to_bits, to_dev

pytestmark = pytest.mark.gpu


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


def inputs(seed, tp, rows, K, N):
    shards = [synth.normal_bf16(seed, (0, q), rows, K, 1.0) for q in range(tp)]
    w = synth.normal_bf16(seed, (1,), K, N, float(np.sqrt(1.0 / K)))
    return shards, w


def run_and_check(env, tp, n_chunks, rows, K, N, rank, seed, copy=None):
    torch, sptl, ctx = env
    shards_b, w_b = inputs(seed, tp, rows, K, N)
    M = tp * rows
    shards = [to_dev(b) for b in shards_b]
    xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sptl.agmm_chunked(shards, xg, to_dev(w_b), y, n_chunks=n_chunks, rank=rank, ctx=ctx, copy=copy)
    torch.cuda.synchronize()
    ctx.check()
    assert np.array_equal(to_bits(xg), np.concatenate(shards_b)), "x_gathered != concat of the shards"
    _, y_want = O.agmm(shards_b, w_b)
    assert_within(y.cpu().numpy().astype(np.float64), y_want, fp32_tol(y_want), f"tp={tp} n={n_chunks} y")
    return y


def test_staged_at_max_tp_and_max_staged_chunks(env):
    torch, sptl, ctx = env
    from sp_transformer_linear_amd.sptl import MAX_TP
    tp, n_chunks, rows, K, N, rank = MAX_TP, 64, 128, 128, 256, MAX_TP - 1
    y = run_and_check(env, tp, n_chunks, rows, K, N, rank, seed=41)
    assert "sdma-striped" in ctx.info(), ctx.info()
    # the per-chunk event path gives the same bits
    y2 = run_and_check(env, tp, n_chunks, rows, K, N, rank, seed=41, copy=torch.cuda.Stream())
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def test_interleaved_links_at_max_tp(env):
    """The interleaved order and the link model with the most ranks: 63 peers share the copy
    engines round-robin (one each), and the bits are the default's."""
    torch, sptl, ctx = env
    from sp_transformer_linear_amd.sptl import MAX_TP
    tp, n_chunks, rows, K, N, rank = MAX_TP, 64, 128, 128, 256, 17
    y0 = run_and_check(env, tp, n_chunks, rows, K, N, rank, seed=44)
    ctx.set_staging("interleaved", 1)
    try:
        y1 = run_and_check(env, tp, n_chunks, rows, K, N, rank, seed=44)
    finally:
        ctx.set_staging("ring", 0)
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))


@pytest.mark.parametrize("tp,n_chunks,order,per", [(64, 64, "ring", 0), (8, 64, "interleaved", 0),
                                                   (8, 64, "interleaved", 2)])
def test_reduce_scatter_at_most_sub_slices(env, tp, n_chunks, order, per):
    """gemm_rs_chunked with the most sub-slices a call takes (64): 128-row sub-slices, the partial
    equal to gemm_partial bit for bit and every destination to its slice."""
    torch, sptl, ctx = env
    M, K, H, rank = 8192, 256, 256, 5
    a = to_dev(synth.normal_bf16(45, (0,), M, K, 1.0))
    w = to_dev(synth.normal_bf16(45, (1,), K, H, float(np.sqrt(1.0 / K))))
    R = M // tp
    part = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dst = [None if q == rank else torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda")
           for q in range(tp)]
    ref = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ctx.set_staging(order, per)
    try:
        sptl.gemm_rs_chunked(a, w, part, dst, rank=rank, n_chunks=n_chunks, ctx=ctx)
    finally:
        ctx.set_staging("ring", 0)
    sptl.gemm_partial(a, w, ref, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    assert torch.equal(part.view(torch.int16), ref.view(torch.int16))
    for q in range(tp):
        if q != rank:
            assert torch.equal(dst[q].view(torch.int16), part[q * R:(q + 1) * R].view(torch.int16)), f"dst[{q}]"


def test_more_chunks_than_the_staged_launch_takes(env):
    # 128 chunks of 128 rows (two per rank): beyond the chunk-ordered launch, so the call
    # takes the per-chunk event path
    run_and_check(env, 64, 128, 256, 64, 128, 5, seed=42)


def test_max_chunks_per_call(env):
    from sp_transformer_linear_amd.sptl import MAX_CHUNKS
    tp = 8
    rows = MAX_CHUNKS // tp  # one row per chunk
    run_and_check(env, tp, MAX_CHUNKS, rows, 64, 64, 3, seed=43)


CHILD = textwrap.dedent("""
    import sys, numpy as np, torch
    sys.path.insert(0, {root!r})
    from sp_transformer_linear_amd import sptl
    data = np.load({inp!r})
    tp = {tp}
    shards = [torch.from_numpy(data[f"s{{q}}"]).cuda().view(torch.bfloat16) for q in range(tp)]
    w = torch.from_numpy(data["w"]).cuda().view(torch.bfloat16)
    M, K = tp * shards[0].shape[0], shards[0].shape[1]
    xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, w.shape[1]), dtype=torch.float32, device="cuda")
    ctx = sptl.Context(0)
    for _ in range(3):  # the signal sets rotate: reuse after the first calls
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=tp, rank=1, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    info = ctx.info()
    ctx.close()
    np.savez({outp!r}, xg=xg.cpu().view(torch.int16).numpy(), y=y.cpu().numpy(), info=np.array(info))
""")


def test_most_pieces_per_chunk(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # 4 MiB chunks striped 16 ways per engine: capped at 16 pieces per chunk
    tp, rows, K, N = 2, 1024, 2048, 128
    shards_b, w_b = inputs(44, tp, rows, K, N)
    inp, outp = str(tmp_path / "in.npz"), str(tmp_path / "out.npz")
    np.savez(inp, w=w_b.view(np.int16), **{f"s{q}": s.view(np.int16) for q, s in enumerate(shards_b)})
    env = dict(os.environ, SPTL_SDMA_SPLIT="16")
    print("child process with SPTL_SDMA_SPLIT=16", flush=True)
    subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, inp=inp, outp=outp, tp=tp)], env=env, check=True,
                   timeout=300)
    got = np.load(outp)
    assert "sdma-striped" in str(got["info"]), str(got["info"])
    assert np.array_equal(got["xg"].view(np.uint16), np.concatenate(shards_b))
    _, y_want = O.agmm(shards_b, w_b)
    assert_within(got["y"].astype(np.float64), y_want, fp32_tol(y_want), "16-piece chunks y")
