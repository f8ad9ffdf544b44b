"""The chunk order and link model of a context (sptl_ctx_set_staging) on the GPU.

Each chunk's matmul starts as soon as its chunk has arrived (AReaL "Potential Solution"), so the
order in which chunks are processed should be the order in which they arrive: peer by peer for
a ring, sub-chunk by sub-chunk for a direct gather over one link per peer.  The link model runs
each peer's copies on copy engines of its own.  No setting may change a bit: every output and
gather is compared with the default context's, x_gathered with the rank-major concatenation,
and y with the oracle, with x_gathered and y NaN-poisoned first; the settings are also switched
back and forth on one context between calls.
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

SETTINGS = [("interleaved", 0), ("ring", 1), ("ring", 2), ("interleaved", 2), ("interleaved", 16)]
SHAPES = [  # tp, n_chunks, rows per rank, K, N, rank
    (4, 8, 512, 512, 384, 1),      # two sub-chunks per rank
    (8, 16, 512, 256, 256, 5),     # tp = 8, two sub-chunks per rank
    (2, 8, 1024, 384, 512, 0),     # four sub-chunks per rank, one peer
    (4, 4, 256, 512, 384, 2),      # one chunk per rank: interleaved is the ring order
]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    ref = sptl.Context(0)
    alt = sptl.Context(0)
    yield torch, sptl, ref, alt
    torch.cuda.synchronize()
    alt.close()
    ref.close()


def test_staging_validation(env):
    torch, sptl, ref, alt = env
    h = alt.handle
    assert sptl._lib.sptl_ctx_set_staging(h, 2, 0) == 6
    assert sptl._lib.sptl_ctx_set_staging(h, -1, 0) == 6
    assert sptl._lib.sptl_ctx_set_staging(h, 0, -1) == 6
    assert sptl._lib.sptl_ctx_set_staging(h, 0, 17) == 6
    alt.set_staging("ring", 0)


def inputs(seed, tp, rows, K, N):
    shards_b = [synth.normal_bf16(seed, (0, q), rows, K, 1.0) for q in range(tp)]
    w_b = synth.normal_bf16(seed, (1,), K, N, float(np.sqrt(1.0 / K)))
    return shards_b, w_b


@pytest.mark.parametrize("tp,n_chunks,rows,K,N,rank", SHAPES)
def test_orders_and_links_bitwise(env, tp, n_chunks, rows, K, N, rank):
    torch, sptl, ref, alt = env
    print(f"staging tp={tp} n={n_chunks} rows={rows} K={K} N={N} rank={rank}", flush=True)
    shards_b, w_b = inputs(900 + tp * 10 + n_chunks, tp, rows, K, N)
    M = tp * rows
    shards = [to_dev(b) for b in shards_b]
    w = to_dev(w_b)

    def run(ctx):
        xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=n_chunks, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
        ctx.check()
        return to_bits(xg), to_bits(y)

    x0, y0 = run(ref)
    assert np.array_equal(x0, np.concatenate(shards_b))
    _, want = O.agmm(shards_b, w_b)
    assert_within(O.bf16_bits_to_f64(y0), want, bf16_tol(want), "default vs oracle")
    try:
        for order, per in SETTINGS + SETTINGS[:2]:  # the first two again, after the others
            alt.set_staging(order, per)
            x, y = run(alt)
            assert np.array_equal(x, x0), f"x_gathered, {order}/{per}"
            assert np.array_equal(y, y0), f"y, {order}/{per}"
    finally:
        alt.set_staging("ring", 0)


def test_interleaved_event_path_and_timeline(env):
    """The per-chunk event path takes the interleaved order too; the timeline of a staged call under
    the link model has every peer chunk land before its GEMM starts."""
    torch, sptl, ref, alt = env
    tp, n_chunks, rows, K, N, rank = 4, 8, 512, 512, 384, 3
    shards_b, w_b = inputs(977, tp, rows, K, N)
    M = tp * rows
    shards = [to_dev(b) for b in shards_b]
    w = to_dev(w_b)
    xg0 = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg0, w, y0, n_chunks=n_chunks, rank=rank, ctx=ref)
    try:
        alt.set_copy_mode("events")
        alt.set_staging("interleaved", 0)
        xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=n_chunks, rank=rank, ctx=alt)
        torch.cuda.synchronize()
        alt.check()
        assert torch.equal(xg.view(torch.int16), xg0.view(torch.int16))
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
        alt.set_copy_mode("staged")
        alt.set_staging("interleaved", 2)
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=n_chunks, rank=rank, ctx=alt, timing=True)
        torch.cuda.synchronize()
        alt.check()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
        tl = alt.timeline(n_chunks)
        cpr = n_chunks // tp
        for c in range(n_chunks):
            if rank * cpr <= c < (rank + 1) * cpr:
                continue
            copy_start, copy_end, gemm_start, gemm_end = tl[c]
            assert 0.0 <= copy_end <= gemm_start + 1e-3 < gemm_end + 1e-3, f"chunk {c}: {tl[c]}"
    finally:
        alt.set_copy_mode("staged")
        alt.set_staging("ring", 0)


def test_links_reduce_scatter_and_backward_bitwise(env):
    """The link model on the reduce-scatter mirror (each peer slice pushed on its peer's engines)
    and on the backward's re-gather gives the default context's bits."""
    torch, sptl, ref, alt = env
    tp, M, K, H, rank = 4, 2048, 512, 512, 2
    a = to_dev(synth.normal_bf16(991, (0,), M, K, 1.0))
    w = to_dev(synth.normal_bf16(991, (1,), K, H, float(np.sqrt(1.0 / K))))
    R = M // tp

    def rs(ctx):
        part = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        dst = [None if q == rank else torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda")
               for q in range(tp)]
        sptl.gemm_rs_chunked(a, w, part, dst, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
        ctx.check()
        return [to_bits(part)] + [to_bits(d) for d in dst if d is not None]

    tpb, rows, Kb, N, rb = 4, 256, 512, 384, 1
    shards = [to_dev(synth.normal_bf16(992, (0, q), rows, Kb, 1.0)) for q in range(tpb)]
    wb = to_dev(synth.normal_bf16(992, (1,), Kb, N, float(np.sqrt(1.0 / Kb))))
    dy = to_dev(synth.normal_bf16(992, (2,), tpb * rows, N, float(np.sqrt(1.0 / N))))

    def bwd(ctx):
        xg = torch.full((tpb * rows, Kb), float("nan"), dtype=torch.bfloat16, device="cuda")
        dx = torch.full((tpb * rows, Kb), float("nan"), dtype=torch.bfloat16, device="cuda")
        dw = torch.full((Kb, N), float("nan"), dtype=torch.float32, device="cuda")
        sptl.agmm_backward(shards, xg, wb, dy, dx, dw, rank=rb, ctx=ctx)
        torch.cuda.synchronize()
        ctx.check()
        return [to_bits(xg), to_bits(dx), to_bits(dw)]

    want_rs, want_bwd = rs(ref), bwd(ref)
    for q in range(tp):
        if q != rank:  # each pushed slice is the partial's rows of that peer
            assert np.array_equal(want_rs[1 + q - (q > rank)], want_rs[0][q * R:(q + 1) * R])
    try:
        for per in (2, 1, 16):
            alt.set_staging("ring", per)
            for i, (g, w_) in enumerate(zip(rs(alt), want_rs)):
                assert np.array_equal(g, w_), f"reduce-scatter output {i}, {per} engines per peer"
            for i, (g, w_) in enumerate(zip(bwd(alt), want_bwd)):
                assert np.array_equal(g, w_), f"backward output {i}, {per} engines per peer"
    finally:
        alt.set_staging("ring", 0)
