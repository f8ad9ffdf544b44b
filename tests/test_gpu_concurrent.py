"""Calls running at the same time on two compute streams, against each call made alone.

Two arrangements: two contexts, one per stream, and one context serving both streams.  The
streams (default priority) get interleaved calls with no host wait between them: agmm_chunked
with the lead chunks copied by the launch's workgroups (tp = 8, 256-row chunks), at K = 2048 (the
four-wave kernel), and gemm_rs_chunked.  The calls of both streams share the copy engines and
the compute units, and in the second arrangement the context's signal sets too.  Every output
must equal the lone call's bit for bit, with the gathered rows and destinations NaN-poisoned.
"""
import numpy as np
import pytest

from sp_transformer_linear_amd import synth
from tests.util import to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

NAN = float("nan")


def gen(seed, key, rows, cols, var=1.0):
    return to_dev(synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var))))


def make_calls(torch, sptl):
    calls = []
    for seed, (tp, n, rows, K, N, rank) in enumerate(((8, 8, 256, 1024, 512, 3), (2, 2, 1024, 2048, 512, 1))):
        shards = [gen(60 + seed, (0, q), rows, K) for q in range(tp)]
        w = gen(60 + seed, (1,), K, N, 1.0 / K)

        def agmm(ctx, stream, shards=shards, w=w, tp=tp, n=n, rows=rows, K=K, N=N, rank=rank):
            with torch.cuda.stream(stream):
                xg = torch.full((tp * rows, K), NAN, dtype=torch.bfloat16, device="cuda")
                y = torch.full((tp * rows, N), NAN, dtype=torch.bfloat16, device="cuda")
                sptl.agmm_chunked(shards, xg, w, y, n_chunks=n, rank=rank, compute=stream, ctx=ctx)
            return [xg, y]
        calls.append(agmm)
    M, K, H, tp, rank = 2048, 512, 512, 4, 1
    a = gen(70, (0,), M, K)
    w2 = gen(70, (1,), K, H, 1.0 / K)

    def rs(ctx, stream):
        with torch.cuda.stream(stream):
            part = torch.full((M, H), NAN, dtype=torch.bfloat16, device="cuda")
            dst = [None if q == rank else torch.full((M // tp, H), NAN, dtype=torch.bfloat16, device="cuda")
                   for q in range(tp)]
            sptl.gemm_rs_chunked(a, w2, part, dst, rank=rank, stream=stream, ctx=ctx)
        return [part] + [d for d in dst if d is not None]
    calls.append(rs)
    return calls


@pytest.mark.parametrize("shared_ctx", [False, True])
def test_two_streams_match_lone_calls(shared_ctx):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    calls = make_calls(torch, sptl)
    ref_ctx = sptl.Context(0)
    ctxs = [sptl.Context(0)] if shared_ctx else [sptl.Context(0), sptl.Context(0)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    try:
        main = torch.cuda.current_stream()
        refs = []
        for i, c in enumerate(calls):
            print(f"lone call {i}", flush=True)
            outs = c(ref_ctx, main)
            torch.cuda.synchronize()
            ref_ctx.check()
            refs.append([to_bits(o) for o in outs])
        torch.cuda.synchronize()
        seq = np.random.default_rng(11).integers(0, len(calls), 32).tolist()
        print(f"shared_ctx={shared_ctx} sequence {seq}", flush=True)
        results = []
        for pos, i in enumerate(seq):  # alternate the streams, no host wait
            s = pos % 2
            results.append((i, calls[i](ctxs[s % len(ctxs)], streams[s])))
        torch.cuda.synchronize()
        for c in ctxs:
            c.check()
        for pos, (i, outs) in enumerate(results):
            for j, o in enumerate(outs):
                assert np.array_equal(to_bits(o), refs[i][j]), f"call {pos} (kind {i}), output {j}"
    finally:
        torch.cuda.synchronize()
        for c in ctxs:
            c.close()
        ref_ctx.close()
