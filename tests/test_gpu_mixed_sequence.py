"""A seeded random sequence of calls of every kind on one context and one stream, with no host
wait between them, against each call made alone on another context.

The calls share per-context state on the GPU: signal sets, end counters, landed flags, the
counters of the lead-chunk copy, the reduce-scatter's slice counters and the no-allocation
entry point's scratch.  Each kind of call also reuses one gathered buffer, NaN-poisoned on the
stream before every call, so a call's copies must not start before the work queued ahead of
it.  Kinds: agmm_chunked with the lead chunks copied by the launch's workgroups (eight-wave and
four-wave kernels), with the interleaved order under the link model, gemm_rs_chunked,
agmm_backward and agmm_chunked_noalloc.  Every output must equal the lone call's bit for bit.
"""
import numpy as np
import pytest

from sp_transformer_linear_amd import synth
from tests.util import to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

NAN = float("nan")


def gen(seed, key, rows, cols, var=1.0):
    return to_dev(synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var))))


class Agmm:
    def __init__(self, torch, sptl, seed, tp, n, rows, K, N, rank, staging=None, noalloc=False):
        self.torch, self.sptl = torch, sptl
        self.tp, self.n, self.rank, self.staging, self.noalloc = tp, n, rank, staging, noalloc
        self.M, self.K, self.N = tp * rows, K, N
        self.shards = [gen(seed, (0, q), rows, K) for q in range(tp)]
        self.w = gen(seed, (1,), K, N, 1.0 / K)
        self.xg = torch.empty((self.M, K), dtype=torch.bfloat16, device="cuda")
        self.name = f"agmm tp={tp} n={n} M={self.M} K={K} N={N} rank={rank} staging={staging} noalloc={noalloc}"

    def __call__(self, ctx):
        torch, sptl = self.torch, self.sptl
        self.xg.fill_(NAN)
        y = torch.full((self.M, self.N), NAN, dtype=torch.bfloat16, device="cuda")
        if self.staging:
            ctx.set_staging(*self.staging)
        try:
            if self.noalloc:
                rc = sptl.raw_agmm_chunked_noalloc(ctx.handle, self.M, self.K, self.N, self.tp, self.n, self.rank,
                                                   [s.data_ptr() for s in self.shards], self.xg.data_ptr(),
                                                   self.w.data_ptr(), y.data_ptr(), sptl.BF16,
                                                   torch.cuda.current_stream().cuda_stream)
                assert rc == 0, sptl.last_error()
            else:
                sptl.agmm_chunked(self.shards, self.xg, self.w, y, n_chunks=self.n, rank=self.rank, ctx=ctx)
        finally:
            if self.staging:
                ctx.set_staging("ring", 0)
        return [y]


class Rs:
    def __init__(self, torch, sptl, seed, tp, M, K, H, rank):
        self.torch, self.sptl, self.tp, self.M, self.H, self.rank = torch, sptl, tp, M, H, rank
        self.a = gen(seed, (2,), M, K)
        self.w = gen(seed, (3,), K, H, 1.0 / K)
        self.name = f"gemm_rs_chunked tp={tp} M={M} K={K} H={H} rank={rank}"

    def __call__(self, ctx):
        torch = self.torch
        part = torch.full((self.M, self.H), NAN, dtype=torch.bfloat16, device="cuda")
        dst = [None if q == self.rank else torch.full((self.M // self.tp, self.H), NAN, dtype=torch.bfloat16,
                                                       device="cuda") for q in range(self.tp)]
        self.sptl.gemm_rs_chunked(self.a, self.w, part, dst, rank=self.rank, ctx=ctx)
        return [part] + [d for d in dst if d is not None]


class Bwd:
    def __init__(self, torch, sptl, seed, tp, rows, K, N, rank):
        self.torch, self.sptl, self.rank = torch, sptl, rank
        self.M, self.K, self.N = tp * rows, K, N
        self.shards = [gen(seed, (4, q), rows, K) for q in range(tp)]
        self.w = gen(seed, (5,), K, N, 1.0 / K)
        self.dy = gen(seed, (6,), self.M, N, 1.0 / N)
        self.xg = torch.empty((self.M, K), dtype=torch.bfloat16, device="cuda")
        self.name = f"agmm_backward tp={tp} M={self.M} K={K} N={N} rank={rank}"

    def __call__(self, ctx):
        torch = self.torch
        self.xg.fill_(NAN)
        dx = torch.full((self.M, self.K), NAN, dtype=torch.bfloat16, device="cuda")
        dw = torch.full((self.K, self.N), NAN, dtype=torch.float32, device="cuda")
        self.sptl.agmm_backward(self.shards, self.xg, self.w, self.dy, dx, dw, rank=self.rank, ctx=ctx)
        return [dx, dw]


def test_mixed_sequence_matches_lone_calls():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    kinds = [
        Agmm(torch, sptl, 41, 8, 8, 256, 1024, 512, 2),                      # lead copy, eight-wave kernel
        Agmm(torch, sptl, 42, 4, 8, 512, 512, 384, 1),                       # lead copy, two sub-chunks per rank
        Agmm(torch, sptl, 43, 2, 2, 1024, 2048, 512, 1),                     # four-wave kernel, one lead chunk
        Agmm(torch, sptl, 44, 4, 16, 1024, 512, 256, 3, staging=("interleaved", 2)),
        Rs(torch, sptl, 45, 4, 2048, 512, 512, 2),
        Bwd(torch, sptl, 46, 4, 256, 512, 384, 1),
        Agmm(torch, sptl, 47, 4, 8, 256, 512, 384, 0, noalloc=True),
    ]
    ref_ctx = sptl.Context(0)
    ctx = sptl.Context(0)
    try:
        refs = []
        for k in kinds:
            print(f"lone call: {k.name}", flush=True)
            outs = k(ref_ctx)
            torch.cuda.synchronize()
            ref_ctx.check()
            refs.append([to_bits(o) for o in outs])
        seq = np.random.default_rng(2024).integers(0, len(kinds), 48).tolist()
        print(f"sequence: {seq}", flush=True)
        results = [kinds[i](ctx) for i in seq]  # no host wait between the calls
        torch.cuda.synchronize()
        ctx.check()
        for pos, (i, outs) in enumerate(zip(seq, results)):
            for j, o in enumerate(outs):
                assert np.array_equal(to_bits(o), refs[i][j]), f"call {pos} ({kinds[i].name}), output {j}"
    finally:
        torch.cuda.synchronize()
        ctx.close()
        ref_ctx.close()
