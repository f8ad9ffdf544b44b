"""Graph capture of the layer's calls (launch-gap removal, "Add forward all-gather overlap",
follow-up on CPU launch timing): on a stream under capture, agmm_chunked and gemm_rs_chunked take
the per-chunk event path, whose copies, events and launches a graph can hold.  One captured pass
of gather + column GEMM, reduce-scatter mirror, boundary epilogue and delayed-TP accumulation is
replayed several times, with eager work and NaN-poisoned outputs between the replays, and each
replay is compared bit for bit with the same calls run eagerly (on the default staged path)."""
import numpy as np
import pytest

from sp_transformer_linear_amd import synth
from tests.util import to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]


def gen(seed, key, rows, cols, var=1.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)))


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


class Layer:
    """Buffers of one pass: gather + column GEMM (tp=4, 256 rows per rank), the reduce-scatter
    mirror of the row GEMM, the boundary epilogue of the own rows and a delayed-TP step."""

    def __init__(self, torch, seed, tp=4, rows=256, K=512, N=512, H=512):
        bf = torch.bfloat16
        self.tp, self.rows = tp, rows
        M = tp * rows
        self.shards = [to_dev(gen(seed, (0, q), rows, K)) for q in range(tp)]
        self.w1 = to_dev(gen(seed, (1,), K, N, 1.0 / K))
        self.w2 = to_dev(gen(seed, (2,), N, H, 1.0 / N))
        self.peers = [to_dev(gen(seed, (3, p), rows, H, 0.02)) for p in range(tp - 1)]
        self.residual = to_dev(gen(seed, (4,), rows, H))
        self.gamma = (1.0 + to_dev(gen(seed, (5,), 1, H, 0.01)).float()).to(bf).reshape(H)
        self.xg = torch.empty((M, K), dtype=bf, device="cuda")
        self.y = torch.empty((M, N), dtype=bf, device="cuda")
        self.part = torch.empty((M, H), dtype=bf, device="cuda")
        self.dst = [None] + [torch.empty((rows, H), dtype=bf, device="cuda") for _ in range(tp - 1)]
        self.h = torch.empty((rows, H), dtype=bf, device="cuda")
        self.yn = torch.empty((rows, H), dtype=bf, device="cuda")
        self.x_dtp = torch.empty((rows, H), dtype=bf, device="cuda")
        self.y_dtp = torch.empty((rows, H), dtype=bf, device="cuda")

    def outputs(self):
        return [self.xg, self.y, self.part, *self.dst[1:], self.h, self.yn, self.x_dtp, self.y_dtp]

    def run(self, sptl, ctx):
        sptl.agmm_chunked(self.shards, self.xg, self.w1, self.y, n_chunks=self.tp, rank=0, ctx=ctx)
        sptl.gemm_rs_chunked(self.y, self.w2, self.part, self.dst, rank=0, ctx=ctx)
        own = self.part[:self.rows]
        sptl.reduce_residual_rmsnorm([own] + self.peers, self.residual, self.gamma, 1e-6, self.yn,
                                     residual_out=self.h, ctx=ctx)
        self.x_dtp.copy_(self.residual)  # a plain device copy kernel, capturable
        sptl.dtp_accumulate(self.x_dtp, own, self.peers, self.gamma, 1e-6, self.y_dtp, tp=self.tp, delta=1,
                            module_idx=1, ctx=ctx)


def snapshot(torch, L):
    return [t.clone() for t in L.outputs()]


def same(torch, got, want):
    return all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(got, want))


def test_graph_replays_match_eager(env):
    torch, sptl, ctx = env
    L = Layer(torch, 31)
    L.run(sptl, ctx)  # eager, staged path
    torch.cuda.synchronize()
    ctx.check()
    want = snapshot(torch, L)
    # the copy stream of the per-chunk path exists before the capture
    ctx.set_copy_mode("events")
    L.run(sptl, ctx)
    torch.cuda.synchronize()
    ctx.set_copy_mode("staged")
    assert same(torch, L.outputs(), want), "event path differs from the staged path"

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        L.run(sptl, ctx)
    torch.cuda.synchronize()
    scratch_a = torch.empty((1024, 512), dtype=torch.bfloat16, device="cuda")
    scratch_p = torch.empty((1024, 512), dtype=torch.bfloat16, device="cuda")
    for i in range(4):
        print(f"replay {i}", flush=True)
        for t in L.outputs():
            t.fill_(float("nan"))
        sptl.gemm_partial(L.xg if i % 2 else scratch_a.zero_(), L.w1, scratch_p, ctx=ctx)  # eager work between
        g.replay()
        torch.cuda.synchronize()
        ctx.check()
        assert same(torch, L.outputs(), want), f"replay {i} differs from the eager pass"

    # new inputs: the graph reads the buffers' current contents
    L2 = Layer(torch, 32)
    for a, b in zip(L.shards + L.peers + [L.residual, L.w1, L.w2, L.gamma],
                    L2.shards + L2.peers + [L2.residual, L2.w1, L2.w2, L2.gamma]):
        a.copy_(b)
    L2.run(sptl, ctx)
    torch.cuda.synchronize()
    want2 = snapshot(torch, L2)
    g.replay()
    torch.cuda.synchronize()
    ctx.check()
    assert same(torch, L.outputs(), want2), "replay on new inputs differs from the eager pass"
    del g


def test_capture_rejects_what_needs_the_worker(env):
    torch, sptl, ctx = env
    a = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    p = a.data_ptr()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream().cuda_stream
        rc_timing = sptl.raw_agmm_chunked(ctx.handle, 512, 256, 256, 2, 2, 0, [p, p], p, p, p, 0, cs, None, 1)
        rc_noalloc = sptl.raw_agmm_chunked_noalloc(ctx.handle, 512, 256, 256, 2, 2, 0, [p, p], p, p, p, 0, cs)
        a.add_(1)  # the graph must hold some work
    torch.cuda.synchronize()
    assert rc_timing == 8, sptl.last_error()
    assert rc_noalloc == 8, sptl.last_error()
    del g
