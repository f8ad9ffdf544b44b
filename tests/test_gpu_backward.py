"""Backward of the gather + column GEMM (agmm_backward) on the GPU, against the float64 oracle.

The re-gather of the activation runs on the copy engines under the input-gradient GEMM
("Add forward all-gather overlap", "Scope": the backward gathers, not yet overlapped there).
Checked: x_gathered bit for bit against the rank-major concat; dx = dy w^T and dw = x^T dy
against the oracle (bf16 outputs 8e-3 |o| + 1e-2; fp32 outputs 1e-3 ||oracle row||_2 / sqrt(N)
+ 1e-5); the transposed-operand kernels bit for bit against the row-major kernel on explicitly
transposed copies (one K order); every copy mode bit for bit; a poisoned, freshly cached
x_gathered; calls back to back; and the largest workload's shapes in full.
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, fp32_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    ctx = sptl.Context(0)
    alt = sptl.Context(0)
    yield torch, sptl, ctx, alt
    torch.cuda.synchronize()
    alt.close()
    ctx.close()


def gen(seed, key, rows, cols, var=1.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)))


def host(t):
    import torch
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    return O.bf16_bits_to_f64(to_bits(t))


class Case:
    def __init__(self, torch, tp, rows, K, N, seed):
        self.tp, self.M, self.K, self.N = tp, tp * rows, K, N
        self.shards_b = [gen(seed, (0, q), rows, K) for q in range(tp)]
        self.w_b = gen(seed, (1,), K, N, 1.0 / K)
        self.dy_b = gen(seed, (2,), tp * rows, N, 0.02)
        self.shards = [to_dev(b) for b in self.shards_b]
        self.w, self.dy = to_dev(self.w_b), to_dev(self.dy_b)

    def outputs(self, torch, dw_f32=True):
        nan = float("nan")
        xg = torch.full((self.M, self.K), nan, dtype=torch.bfloat16, device="cuda")
        dx = torch.full((self.M, self.K), nan, dtype=torch.bfloat16, device="cuda")
        dw = torch.full((self.K, self.N), nan, dtype=torch.float32 if dw_f32 else torch.bfloat16, device="cuda")
        return xg, dx, dw


CASES = [
    # tp, rows per rank, K (hidden), N (n_local), rank
    (2, 128, 256, 512, 0),
    (3, 100, 200, 136, 2),      # ragged: the dw reduction (300) ends mid-stage, K and N mid-tile
    (4, 300, 320, 264, 1),
    (8, 64, 128, 256, 3),
    (4, 512, 512, 256, 0),      # dw reduction 2048: the four-wave k-major kernel
    (2, 256, 264, 2048, 1),     # dx reduction 2048: the four-wave n-major kernel
]


@pytest.mark.parametrize("dw_f32", [True, False])
@pytest.mark.parametrize("tp,rows,K,N,rank", CASES)
def test_backward_parity(env, tp, rows, K, N, rank, dw_f32):
    torch, sptl, ctx, alt = env
    print(f"agmm_backward tp={tp} rows={rows} K={K} N={N} rank={rank} dw_f32={dw_f32}", flush=True)
    c = Case(torch, tp, rows, K, N, 40 + tp * 3 + rows)
    xg, dx, dw = c.outputs(torch, dw_f32)
    sptl.agmm_backward(c.shards, xg, c.w, c.dy, dx, dw, rank=rank, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    x_want, dx_want, dw_want = O.agmm_backward(c.shards_b, c.w_b, c.dy_b)
    assert np.array_equal(to_bits(xg), np.concatenate(c.shards_b)), "x_gathered is not the rank-major concat"
    assert_within(host(dx), dx_want, bf16_tol(dx_want), "dx")
    assert_within(host(dw), dw_want, fp32_tol(dw_want) if dw_f32 else bf16_tol(dw_want), "dw")
    # the transposed-operand kernels against the row-major kernel on transposed copies
    wt = c.w.t().contiguous()
    xt = xg.t().contiguous()
    dx_rm = torch.empty_like(dx)
    dw_rm = torch.empty_like(dw)
    sptl.gemm_partial(c.dy, wt, dx_rm, ctx=ctx)
    if c.M % 8 == 0:  # the row-major kernel needs its reduction (here M) in whole 16-byte pieces
        sptl.gemm_partial(xt, c.dy, dw_rm, ctx=ctx)
    torch.cuda.synchronize()
    iv = torch.int32 if dw_f32 else torch.int16
    assert torch.equal(dx.view(torch.int16), dx_rm.view(torch.int16)), "dx differs from the row-major kernel"
    if c.M % 8 == 0:
        assert torch.equal(dw.view(iv), dw_rm.view(iv)), "dw differs from the row-major kernel"


@pytest.mark.parametrize("mode,wgs", [("events", 0), ("blit", 0), ("blit", 5), ("serial", 0)])
def test_backward_modes_bitwise(env, mode, wgs):
    torch, sptl, ctx, alt = env
    c = Case(torch, 4, 256, 384, 256, 77)
    ref = c.outputs(torch)
    sptl.agmm_backward(c.shards, ref[0], c.w, c.dy, ref[1], ref[2], rank=1, ctx=ctx)
    alt.set_copy_mode(mode, wgs)
    try:
        got = c.outputs(torch)
        sptl.agmm_backward(c.shards, got[0], c.w, c.dy, got[1], got[2], rank=1, ctx=alt)
        torch.cuda.synchronize()
        alt.check()
    finally:
        alt.set_copy_mode("staged")
    ctx.check()
    for a, b, what in zip(ref, got, ("x_gathered", "dx", "dw")):
        iv = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(iv), b.view(iv)), what


def test_backward_stale_cache_and_back_to_back(env):
    """x_gathered poisoned and just read by a kernel (its lines cached) before each call; more
    calls in flight than the stager has signal sets."""
    torch, sptl, ctx, alt = env
    cases = [Case(torch, 4, 256, 256, 256, 90 + i) for i in range(9)]
    xg = torch.full((1024, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    scratch = torch.empty((1024, 256), dtype=torch.bfloat16, device="cuda")
    outs = []
    for i, c in enumerate(cases):
        xg.fill_(float("nan"))
        sptl.gemm_partial(xg, c.w, scratch, ctx=ctx)  # reads the poisoned rows into the caches
        _, dx, dw = c.outputs(torch)
        sptl.agmm_backward(c.shards, xg, c.w, c.dy, dx, dw, rank=i % 4, ctx=ctx)
        outs.append((dx, dw, xg.clone()))
    torch.cuda.synchronize()
    ctx.check()
    for i, (c, (dx, dw, xgi)) in enumerate(zip(cases, outs)):
        print(f"call {i}", flush=True)
        assert torch.equal(xgi, torch.cat(c.shards)), f"x_gathered, call {i}"
        assert not torch.isnan(dw).any(), f"dw read a stale row, call {i}"
        if i < 2:
            _, dx_want, dw_want = O.agmm_backward(c.shards_b, c.w_b, c.dy_b)
            assert_within(host(dx), dx_want, bf16_tol(dx_want), "dx")
            assert_within(host(dw), dw_want, fp32_tol(dw_want), "dw")


def test_backward_fullsize(env):
    """The largest workload's shapes (65536 x 4096 gathered, 4096 x 4096 weight, tp 8), every
    element of dx and dw against the oracle."""
    torch, sptl, ctx, alt = env
    wl = synth.WORKLOADS["msweep_65536x4096"]
    print(f"agmm_backward {wl.name}", flush=True)
    shards_b = [wl.shard(q) for q in range(wl.tp)]
    w_b = wl.w_col()
    dy_b = synth.normal_bf16(wl.seed, (99,), wl.M, wl.N, float(np.sqrt(0.02)))
    shards = [to_dev(b) for b in shards_b]
    xg = torch.empty((wl.M, wl.K), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((wl.M, wl.K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((wl.K, wl.N), dtype=torch.float32, device="cuda")
    sptl.agmm_backward(shards, xg, to_dev(w_b), to_dev(dy_b), dx, dw, rank=0, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    assert torch.equal(xg, torch.cat(shards)), "x_gathered != rank-major concat of the shards"
    del xg, shards
    got_dx, got_dw = host(dx), host(dw)
    del dx, dw
    _, dx_want, dw_want = O.agmm_backward(shards_b, w_b, dy_b)
    for r0 in range(0, wl.M, 4096):
        want = dx_want[r0:r0 + 4096]
        assert_within(got_dx[r0:r0 + 4096], want, bf16_tol(want), f"dx rows [{r0}, {r0 + 4096})")
    assert_within(got_dw, dw_want, fp32_tol(dw_want), "dw")
