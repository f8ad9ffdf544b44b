"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Every element of every output is compared with the float64 oracle: the oracle runs block by
block (BLOCK rows at a time) on the same seeded inputs, and each block of the GPU output is
checked element by element against it.  Whole-tensor properties are checked too: the gathered
activations equal the rank-major concat of the shards bit for bit, the chunked result equals a
monolithic GEMM of the gathered rows bit for bit, and the epilogue of a leading slice of rows
equals the same rows of the full call bit for bit.  Tolerances as in test_gpu_parity.py:
fp32 outputs 1e-3 * ||oracle row||_2 / sqrt(N) + 1e-5, bf16 outputs 8e-3 * |oracle| + 1e-2.
"""
import time

import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, fp32_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

BLOCK = 2048  # oracle rows per block (any split gives the same float64 rows)


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


def host_values(t):
    """Host copy of a bf16 (as float64 values) or fp32 (as float64) GPU tensor."""
    import torch
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    return O.bf16_bits_to_f64(to_bits(t))


def compare_blocks(got_host, want_block, tol_fn, what, rows, block=BLOCK):
    """got_host: full host array; want_block(r0, r1): oracle rows [r0, r1)."""
    t0 = time.perf_counter()
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        want = want_block(r0, r1)
        assert_within(got_host[r0:r1], want, tol_fn(want), f"{what} rows [{r0}, {r1})")
    print(f"  {what}: {rows} rows against the oracle in {time.perf_counter() - t0:.1f} s", flush=True)


def run_agmm(env, wl, y_f32):
    torch, sptl, ctx = env
    print(f"agmm {wl.name} y={'fp32' if y_f32 else 'bf16'}", flush=True)
    shards_b = [wl.shard(q) for q in range(wl.tp)]
    shards = [to_dev(b) for b in shards_b]
    w_b = wl.w_col()
    w = to_dev(w_b)
    xg = torch.empty((wl.M, wl.K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((wl.M, wl.N), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg, w, y, n_chunks=wl.n_chunks, rank=0, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    assert torch.equal(xg, torch.cat(shards)), "x_gathered != rank-major concat of the shards"
    # chunked == monolithic, bit for bit
    y_mono = torch.empty_like(y)
    sptl.gemm_partial(xg, w, y_mono, ctx=ctx)
    torch.cuda.synchronize()
    iv = torch.int32 if y_f32 else torch.int16
    assert torch.equal(y.view(iv), y_mono.view(iv)), "chunked != monolithic"
    del y_mono, xg, shards
    got = host_values(y)
    del y
    per_rank = wl.M // wl.tp

    def want(r0, r1):
        # rows [r0, r1) of the gathered sequence lie in one rank's shard (the block divides M / tp)
        q = r0 // per_rank
        assert (r1 - 1) // per_rank == q
        _, yb = O.agmm([shards_b[q][r0 - q * per_rank:r1 - q * per_rank]], w_b)
        return yb

    compare_blocks(got, want, fp32_tol if y_f32 else bf16_tol, f"{wl.name} agmm y", wl.M,
                   block=min(BLOCK, per_rank))
    return ctx.info()


@pytest.mark.parametrize("name,y_f32", [("h100_page_8192x4096", False), ("h100_page_8192x4096", True),
                                        ("qwen2_7b_tp4_16384", False), ("msweep_65536x4096", False)])
def test_agmm_fullsize(env, name, y_f32):
    info = run_agmm(env, synth.WORKLOADS[name], y_f32)
    assert "sdma-striped" in info, f"the benchmarked staging path was not used: {info}"


@pytest.mark.parametrize("name", ["h100_page_8192x4096", "qwen2_7b_tp4_16384", "msweep_65536x4096",
                                  "dtp_qwen3_0p6b_tp4"])
def test_gemm_partial_fullsize(env, name):
    torch, sptl, ctx = env
    wl = synth.WORKLOADS[name]
    print(f"gemm_partial {wl.name}: {wl.M} x {wl.K_row} x {wl.H}", flush=True)
    a_b = wl.a_row()
    w_b = wl.w_row()
    out = torch.empty((wl.M, wl.H), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(to_dev(a_b), to_dev(w_b), out, ctx=ctx)
    torch.cuda.synchronize()
    got = host_values(out)
    del out
    compare_blocks(got, lambda r0, r1: O.gemm_partial(a_b[r0:r1], w_b), bf16_tol, f"{wl.name} partial", wl.M)


@pytest.mark.parametrize("name", ["h100_page_8192x4096", "qwen2_7b_tp4_16384", "msweep_65536x4096",
                                  "dtp_qwen3_0p6b_tp4"])
def test_reduce_residual_rmsnorm_fullsize(env, name):
    torch, sptl, ctx = env
    wl = synth.WORKLOADS[name]
    print(f"reduce_residual_rmsnorm {wl.name}: P={wl.P}, {wl.M} x {wl.H}", flush=True)
    parts_b = [wl.partial(p) for p in range(wl.P)]
    res_b = wl.residual()
    g_b = wl.gamma()
    parts = [to_dev(b) for b in parts_b]
    res = to_dev(res_b)
    y = torch.empty_like(res)
    h = torch.empty_like(res)
    sptl.reduce_residual_rmsnorm(parts, res, to_dev(g_b), wl.eps, y, residual_out=h, ctx=ctx)
    torch.cuda.synchronize()
    # rows are independent: the first rows of the full call equal a call on those rows alone
    y2 = torch.empty_like(y[:333])
    sptl.reduce_residual_rmsnorm([p[:333] for p in parts], res[:333], to_dev(g_b), wl.eps, y2, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y[:333].view(torch.int16))
    del parts, res, y2
    got_h, got_y = host_values(h), host_values(y)
    del h, y
    cache = {}

    def oracle_block(r0, r1):
        if cache.get("rows") != (r0, r1):
            cache["rows"] = (r0, r1)
            cache["hy"] = O.reduce_residual_rmsnorm([p[r0:r1] for p in parts_b], res_b[r0:r1], g_b, wl.eps)
        return cache["hy"]

    t0 = time.perf_counter()
    for r0 in range(0, wl.M, BLOCK):
        r1 = min(wl.M, r0 + BLOCK)
        h_want, y_want = oracle_block(r0, r1)
        assert_within(got_h[r0:r1], h_want, bf16_tol(h_want), f"{wl.name} h rows [{r0}, {r1})")
        assert_within(got_y[r0:r1], y_want, bf16_tol(y_want), f"{wl.name} y rows [{r0}, {r1})")
    print(f"  {wl.M} rows of h and y against the oracle in {time.perf_counter() - t0:.1f} s", flush=True)


def test_dtp_sequence_fullsize(env):
    """Delayed TP at the Qwen3-0.6B-shaped shard: 4 modules, delta = 1, then the flush."""
    torch, sptl, ctx = env
    wl = synth.WORKLOADS["dtp_qwen3_0p6b_tp4"]
    L, delta, tp = wl.dtp_modules, wl.delta, wl.tp
    print(f"dtp_accumulate {wl.name}: {L} modules, delta={delta}, tp={tp}", flush=True)
    g_b = wl.gamma()
    g = to_dev(g_b)
    x0_b = wl.residual()
    owns_b = [wl.own(l) for l in range(L)]
    peers_b = [[wl.peer(l, q) for q in range(tp - 1)] for l in range(L)]
    x = to_dev(x0_b)
    owns = [to_dev(b) for b in owns_b]
    peers = [[to_dev(b) for b in row] for row in peers_b]
    steps, _, x_imm = O.dtp_sequence(x0_b, owns_b, peers_b, delta, g_b, wl.eps, store_bf16=True)
    for l in range(L + delta):
        own = owns[l] if l < L else None
        late = peers[l - delta] if l >= delta else None
        y = torch.empty_like(x) if l < L else None
        sptl.dtp_accumulate(x, own, late, g if y is not None else None, wl.eps, y, tp=tp, delta=delta,
                            module_idx=l, ctx=ctx)
        torch.cuda.synchronize()
        xs, ys = steps[l]
        assert_within(host_values(x), xs, bf16_tol(xs), f"x after step {l}")
        if y is not None:
            assert_within(host_values(y), ys, bf16_tol(ys), f"y of module {l}")
    tol = sum(8e-3 * np.abs(xs) for xs, _ in steps) + 1e-2
    assert_within(host_values(x), x_imm, tol, "delayed vs immediate")
