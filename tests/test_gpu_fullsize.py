"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Every output row the oracle checks is computed by the oracle one row at a time (float64),
on sampled rows: the first and last row of every chunk plus seeded random rows.  Whole-tensor
properties are checked on the GPU: the gathered activations equal the rank-major concat of
the shards bit for bit, and the chunked result equals a monolithic GEMM of the gathered rows
bit for bit.  Tolerances as in test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, fp32_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

RANDOM_ROWS_PER_CHUNK = 6


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


def sample_rows(M, n_chunks, seed):
    rng = np.random.default_rng(seed)
    per = M // n_chunks
    rows = set()
    for c in range(n_chunks):
        rows.update((c * per, c * per + per - 1))
        rows.update(rng.integers(c * per, (c + 1) * per, RANDOM_ROWS_PER_CHUNK).tolist())
    return np.array(sorted(rows))


def dec_rows(t, rows):
    import torch
    idx = torch.from_numpy(rows).to(t.device)
    return O.bf16_bits_to_f64(to_bits(t.index_select(0, idx)))


def run_agmm(env, wl, y_f32):
    torch, sptl, ctx = env
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
    rows = sample_rows(wl.M, wl.n_chunks, 7)
    # oracle, row by row: the gathered row is row r of the concat, i.e. row r % (M/tp) of shard r // (M/tp)
    per_rank = wl.M // wl.tp
    x_rows = np.stack([shards_b[int(r) // per_rank][int(r) % per_rank] for r in rows])
    want = O.gemm_partial(x_rows, w_b)
    if y_f32:
        got = y.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy().astype(np.float64)
        assert_within(got, want, fp32_tol(want), f"{wl.name} agmm y (fp32)")
    else:
        got = dec_rows(y, rows)
        assert_within(got, want, bf16_tol(want), f"{wl.name} agmm y (bf16)")
    # chunked == monolithic, bit for bit
    y_mono = torch.empty_like(y)
    sptl.gemm_partial(xg, w, y_mono, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16 if not y_f32 else torch.int32),
                       y_mono.view(torch.int16 if not y_f32 else torch.int32)), "chunked != monolithic"
    return ctx.info()


@pytest.mark.parametrize("name,y_f32", [("h100_page_8192x4096", False), ("h100_page_8192x4096", True),
                                        ("qwen2_7b_tp4_16384", False), ("msweep_65536x4096", False)])
def test_agmm_fullsize(env, name, y_f32):
    info = run_agmm(env, synth.WORKLOADS[name], y_f32)
    assert "sdma-striped" in info, f"the benchmarked staging path was not used: {info}"


@pytest.mark.parametrize("name", ["h100_page_8192x4096", "qwen2_7b_tp4_16384", "dtp_qwen3_0p6b_tp4"])
def test_gemm_partial_fullsize(env, name):
    torch, sptl, ctx = env
    wl = synth.WORKLOADS[name]
    a_b = wl.a_row()
    a = to_dev(a_b)
    w_b = wl.w_row()
    out = torch.empty((wl.M, wl.H), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(a, to_dev(w_b), out, ctx=ctx)
    torch.cuda.synchronize()
    rows = sample_rows(wl.M, wl.n_chunks, 8)
    want = O.gemm_partial(a_b[rows], w_b)
    assert_within(dec_rows(out, rows), want, bf16_tol(want), f"{wl.name} partial")


@pytest.mark.parametrize("name", ["h100_page_8192x4096", "qwen2_7b_tp4_16384", "msweep_65536x4096",
                                  "dtp_qwen3_0p6b_tp4"])
def test_reduce_residual_rmsnorm_fullsize(env, name):
    torch, sptl, ctx = env
    wl = synth.WORKLOADS[name]
    rows = sample_rows(wl.M, wl.n_chunks, 9)
    parts, parts_rows = [], []
    for p in range(wl.P):
        b = wl.partial(p)
        parts.append(to_dev(b))
        parts_rows.append(b[rows])
        del b
    res_b = wl.residual()
    res = to_dev(res_b)
    res_rows = res_b[rows]
    del res_b
    g_b = wl.gamma()
    y = torch.empty_like(res)
    h = torch.empty_like(res)
    sptl.reduce_residual_rmsnorm(parts, res, to_dev(g_b), wl.eps, y, residual_out=h, ctx=ctx)
    torch.cuda.synchronize()
    h_want, y_want = O.reduce_residual_rmsnorm(parts_rows, res_rows, g_b, wl.eps)
    assert_within(dec_rows(h, rows), h_want, bf16_tol(h_want), f"{wl.name} h")
    assert_within(dec_rows(y, rows), y_want, bf16_tol(y_want), f"{wl.name} y")
    # rows are independent: the first rows of the full call equal a call on those rows alone
    y2 = torch.empty_like(y[:333])
    sptl.reduce_residual_rmsnorm([p[:333] for p in parts], res[:333], to_dev(g_b), wl.eps, y2, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y[:333].view(torch.int16))


def test_dtp_sequence_fullsize(env):
    """Delayed TP at the Qwen3-0.6B-shaped shard: 4 modules, delta = 1, then the flush."""
    torch, sptl, ctx = env
    wl = synth.WORKLOADS["dtp_qwen3_0p6b_tp4"]
    L, delta, tp = wl.dtp_modules, wl.delta, wl.tp
    rows = sample_rows(wl.M, wl.n_chunks, 10)
    g_b = wl.gamma()
    g = to_dev(g_b)
    x = to_dev(wl.residual())
    owns = [to_dev(wl.own(l)) for l in range(L)]
    peers = [[to_dev(wl.peer(l, q)) for q in range(tp - 1)] for l in range(L)]
    steps, _, x_imm = O.dtp_sequence(
        wl.residual(row_idx=rows), [wl.own(l, row_idx=rows) for l in range(L)],
        [[wl.peer(l, q, row_idx=rows) for q in range(tp - 1)] for l in range(L)], delta, g_b, wl.eps,
        store_bf16=True)
    for l in range(L + delta):
        own = owns[l] if l < L else None
        late = peers[l - delta] if l >= delta else None
        y = torch.empty_like(x) if l < L else None
        sptl.dtp_accumulate(x, own, late, g if y is not None else None, wl.eps, y, tp=tp, delta=delta,
                            module_idx=l, ctx=ctx)
        torch.cuda.synchronize()
        xs, ys = steps[l]
        assert_within(dec_rows(x, rows), xs, bf16_tol(xs), f"x after step {l}")
        if y is not None:
            assert_within(dec_rows(y, rows), ys, bf16_tol(ys), f"y of module {l}")
    tol = sum(8e-3 * np.abs(xs) for xs, _ in steps) + 1e-2
    assert_within(dec_rows(x, rows), x_imm, tol, "delayed vs immediate")
