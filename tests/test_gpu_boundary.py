"""Sub-layer boundary overlap (reduce_norm_agmm_chunked) on the GPU.

The boundary epilogue of this rank's rows (reduce + residual + RMSNorm, "Potential Solution" of
the AReaL async-TP issue: the window between a reduce-scatter and the next all-gather) writes its
normalised rows into the rank's slot of x_gathered, and the peers' rows start staging before it;
the page's observation that the norm commutes with the sequence gather makes this the same
computation.  Checked: bit for bit against the unfused pair (reduce_residual_rmsnorm into the own
slot, then agmm_chunked reading it in place) on the same stream, and against the float64 oracle
chain, in which the oracle normalises the own rows itself, rounds them to bf16 as the layer stores
them, gathers them with the peers' shards and multiplies.  Tolerances as in test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, fp32_tol, to_bits, to_dev

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


def gen(seed, key, rows, cols, var=1.0, mean=0.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)), mean=mean)


# (tp, n_chunks, rows per rank, K = hidden, N, rank, P partials, fp32 y)
CASES = [(8, 8, 1024, 4096, 4096, 0, 8, False), (4, 8, 256, 512, 384, 1, 4, False),
         (2, 2, 256, 256, 512, 1, 2, True), (4, 4, 512, 1024, 768, 3, 3, False)]


@pytest.mark.parametrize("tp,n_chunks,rows,K,N,rank,P,y_f32", CASES)
def test_boundary_matches_unfused_pair_and_oracle(env, tp, n_chunks, rows, K, N, rank, P, y_f32):
    torch, sptl, ctx = env
    print(f"boundary tp={tp} n_chunks={n_chunks} rows/rank={rows} K={K} N={N} rank={rank} P={P} y_f32={y_f32}",
          flush=True)
    M = tp * rows
    seed = 300 + tp + rank
    shards_b = [gen(seed, (0, q), rows, K) for q in range(tp)]
    parts_b = [gen(seed, (4, p), rows, K, 0.02) for p in range(P)]
    res_b = gen(seed, (5,), rows, K)
    g_b = gen(seed, (6,), 1, K, 0.01, mean=1.0)[0]
    w_b = gen(seed, (1,), K, N, 1.0 / K)
    eps = 1e-6
    shards = [to_dev(b) for b in shards_b]
    parts = [to_dev(b) for b in parts_b]
    res, gamma, w = to_dev(res_b), to_dev(g_b), to_dev(w_b)
    dt = torch.float32 if y_f32 else torch.bfloat16
    iv = torch.int32 if y_f32 else torch.int16
    # fused: the peers' staging starts before the boundary epilogue
    xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=dt, device="cuda")
    h = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
    sptl.reduce_norm_agmm_chunked(parts, res, gamma, eps, shards, xg, w, y, n_chunks=n_chunks, rank=rank,
                                  residual_out=h, ctx=ctx)
    # unfused pair on the same stream
    xg2 = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    h2 = torch.empty_like(h)
    own2 = xg2[rank * rows:(rank + 1) * rows]
    sptl.reduce_residual_rmsnorm(parts, res, gamma, eps, own2, residual_out=h2, ctx=ctx)
    src = [own2 if q == rank else shards[q] for q in range(tp)]
    sptl.agmm_chunked(src, xg2, w, y2, n_chunks=n_chunks, rank=rank, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    assert torch.equal(xg.view(torch.int16), xg2.view(torch.int16)), "x_gathered differs from the unfused pair"
    assert torch.equal(y.view(iv), y2.view(iv)), "y differs from the unfused pair"
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), "h differs from the unfused pair"
    # the peers' slots hold their shards bit for bit
    for q in range(tp):
        if q != rank:
            assert torch.equal(xg[q * rows:(q + 1) * rows], shards[q]), f"slot of rank {q}"
    # oracle chain
    h_o, y_own = O.reduce_residual_rmsnorm(parts_b, res_b, g_b, eps)
    got_h = O.bf16_bits_to_f64(to_bits(h))
    assert_within(got_h, h_o, bf16_tol(h_o), "h")
    got_own = O.bf16_bits_to_f64(to_bits(xg[rank * rows:(rank + 1) * rows]))
    assert_within(got_own, y_own, bf16_tol(y_own), "normalised own rows")
    own_o = O.round_to_bf16(y_own)
    gathered = [own_o if q == rank else shards_b[q] for q in range(tp)]
    _, y_o = O.agmm(gathered, w_b)
    got = y.cpu().numpy().astype(np.float64) if y_f32 else O.bf16_bits_to_f64(to_bits(y))
    tol = fp32_tol(y_o) if y_f32 else bf16_tol(y_o)
    # The own rows reach the GEMM as bf16 on both sides, each element within half an ulp of the
    # exact norm, so the two stored rows differ by at most one ulp <= 2^-7 |x| per element; their
    # GEMM rows may then differ by up to 2^-7 (|x_own| @ |w|) beyond the GEMM's own bound.
    tol = np.broadcast_to(tol, y_o.shape).copy()
    tol[rank * rows:(rank + 1) * rows] += 2.0 ** -7 * (np.abs(own_o) @ np.abs(O.bf16_bits_to_f64(w_b)))
    assert_within(got, y_o, tol, "y")
