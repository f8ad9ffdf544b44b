"""agmm_chunked_noalloc (the allocation-free variant) against agmm_chunked, through the C ABI.

Two calls in a row on one context, the second with a smaller input: each gathers fresh seeded
shards into a NaN-poisoned buffer and must give the same bits as agmm_chunked on the same
inputs (both run the same chunk-ordered kernel with one fixed K order), and the gathered
buffer must equal the rank-major concat of the shards.  The smaller call is also compared with
the float64 oracle at the fp32 bound.  The first call also sees the scratch left by earlier
calls of any test in the process: the end counters are zeroed per call and the landed flags
carry a new epoch per call, so leftovers must not matter.
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, fp32_tol, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]


def gen(seed, key, rows, cols, var=1.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)))


@pytest.mark.parametrize("y_f32", [False, True])
def test_noalloc_matches_agmm_chunked(y_f32):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    ctx = sptl.Context(0)
    cs = torch.cuda.current_stream()
    dt = torch.float32 if y_f32 else torch.bfloat16
    iv = torch.int32 if y_f32 else torch.int16
    try:
        # (tp, n_chunks, rows per rank, K, N): the second call is smaller
        for i, (tp, n_chunks, rows, K, N) in enumerate(((8, 8, 1024, 4096, 2048), (4, 8, 256, 512, 384))):
            print(f"no-alloc call {i}: tp={tp} n_chunks={n_chunks} M={tp * rows} K={K} N={N} y={dt}", flush=True)
            M = tp * rows
            shards_b = [gen(200 + i, (0, q), rows, K) for q in range(tp)]
            w_b = gen(210 + i, (1,), K, N, 1.0 / K)
            shards = [to_dev(b) for b in shards_b]
            w = to_dev(w_b)
            xg_ref = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            y_ref = torch.empty((M, N), dtype=dt, device="cuda")
            sptl.agmm_chunked(shards, xg_ref, w, y_ref, n_chunks=n_chunks, rank=0, ctx=ctx)
            xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
            y = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            rc = sptl.raw_agmm_chunked_noalloc(ctx.handle, M, K, N, tp, n_chunks, 0,
                                               [s.data_ptr() for s in shards], xg.data_ptr(), w.data_ptr(),
                                               y.data_ptr(), sptl.F32 if y_f32 else sptl.BF16, cs.cuda_stream)
            assert rc == 0, sptl.last_error()
            torch.cuda.synchronize()
            ctx.check()
            assert torch.equal(xg, torch.cat(shards)), f"call {i}: x_gathered"
            assert torch.equal(y.view(iv), y_ref.view(iv)), f"call {i}: differs from agmm_chunked"
            if i == 1:
                _, want = O.agmm(shards_b, w_b)
                got = y.float().cpu().numpy().astype(np.float64)
                assert_within(got, want, fp32_tol(want) if y_f32 else 8e-3 * np.abs(want) + 1e-2,
                              f"call {i} vs oracle")
    finally:
        torch.cuda.synchronize()
        ctx.close()


def test_noalloc_limits():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    ctx = sptl.Context(0)
    try:
        a = torch.empty(16, dtype=torch.bfloat16, device="cuda").data_ptr()
        # more chunks than the scratch holds, and chunks of 64 rows: rejected before any work
        assert sptl.raw_agmm_chunked_noalloc(ctx.handle, 128 * 128, 256, 256, 2, 128, 0, [a, a], a, a, a, 0,
                                             None) == 2
        assert "scratch" in sptl.last_error()
        assert sptl.raw_agmm_chunked_noalloc(ctx.handle, 256, 256, 256, 2, 4, 0, [a, a], a, a, a, 0, None) == 8
    finally:
        ctx.close()
