"""The copy modes of a context (sptl_ctx_set_copy_mode) on the GPU: every mode gives the bits of
the default staged path, for the chunked gather + column GEMM, the fused sub-layer boundary and
the reduce-scatter mirror; x_gathered and the destinations are NaN-poisoned first.  The modes
exist to compare the copy-engine gather with one on the compute units and with no overlap
("Add forward all-gather overlap", "Observations")."""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

MODES = [("events", 0), ("blit", 0), ("blit", 7), ("serial", 0)]


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


def gen(seed, key, rows, cols, var=1.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)))


def test_copy_mode_validation(env):
    torch, sptl, ref, alt = env
    assert sptl._lib.sptl_ctx_set_copy_mode(alt.handle, 4, 0) == 6
    assert sptl._lib.sptl_ctx_set_copy_mode(alt.handle, -1, 0) == 6
    assert sptl._lib.sptl_ctx_set_copy_mode(alt.handle, 2, -1) == 6
    assert sptl._lib.sptl_ctx_set_copy_mode(alt.handle, 2, 65536) == 6
    alt.set_copy_mode("serial")
    a = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    p = lambda t: t.data_ptr()  # noqa: E731
    # timing has nothing to time without overlap
    assert sptl.raw_agmm_chunked(alt.handle, 512, 256, 256, 2, 2, 0, [p(a), p(a)], p(a), p(a), p(a), 0,
                                 torch.cuda.current_stream().cuda_stream, None, 1) == 8
    alt.set_copy_mode("staged")
    assert "sdma" in alt.info() or "events" in alt.info()


@pytest.mark.parametrize("mode,wgs", MODES)
@pytest.mark.parametrize("tp,n_chunks,rows,K,N,rank", [
    (4, 4, 256, 512, 384, 1),      # 256-row chunks (the staged path's shape)
    (3, 6, 100, 200, 136, 2),      # ragged; the default context also takes the event path here
])
def test_agmm_modes_bitwise(env, mode, wgs, tp, n_chunks, rows, K, N, rank):
    torch, sptl, ref, alt = env
    print(f"agmm mode={mode}/{wgs} tp={tp} n={n_chunks} rows={rows} K={K} N={N} rank={rank}", flush=True)
    seed = 700 + rows + tp
    shards_b = [gen(seed, (0, q), rows, K) for q in range(tp)]
    w_b = gen(seed, (1,), K, N, 1.0 / K)
    M = tp * rows
    shards = [to_dev(b) for b in shards_b]
    w = to_dev(w_b)
    xg0 = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg0, w, y0, n_chunks=n_chunks, rank=rank, ctx=ref)
    alt.set_copy_mode(mode, wgs)
    try:
        for it in range(2):  # twice: the second call reuses the context's events and copy stream
            xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
            y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            sptl.agmm_chunked(shards, xg, w, y, n_chunks=n_chunks, rank=rank, ctx=alt)
            torch.cuda.synchronize()
            alt.check()
            assert torch.equal(xg.view(torch.int16), xg0.view(torch.int16)), f"x_gathered, call {it}"
            assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"y, call {it}"
    finally:
        alt.set_copy_mode("staged")
    ref.check()
    _, y_want = O.agmm(shards_b, w_b)
    assert_within(O.bf16_bits_to_f64(to_bits(y0)), y_want, bf16_tol(y_want), "y vs oracle")


@pytest.mark.parametrize("mode,wgs", MODES)
def test_boundary_modes_bitwise(env, mode, wgs):
    """The fused sub-layer boundary with the copies of each mode (unfused when not staged)."""
    torch, sptl, ref, alt = env
    tp, rows, H, N = 4, 256, 512, 256
    M = tp * rows
    seed = 811
    parts = [to_dev(gen(seed, (2, p), rows, H, 0.02)) for p in range(tp)]
    residual = to_dev(gen(seed, (3,), rows, H))
    gamma = to_dev(gen(seed, (4,), 1, H, 0.01)).reshape(H)
    shards = [None] + [to_dev(gen(seed, (5, q), rows, H)) for q in range(1, tp)]
    w = to_dev(gen(seed, (6,), H, N, 1.0 / H))
    outs = []
    for c, m in ((ref, None), (alt, (mode, wgs))):
        if m:
            c.set_copy_mode(*m)
        xg = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        h = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
        sptl.reduce_norm_agmm_chunked(parts, residual, gamma, 1e-6, shards, xg, w, y, n_chunks=tp, rank=0,
                                      residual_out=h, ctx=c)
        torch.cuda.synchronize()
        c.check()
        outs.append((xg, y, h))
    alt.set_copy_mode("staged")
    for a, b, what in zip(outs[0], outs[1], ("x_gathered", "y", "h")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


@pytest.mark.parametrize("mode,wgs", MODES + [("staged", 0)])
@pytest.mark.parametrize("M,K,H,tp,rank", [(2048, 512, 512, 4, 1), (600, 256, 256, 2, 0), (1024, 768, 256, 8, 5)])
def test_rs_modes_bitwise(env, mode, wgs, M, K, H, tp, rank):
    torch, sptl, ref, alt = env
    print(f"rs mode={mode}/{wgs} M={M} K={K} H={H} tp={tp} rank={rank}", flush=True)
    a = to_dev(gen(900 + M, (0,), M, K))
    w = to_dev(gen(900 + M, (1,), K, H, 1.0 / K))
    want = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(a, w, want, ctx=ref)
    R = M // tp
    alt.set_copy_mode(mode, wgs)
    try:
        for it in range(2):
            part = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
            dst = [None if q == rank else torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda")
                   for q in range(tp)]
            sptl.gemm_rs_chunked(a, w, part, dst, rank=rank, ctx=alt)
            torch.cuda.synchronize()
            alt.check()
            assert torch.equal(part.view(torch.int16), want.view(torch.int16)), f"partial, call {it}"
            for q in range(tp):
                if q != rank:
                    assert torch.equal(dst[q].view(torch.int16), want[q * R:(q + 1) * R].view(torch.int16)), \
                        f"dst[{q}], call {it}"
    finally:
        alt.set_copy_mode("staged")
