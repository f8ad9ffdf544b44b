"""The staged gather's copies start only after the work queued ahead of the call on its stream.

Each trial, on the call's stream and with no host wait: every rank's shard is overwritten with
new values, x_gathered is NaN-poisoned, then agmm_chunked runs.  The copies must read the new
shards (not the previous trial's) and must not land before the poison, and the next trial's
overwrite must not reach a shard before this call's copies have read it.  Every output is checked
against the oracle with that trial's values.  Two forks are covered: the GEMM's start (the lead
copy takes every first-round peer chunk) and the event recorded before the launch (the link
model, whose first round waits for engine copies).
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, fp32_tol, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]


@pytest.mark.parametrize("staging", [("ring", 0), ("ring", 1)], ids=["fork_at_start", "fork_event"])
def test_sources_written_just_before_the_call(staging):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    tp, rows, K, N, rank, trials = 8, 256, 2048, 512, 3, 4
    M = tp * rows
    w_b = synth.normal_bf16(300, (1,), K, N, float(np.sqrt(1.0 / K)))
    w = to_dev(w_b)
    values_b = [[synth.normal_bf16(301 + t, (0, q), rows, K, 1.0) for q in range(tp)] for t in range(trials)]
    values = [[to_dev(b) for b in vt] for vt in values_b]
    shards = [torch.empty((rows, K), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
    xg = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(trials)]
    ctx = sptl.Context(0)
    try:
        ctx.set_staging(*staging)
        torch.cuda.synchronize()
        print(f"fork order: staging {staging}", flush=True)
        for t in range(trials):  # all on the current stream, no host wait
            for q in range(tp):
                shards[q].copy_(values[t][q])
            xg.fill_(float("nan"))
            sptl.agmm_chunked(shards, xg, w, ys[t], n_chunks=tp, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
        ctx.check()
        for t in range(trials):
            _, want = O.agmm(values_b[t], w_b)
            got = ys[t].cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all(), f"trial {t}: poisoned rows were read"
            assert_within(got, want, fp32_tol(want), f"trial {t}")
    finally:
        torch.cuda.synchronize()
        ctx.close()
