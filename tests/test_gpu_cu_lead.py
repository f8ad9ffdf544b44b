"""The lead chunks that a chunk-ordered launch's own workgroups copy give the same bits as the
copy engines.

When the own chunks do not fill the GEMM's first round of tiles, the tiles of the first peer
chunks copy those chunks themselves (the copy engines take the later ones).  The switch that
leaves every chunk to the engines (SPTL_CU_LEAD=0) is read once per process, so that case runs in
a child process; both outputs and gathers must match bit for bit, with x_gathered NaN-poisoned
and the result checked against the oracle, at the page's shape (8 chunks of 1024 rows, a quarter
of the chip each) and at a tp = 2 shape with two chunks per rank.
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import ROOT, assert_within, bf16_tol, to_bits, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

CASES = [(8, 8, 1024, 4096, 1024, 0), (2, 4, 512, 1024, 512, 1)]  # tp, n_chunks, rows/rank, K, N, rank

CHILD = textwrap.dedent("""
    import sys, numpy as np, torch
    sys.path.insert(0, {root!r})
    from sp_transformer_linear_amd import sptl
    data = np.load({inp!r})
    out = {{}}
    ctx = sptl.Context(0)
    for i, (tp, n, rows, K, N, rank) in enumerate({cases!r}):
        shards = [torch.from_numpy(data[f"s{{i}}_{{q}}"]).cuda().view(torch.bfloat16) for q in range(tp)]
        w = torch.from_numpy(data[f"w{{i}}"]).cuda().view(torch.bfloat16)
        xg = torch.full((tp * rows, K), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((tp * rows, N), dtype=torch.bfloat16, device="cuda")
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=n, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
        out[f"y{{i}}"] = y.cpu().view(torch.int16).numpy()
        out[f"x{{i}}"] = xg.cpu().view(torch.int16).numpy()
    ctx.check()
    ctx.close()
    np.savez({outp!r}, **out)
""")


def test_cu_lead_matches_engines_only(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sp_transformer_linear_amd import sptl
    data = {}
    for i, (tp, n, rows, K, N, rank) in enumerate(CASES):
        for q in range(tp):
            data[f"s{i}_{q}"] = synth.normal_bf16(300 + i, (0, q), rows, K, 1.0).view(np.int16)
        data[f"w{i}"] = synth.normal_bf16(300 + i, (1,), K, N, float(np.sqrt(1.0 / K))).view(np.int16)
    inp = str(tmp_path / "in.npz")
    np.savez(inp, **data)
    ctx = sptl.Context(0)
    ref = {}
    for i, (tp, n, rows, K, N, rank) in enumerate(CASES):
        print(f"case tp={tp} n={n} rows={rows} K={K} N={N} rank={rank}", flush=True)
        shards_b = [data[f"s{i}_{q}"].view(np.uint16) for q in range(tp)]
        w_b = data[f"w{i}"].view(np.uint16)
        xg = torch.full((tp * rows, K), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((tp * rows, N), dtype=torch.bfloat16, device="cuda")
        sptl.agmm_chunked([to_dev(b) for b in shards_b], xg, to_dev(w_b), y, n_chunks=n, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
        ctx.check()
        ref[f"y{i}"], ref[f"x{i}"] = to_bits(y), to_bits(xg)
        assert np.array_equal(ref[f"x{i}"], np.concatenate(shards_b))
        _, want = O.agmm(shards_b, w_b)
        assert_within(O.bf16_bits_to_f64(ref[f"y{i}"]), want, bf16_tol(want), f"case {i} vs oracle")
    ctx.close()
    outp = str(tmp_path / "out.npz")
    env = dict(os.environ, SPTL_CU_LEAD="0")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, inp=inp, outp=outp, cases=CASES)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    got = np.load(outp)
    for i in range(len(CASES)):
        assert np.array_equal(got[f"x{i}"].view(np.uint16), ref[f"x{i}"]), f"case {i}: x_gathered"
        assert np.array_equal(got[f"y{i}"].view(np.uint16), ref[f"y{i}"]), f"case {i}: y"
