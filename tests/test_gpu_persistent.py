"""GEMM launches with more tiles than workgroups: each workgroup of the 256 x 256 kernel takes
several tiles, and near the end of a tile it may load the next tile's first stages.

Shapes are chosen so that some workgroups run two tiles, with ragged M, N and K (partial last
stages, partial last row and column tiles), with K short enough that no stage is left for the
look-ahead (three stages or fewer) and long enough for it.  The chunk-ordered launches use
chunks of two 256-row tiles, so a second tile may belong to a chunk that has or has not landed
when its predecessor nears its end.  Outputs are compared with the float64 oracle (tolerances
as in test_gpu_parity.py) and, bit for bit, with the register-staged configuration, which runs
one tile per workgroup (forced in a child process, since the configuration is read once per
process).
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import ROOT, assert_within, bf16_tol, fp32_tol

pytestmark = pytest.mark.gpu

# (M, K, N): 17 x 17 = 289 tiles (more than one per CU); K = 96 leaves no look-ahead stage,
# K = 520 ends on a partial stage, K = 1024 is a whole number of stages
GEMM_SHAPES = [(4100, 96, 4104), (4100, 520, 4104), (4352, 1024, 4352)]
# chunk-ordered: tp = n_chunks = 8 chunks of 512 rows (2 row tiles), N = 4352 (17 column tiles):
# 272 tiles; K = 96 (no look-ahead), K = 640
AGMM_CASES = [(8, 512, 96, 4352, 3), (8, 512, 640, 4352, 0)]

CHILD = textwrap.dedent("""
    import sys, numpy as np, torch
    sys.path.insert(0, {root!r})
    from sp_transformer_linear_amd import sptl
    data = np.load({inp!r})
    out = {{}}
    ctx = sptl.Context(0)
    for i, (M, K, N) in enumerate({shapes!r}):
        a = torch.from_numpy(data[f"a{{i}}"]).cuda().view(torch.bfloat16)
        w = torch.from_numpy(data[f"w{{i}}"]).cuda().view(torch.bfloat16)
        for name, dt in (("f", torch.float32), ("b", torch.bfloat16)):
            y = torch.empty((M, N), dtype=dt, device="cuda")
            sptl.gemm_partial(a, w, y, ctx=ctx)
            torch.cuda.synchronize()
            out[f"y{{name}}{{i}}"] = y.cpu().view(torch.int32 if name == "f" else torch.int16).numpy()
    for i, (tp, rows, K, N, rank) in enumerate({agmm!r}):
        shards = [torch.from_numpy(data[f"s{{i}}_{{q}}"]).cuda().view(torch.bfloat16) for q in range(tp)]
        w = torch.from_numpy(data[f"wa{{i}}"]).cuda().view(torch.bfloat16)
        xg = torch.empty((tp * rows, K), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((tp * rows, N), dtype=torch.bfloat16, device="cuda")
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=tp, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
        out[f"agmm{{i}}"] = y.cpu().view(torch.int16).numpy()
    ctx.check()
    ctx.close()
    np.savez({outp!r}, **out)
""")


@pytest.fixture(scope="module")
def inputs(tmp_path_factory):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    data = {}
    for i, (M, K, N) in enumerate(GEMM_SHAPES):
        data[f"a{i}"] = synth.normal_bf16(31, (i, 0), M, K, 1.0)
        data[f"w{i}"] = synth.normal_bf16(31, (i, 1), K, N, float(K ** -0.5))
    for i, (tp, rows, K, N, rank) in enumerate(AGMM_CASES):
        for q in range(tp):
            data[f"s{i}_{q}"] = synth.normal_bf16(37, (i, 0, q), rows, K, 1.0)
        data[f"wa{i}"] = synth.normal_bf16(37, (i, 1), K, N, float(K ** -0.5))
    d = tmp_path_factory.mktemp("persist")
    path = str(d / "inputs.npz")
    np.savez(path, **{k: v.view(np.int16) for k, v in data.items()})
    return d, path, data


def run_child(d, inp, cfg):
    outp = str(d / f"out_{cfg or 'default'}.npz")
    code = CHILD.format(root=ROOT, inp=inp, outp=outp, shapes=GEMM_SHAPES, agmm=AGMM_CASES)
    env = dict(os.environ)
    env.pop("SPTL_GEMM_CFG", None)
    if cfg:
        env["SPTL_GEMM_CFG"] = cfg
    print(f"child process with SPTL_GEMM_CFG={cfg}", flush=True)
    subprocess.run([sys.executable, "-c", code], env=env, check=True, timeout=300)
    return dict(np.load(outp))


@pytest.fixture(scope="module")
def default_out(inputs):
    d, inp, _ = inputs
    return run_child(d, inp, None)


def test_several_tiles_per_workgroup_match_oracle(inputs, default_out):
    _, _, data = inputs
    for i, (M, K, N) in enumerate(GEMM_SHAPES):
        want = O.gemm_partial(data[f"a{i}"], data[f"w{i}"])
        got_f = default_out[f"yf{i}"].view(np.float32).astype(np.float64)
        assert_within(got_f, want, fp32_tol(want), f"gemm {M}x{K}x{N} fp32")
        got_b = O.bf16_bits_to_f64(default_out[f"yb{i}"].view(np.uint16))
        assert_within(got_b, want, bf16_tol(want), f"gemm {M}x{K}x{N} bf16")
    for i, (tp, rows, K, N, rank) in enumerate(AGMM_CASES):
        _, want = O.agmm([data[f"s{i}_{q}"] for q in range(tp)], data[f"wa{i}"])
        got = O.bf16_bits_to_f64(default_out[f"agmm{i}"].view(np.uint16))
        assert_within(got, want, bf16_tol(want), f"agmm tp={tp} rows={rows} K={K} N={N}")


def test_several_tiles_per_workgroup_bitwise_vs_one_tile_per_workgroup(inputs, default_out):
    d, inp, _ = inputs
    one = run_child(d, inp, "256x256w4x2")
    for key in default_out:
        assert np.array_equal(default_out[key], one[key]), f"{key} differs from the one-tile-per-workgroup kernel"
