"""Every GEMM tile configuration gives the same bits.

All configurations use the same MFMA instruction and the same ascending K order (no split-K),
so forcing any of them through SPTL_GEMM_CFG must reproduce the default configuration's
output bit for bit, for the plain GEMM (ragged shapes) and for the chunk-ordered agmm.  The
variable is read once per process, so each configuration runs in a child process; the parent
computes the default-configuration result and checks it against the oracle.
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle.sptl_oracle as O
from tests.util import ROOT, assert_within, bf16_tol, fp32_tol

pytestmark = pytest.mark.gpu

# (M, K, N): several tiles, ragged in every dimension, and a tall one
GEMM_SHAPES = [(520, 264, 392), (1024, 512, 768), (300, 1000, 136)]
AGMM = dict(tp=4, rows=256, K=512, N=384)

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
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        sptl.gemm_partial(a, w, y, ctx=ctx)
        yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        sptl.gemm_partial(a, w, yb, ctx=ctx)
        torch.cuda.synchronize()
        out[f"y{{i}}"] = y.cpu().numpy().view(np.uint32)
        out[f"yb{{i}}"] = yb.cpu().view(torch.int16).numpy()
    shards = [torch.from_numpy(data[f"s{{q}}"]).cuda().view(torch.bfloat16) for q in range({tp})]
    wc = torch.from_numpy(data["wc"]).cuda().view(torch.bfloat16)
    xg = torch.empty(({tp} * {rows}, {K}), dtype=torch.bfloat16, device="cuda")
    ya = torch.empty(({tp} * {rows}, {N}), dtype=torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg, wc, ya, n_chunks={tp}, rank=1, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    out["agmm"] = ya.cpu().view(torch.int16).numpy()
    out["info"] = np.array(ctx.info())
    ctx.close()
    np.savez({outp!r}, **out)
""")


@pytest.fixture(scope="module")
def inputs(tmp_path_factory):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(11)
    bits = lambda shape, scale: O.f64_to_bf16_bits(rng.standard_normal(shape) * scale)  # noqa: E731
    data = {}
    for i, (M, K, N) in enumerate(GEMM_SHAPES):
        data[f"a{i}"] = bits((M, K), 1.0)
        data[f"w{i}"] = bits((K, N), K ** -0.5)
    for q in range(AGMM["tp"]):
        data[f"s{q}"] = bits((AGMM["rows"], AGMM["K"]), 1.0)
    data["wc"] = bits((AGMM["K"], AGMM["N"]), AGMM["K"] ** -0.5)
    d = tmp_path_factory.mktemp("cfg")
    path = str(d / "inputs.npz")
    np.savez(path, **data)
    return d, path, data


def run_child(d, inp, cfg):
    outp = str(d / f"out_{cfg or 'default'}.npz")
    code = CHILD.format(root=ROOT, inp=inp, outp=outp, shapes=GEMM_SHAPES, **AGMM)
    env = dict(os.environ)
    env.pop("SPTL_GEMM_CFG", None)
    if cfg:
        env["SPTL_GEMM_CFG"] = cfg
    print(f"child process with SPTL_GEMM_CFG={cfg}", flush=True)
    subprocess.run([sys.executable, "-c", code], env=env, check=True, timeout=300)
    return dict(np.load(outp))


@pytest.fixture(scope="module")
def reference(inputs):
    d, inp, data = inputs
    ref = run_child(d, inp, None)
    # the default configuration against the oracle
    for i, (M, K, N) in enumerate(GEMM_SHAPES):
        want = O.gemm_partial(data[f"a{i}"], data[f"w{i}"])
        assert_within(ref[f"y{i}"].view(np.float32).astype(np.float64), want, fp32_tol(want), f"gemm {M}x{K}x{N}")
        assert_within(O.bf16_bits_to_f64(ref[f"yb{i}"].view(np.uint16)), want, bf16_tol(want), f"gemm {M}x{K}x{N} bf16")
    _, want = O.agmm([data[f"s{q}"] for q in range(AGMM["tp"])], data["wc"])
    assert_within(O.bf16_bits_to_f64(ref["agmm"].view(np.uint16)), want, bf16_tol(want), "agmm")
    return ref


@pytest.mark.parametrize("cfg", ["256x256w4x2", "256x256w2x4", "256x256w2x2", "256x128w4x2", "256x128w4x1",
                                 "128x128w2x2", "256x256ring", "256x256ring4", "128x256w2x2k32", "256x256w4x2k32",
                                 "256x256bt", "256x256il2", "256x256il4", "256x256btil2"])
def test_forced_config_is_bit_identical(inputs, reference, cfg):
    d, inp, _ = inputs
    got = run_child(d, inp, cfg)
    for key in reference:
        if key == "info":
            continue
        assert np.array_equal(got[key], reference[key]), f"{cfg}: {key} differs from the default configuration"
