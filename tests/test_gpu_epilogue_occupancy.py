"""The epilogue's workgroups-per-CU cap does not change any bit.

The register-resident epilogue keeps all of a row's loads in flight, and for launches of up to
48 rows per CU its launch caps the workgroups resident per CU (through an unused LDS
allocation) so that about a fixed number of bytes of loads is in flight per CU.  Rows are
independent and every row is reduced in the same order whatever the launch, so the outputs
must be identical with the default cap, with no cap (SPTL_EPI_INFLIGHT_KIB=0) and with a tight
one (64 KiB: one workgroup per CU at 9 inputs of 4096 columns).  The variable is read once per process, so each setting runs in a child
process.  The default run is also compared with the float64 oracle (bf16 tolerance).
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle.sptl_oracle as O
from tests.util import ROOT, assert_within, bf16_tol

pytestmark = pytest.mark.gpu

EPS = 1e-6
# (rows, hidden, partials): 9 inputs at 4096 columns (capped at 3 workgroups per CU by
# default), 5 inputs at 3584 columns (capped at 5), 4 inputs at 1024 columns (not capped)
REDUCE = [(700, 4096, 8), (333, 3584, 4), (129, 1024, 3)]
# (rows, hidden, tp, delta, module): own + 7 delayed peers at 4096 columns
DTP = [(517, 4096, 8, 1, 3)]

CHILD = textwrap.dedent("""
    import sys, numpy as np, torch
    sys.path.insert(0, {root!r})
    from sp_transformer_linear_amd import sptl
    data = np.load({inp!r})
    dev = lambda k: torch.from_numpy(data[k]).cuda().view(torch.bfloat16)
    out = {{}}
    ctx = sptl.Context(0)
    for i, (R, H, P) in enumerate({reduce!r}):
        parts = [dev(f"r{{i}}_p{{j}}") for j in range(P)]
        h = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        sptl.reduce_residual_rmsnorm(parts, dev(f"r{{i}}_res"), dev(f"g{{H}}"), {eps!r}, y, residual_out=h, ctx=ctx)
        torch.cuda.synchronize()
        out[f"r{{i}}_h"] = h.cpu().view(torch.int16).numpy()
        out[f"r{{i}}_y"] = y.cpu().view(torch.int16).numpy()
    for i, (R, H, tp, delta, module) in enumerate({dtp!r}):
        x = dev(f"d{{i}}_x").clone()
        y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        peers = [dev(f"d{{i}}_q{{j}}") for j in range(tp - 1)]
        sptl.dtp_accumulate(x, dev(f"d{{i}}_own"), peers, dev(f"g{{H}}"), {eps!r}, y, tp=tp, delta=delta,
                            module_idx=module, ctx=ctx)
        torch.cuda.synchronize()
        out[f"d{{i}}_x"] = x.cpu().view(torch.int16).numpy()
        out[f"d{{i}}_y"] = y.cpu().view(torch.int16).numpy()
    ctx.check()
    ctx.close()
    np.savez({outp!r}, **out)
""")


@pytest.fixture(scope="module")
def inputs(tmp_path_factory):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(23)
    bits = lambda shape, scale: O.f64_to_bf16_bits(rng.standard_normal(shape) * scale)  # noqa: E731
    data = {}
    for H in sorted({H for _, H, _ in REDUCE} | {H for _, H, *_ in DTP}):
        data[f"g{H}"] = O.f64_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(H))
    for i, (R, H, P) in enumerate(REDUCE):
        data[f"r{i}_res"] = bits((R, H), 1.0)
        for j in range(P):
            data[f"r{i}_p{j}"] = bits((R, H), 0.02 ** 0.5)
    for i, (R, H, tp, _, _) in enumerate(DTP):
        data[f"d{i}_x"] = bits((R, H), 1.0)
        data[f"d{i}_own"] = bits((R, H), 0.02 ** 0.5)
        for j in range(tp - 1):
            data[f"d{i}_q{j}"] = bits((R, H), 0.02 ** 0.5)
    d = tmp_path_factory.mktemp("epi_occ")
    path = str(d / "inputs.npz")
    np.savez(path, **{k: v.view(np.int16) for k, v in data.items()})
    return d, path, data


def run_child(d, inp, kib):
    outp = str(d / f"out_{kib}.npz")
    code = CHILD.format(root=ROOT, inp=inp, outp=outp, reduce=REDUCE, dtp=DTP, eps=EPS)
    env = dict(os.environ)
    env.pop("SPTL_EPI_INFLIGHT_KIB", None)
    if kib is not None:
        env["SPTL_EPI_INFLIGHT_KIB"] = str(kib)
    print(f"child process with SPTL_EPI_INFLIGHT_KIB={kib}", flush=True)
    subprocess.run([sys.executable, "-c", code], env=env, check=True, timeout=300)
    return dict(np.load(outp))


@pytest.fixture(scope="module")
def default_out(inputs):
    d, inp, _ = inputs
    return run_child(d, inp, None)


def test_default_cap_matches_oracle(inputs, default_out):
    _, _, data = inputs
    for i, (R, H, P) in enumerate(REDUCE):
        h, y = O.reduce_residual_rmsnorm([data[f"r{i}_p{j}"] for j in range(P)], data[f"r{i}_res"],
                                         data[f"g{H}"], EPS)
        got_h = O.bf16_bits_to_f64(default_out[f"r{i}_h"].view(np.uint16))
        got_y = O.bf16_bits_to_f64(default_out[f"r{i}_y"].view(np.uint16))
        assert_within(got_h, h, bf16_tol(h), f"reduce h {R}x{H} P={P}")
        assert_within(got_y, y, bf16_tol(y), f"reduce y {R}x{H} P={P}")
    for i, (R, H, tp, _, _) in enumerate(DTP):
        x, y = O.dtp_accumulate(data[f"d{i}_x"], data[f"d{i}_own"], [data[f"d{i}_q{j}"] for j in range(tp - 1)],
                                data[f"g{H}"], EPS)
        got_x = O.bf16_bits_to_f64(default_out[f"d{i}_x"].view(np.uint16))
        got_y = O.bf16_bits_to_f64(default_out[f"d{i}_y"].view(np.uint16))
        assert_within(got_x, x, bf16_tol(x), f"dtp x {R}x{H} tp={tp}")
        assert_within(got_y, y, bf16_tol(y), f"dtp y {R}x{H} tp={tp}")


@pytest.mark.parametrize("kib", [0, 64])
def test_cap_setting_changes_no_bit(inputs, default_out, kib):
    d, inp, _ = inputs
    other = run_child(d, inp, kib)
    assert set(other) == set(default_out)
    for key in default_out:
        assert np.array_equal(default_out[key], other[key]), f"{key} differs with SPTL_EPI_INFLIGHT_KIB={kib}"
