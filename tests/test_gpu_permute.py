"""The permutation before sharding (permute_bf16) on the GPU, bit for bit against the oracle
("Affinity-Aware Sharding for Delayed Tensor Parallelism", abstract: the dense model is permuted,
then sharded).  Rows and columns, ragged sizes, the weights of a Qwen3-0.6B-shaped layer sharded
by an optimised layout, and an index out of range (zeros there, reported by sptl_ctx_check)."""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import to_bits, to_dev

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


@pytest.mark.parametrize("rows,cols,dim", [(1000, 264, 0), (1000, 264, 1), (1, 8, 0), (3, 4096, 1), (4097, 16, 0)])
def test_permute_bitwise(env, rows, cols, dim):
    torch, sptl, ctx = env
    x_b = synth.normal_bf16(5, (rows, cols), rows, cols, 1.0)
    perm = np.random.default_rng(rows + cols).permutation(rows if dim == 0 else cols).astype(np.int32)
    x = to_dev(x_b)
    out = torch.full((rows, cols), float("nan"), dtype=torch.bfloat16, device="cuda")
    sptl.permute_bf16(x, out, torch.from_numpy(perm).cuda(), dim=dim, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    assert np.array_equal(to_bits(out), O.permute(x_b, perm, dim))


def test_shard_a_layer_by_an_optimised_layout(env):
    """Qwen3-0.6B-shaped FFN and KV projections (hidden 1024, FFN 3072, 8 KV heads of 128, tp 4):
    the optimised layout's permutation applied to W_up (neuron columns), W_down (neuron rows)
    and W_k (head column blocks); each device's shard holds exactly its neurons / heads."""
    torch, sptl, ctx = env
    H, F, n_kv, hd_dim, tp = 1024, 3072, 8, 128, 4
    rng = np.random.default_rng(12)
    a = np.exp(rng.standard_normal((n_kv, F)))
    heads, neurons, _, _ = sptl.dtp_affinity_layout(a, tp)
    w_up_b = synth.normal_bf16(6, (1,), H, F, 0.03)
    w_down_b = synth.normal_bf16(6, (2,), F, H, 0.02)
    w_k_b = synth.normal_bf16(6, (3,), H, n_kv * hd_dim, 0.03)
    pn = sptl.dtp_layout_permutation(neurons, tp)
    ph = sptl.dtp_layout_permutation(heads, tp, hd_dim)
    outs = []
    for w_b, perm, dim in ((w_up_b, pn, 1), (w_down_b, pn, 0), (w_k_b, ph, 1)):
        out = torch.empty(w_b.shape, dtype=torch.bfloat16, device="cuda")
        sptl.permute_bf16(to_dev(w_b), out, torch.from_numpy(perm).cuda(), dim=dim, ctx=ctx)
        outs.append(out)
    torch.cuda.synchronize()
    ctx.check()
    up, down, k = (to_bits(o) for o in outs)
    for d in range(tp):
        mine = np.flatnonzero(neurons == d)
        assert np.array_equal(up[:, d * (F // tp):(d + 1) * (F // tp)], w_up_b[:, mine])
        assert np.array_equal(down[d * (F // tp):(d + 1) * (F // tp)], w_down_b[mine])
        cols = (np.flatnonzero(heads == d)[:, None] * hd_dim + np.arange(hd_dim)).reshape(-1)
        assert np.array_equal(k[:, d * (n_kv // tp) * hd_dim:(d + 1) * (n_kv // tp) * hd_dim], w_k_b[:, cols])


@pytest.mark.parametrize("dim", [0, 1])
def test_index_out_of_range_is_reported(env, dim):
    torch, sptl, ctx = env
    from sp_transformer_linear_amd.sptl import SptlError
    x_b = synth.normal_bf16(7, (9,), 64, 64, 1.0)
    perm = np.arange(64, dtype=np.int32)[::-1].copy()
    perm[5] = 64  # one past the end
    out = torch.empty((64, 64), dtype=torch.bfloat16, device="cuda")
    sptl.permute_bf16(to_dev(x_b), out, torch.from_numpy(perm).cuda(), dim=dim, ctx=ctx)
    torch.cuda.synchronize()
    with pytest.raises(SptlError):
        ctx.check()
    ctx.check()  # the report was cleared
    got = to_bits(out)
    good = np.delete(np.arange(64), 5)
    want = O.permute(x_b, perm[good], dim)
    assert np.array_equal(np.take(got, good, axis=dim), want)
    assert not np.take(got, [5], axis=dim).any()
