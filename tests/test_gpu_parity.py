"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Inputs come from the seeded generator (sp_transformer_linear_amd.synth); the oracle sees
the same bf16 bits.  Sizes here finish in seconds on the oracle and span several tiles with
ragged tails; full workload sizes are in test_gpu_fullsize.py.

Tolerances: fp32-accumulated outputs |err| <= 1e-3 * ||oracle row||_2 / sqrt(N) + 1e-5;
bf16-stored outputs |err| <= 8e-3 * |oracle| + 1e-2; chunked vs monolithic GEMM, row splits of
the epilogue, and delayed TP with delta = 0 vs the reduce are compared bit for bit.
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests.util import assert_within, bf16_tol, fp32_tol, to_bits, to_dev

pytestmark = pytest.mark.gpu


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


def dec(t):
    return O.bf16_bits_to_f64(to_bits(t))


def gen(seed, key, rows, cols, var=1.0):
    return synth.normal_bf16(seed, key, rows, cols, float(np.sqrt(var)))


# ------------------------------------------------------------------------------------------
# chunked all-gather + column GEMM
# ------------------------------------------------------------------------------------------

AGMM_CASES = [
    # tp, n_chunks, rows per rank, K, N, rank
    (2, 2, 128, 256, 512, 0),      # the tiny tp=2 workload's shapes
    (2, 4, 128, 256, 512, 1),      # two sub-chunks per rank, rank 1
    (3, 6, 100, 200, 136, 2),      # ragged: rows, K and N off every tile size
    (4, 4, 300, 320, 264, 0),      # several 128-row tiles plus tails
    (1, 1, 520, 136, 520, 0),      # tp = 1: nothing to gather
    (8, 8, 64, 128, 256, 3),       # many small chunks
]


@pytest.mark.parametrize("tp,n_chunks,rows,K,N,rank", AGMM_CASES)
@pytest.mark.parametrize("y_f32", [True, False])
def test_agmm_chunked_parity(env, tp, n_chunks, rows, K, N, rank, y_f32):
    torch, sptl, ctx = env
    seed = 100 + tp * 7 + rows
    shards_b = [gen(seed, (0, q), rows, K) for q in range(tp)]
    w_b = gen(seed, (1,), K, N, 1.0 / K)
    M = tp * rows
    shards = [to_dev(b) for b in shards_b]
    w = to_dev(w_b)
    xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")  # poisoned
    y = torch.empty((M, N), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg, w, y, n_chunks=n_chunks, rank=rank, ctx=ctx)
    torch.cuda.synchronize()
    x_want, y_want = O.agmm(shards_b, w_b)
    assert np.array_equal(to_bits(xg), np.concatenate(shards_b)), "x_gathered is not the rank-major concat"
    if y_f32:
        assert_within(y.cpu().numpy().astype(np.float64), y_want, fp32_tol(y_want), "y fp32")
    else:
        assert_within(dec(y), y_want, bf16_tol(y_want), "y bf16")


@pytest.mark.parametrize("tp,n_chunks,rows,K,N,rank", AGMM_CASES[:4])
def test_agmm_chunked_equals_monolithic_bitwise(env, tp, n_chunks, rows, K, N, rank):
    """Chunking splits rows only; with one K order the GPU result bits must not change."""
    torch, sptl, ctx = env
    seed = 200 + rows
    shards = [to_dev(gen(seed, (0, q), rows, K)) for q in range(tp)]
    w = to_dev(gen(seed, (1,), K, N, 1.0 / K))
    M = tp * rows
    xg = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        y_ch = torch.empty((M, N), dtype=dt, device="cuda")
        sptl.agmm_chunked(shards, xg, w, y_ch, n_chunks=n_chunks, rank=rank, ctx=ctx)
        y_mono = torch.empty((M, N), dtype=dt, device="cuda")
        sptl.gemm_partial(xg, w, y_mono, ctx=ctx)
        torch.cuda.synchronize()
        assert torch.equal(y_ch.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           y_mono.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_agmm_own_slot_aliased(env):
    """shard_src[rank] may point into x_gathered's own slot; it is then not copied."""
    torch, sptl, ctx = env
    tp, rows, K, N, rank = 4, 96, 128, 192, 2
    seed = 31
    shards_b = [gen(seed, (0, q), rows, K) for q in range(tp)]
    w_b = gen(seed, (1,), K, N, 1.0 / K)
    xg = torch.zeros((tp * rows, K), dtype=torch.bfloat16, device="cuda")
    xg[rank * rows:(rank + 1) * rows] = to_dev(shards_b[rank])
    shards = [to_dev(b) for b in shards_b]
    shards[rank] = xg[rank * rows:(rank + 1) * rows]
    y = torch.empty((tp * rows, N), dtype=torch.float32, device="cuda")
    sptl.agmm_chunked(shards, xg, to_dev(w_b), y, n_chunks=tp, rank=rank, ctx=ctx)
    torch.cuda.synchronize()
    _, y_want = O.agmm(shards_b, w_b)
    assert np.array_equal(to_bits(xg), np.concatenate(shards_b))
    assert_within(y.cpu().numpy().astype(np.float64), y_want, fp32_tol(y_want), "y")


def test_boundary_epilogue_into_gather_slot(env):
    """Sub-layer boundary: the epilogue writes its normalised rows straight into the own slot of
    the next gather, and agmm_chunked reads them there (no own-slot copy).  The GEMM output is
    bit for bit the one from the same rows in a buffer of their own, and within the oracle's
    bound: the GEMM tolerance plus |y error| @ |W|, the epilogue's own tolerance carried
    through the product."""
    torch, sptl, ctx = env
    tp, rows, H, N, rank, P = 4, 136, 264, 200, 1, 3
    seed = 41
    parts_b, res_b, g_b = epi_inputs(seed, rows, H, P)
    shards_b = [gen(seed, (0, q), rows, H) for q in range(tp)]
    w_b = gen(seed, (1,), H, N, 1.0 / H)
    w, res, g = to_dev(w_b), to_dev(res_b), to_dev(g_b)
    parts = [to_dev(b) for b in parts_b]
    h_out = torch.empty_like(res)
    xg = torch.zeros((tp * rows, H), dtype=torch.bfloat16, device="cuda")
    slot = xg[rank * rows:(rank + 1) * rows]
    y_sep = torch.empty_like(res)
    outs = {}
    for name, dst in (("separate", y_sep), ("in_place", slot)):
        sptl.reduce_residual_rmsnorm(parts, res, g, 1e-6, dst, residual_out=h_out, ctx=ctx)
        src = [to_dev(b) for b in shards_b]
        src[rank] = dst
        outs[name] = torch.empty((tp * rows, N), dtype=torch.float32, device="cuda")
        sptl.agmm_chunked(src, xg, w, outs[name], n_chunks=tp, rank=rank, ctx=ctx)
        torch.cuda.synchronize()
    assert np.array_equal(to_bits(slot), to_bits(y_sep))
    assert torch.equal(outs["separate"], outs["in_place"])
    _, y_norm = O.reduce_residual_rmsnorm(parts_b, res_b, g_b, 1e-6)
    tol_norm = bf16_tol(y_norm)
    assert_within(dec(slot), y_norm, tol_norm, "normalised rows in the gather slot")
    gathered = list(shards_b)
    gathered[rank] = y_norm
    _, y_want = O.agmm(gathered, w_b)
    tol = fp32_tol(y_want) + np.zeros_like(y_want)
    tol[rank * rows:(rank + 1) * rows] += tol_norm @ np.abs(O.bf16_bits_to_f64(w_b))
    assert_within(outs["in_place"].cpu().numpy().astype(np.float64), y_want, tol, "y")
    others = [q for q in range(tp) if q != rank]
    for q in others:
        assert np.array_equal(to_bits(xg[q * rows:(q + 1) * rows]), shards_b[q])


def test_agmm_default_context_and_copy_stream(env):
    """ctx NULL (per-device default) and a caller-supplied copy stream give the same bits."""
    torch, sptl, ctx = env
    tp, rows, K, N = 2, 128, 256, 256
    shards = [to_dev(gen(5, (0, q), rows, K)) for q in range(tp)]
    w = to_dev(gen(5, (1,), K, N, 1.0 / K))
    xg = torch.empty((tp * rows, K), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((tp * rows, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    sptl.agmm_chunked(shards, xg, w, y1, n_chunks=2, rank=0, ctx=None)
    side = torch.cuda.Stream()
    sptl.agmm_chunked(shards, xg, w, y2, n_chunks=2, rank=0, ctx=ctx, copy=side)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_agmm_timeline(env):
    torch, sptl, ctx = env
    tp, rows, K, N = 4, 256, 512, 512
    shards = [to_dev(gen(6, (0, q), rows, K)) for q in range(tp)]
    w = to_dev(gen(6, (1,), K, N, 1.0 / K))
    xg = torch.empty((tp * rows, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((tp * rows, N), dtype=torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg, w, y, n_chunks=tp, rank=1, ctx=ctx, timing=True)
    tl = ctx.timeline(tp)
    for c in (0, 2, 3):  # peer chunks: each GEMM starts after its copy has landed
        cs, ce, gs, ge = tl[c]
        assert 0.0 <= cs <= ce <= ge
        assert ce <= gs, "a chunk GEMM started before its copy landed"
    for c in range(tp):
        assert tl[c][2] <= tl[c][3]
    # the own chunk's GEMM does not wait for the copy of the own slot
    assert tl[1][2] <= tl[0][2]
    # an aliased own slot has no copy at all
    shards[1] = xg[rows:2 * rows]
    sptl.agmm_chunked(shards, xg, w, y, n_chunks=tp, rank=1, ctx=ctx, timing=True)
    tl = ctx.timeline(tp)
    assert tl[1][0] == -1.0 and tl[1][1] == -1.0


# ------------------------------------------------------------------------------------------
# row-parallel partial GEMM
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,H", [(256, 512, 256), (300, 200, 136), (1, 8, 8), (777, 1032, 520),
                                   (2048, 256, 2048),
                                   # 17 x 17 tiles of 256 x 256 at K >= 2048: the four-wave form,
                                   # ragged in M, N and K
                                   (4100, 2056, 4104)])
@pytest.mark.parametrize("out_f32", [True, False])
def test_gemm_partial_parity(env, M, K, H, out_f32):
    torch, sptl, ctx = env
    a_b = gen(7 + M, (3,), M, K)
    w_b = gen(7 + M, (2,), K, H, 1.0 / K)
    out = torch.empty((M, H), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    sptl.gemm_partial(to_dev(a_b), to_dev(w_b), out, ctx=ctx)
    torch.cuda.synchronize()
    want = O.gemm_partial(a_b, w_b)
    if out_f32:
        assert_within(out.cpu().numpy().astype(np.float64), want, fp32_tol(want), "partial fp32")
    else:
        assert_within(dec(out), want, bf16_tol(want), "partial bf16")


def test_gemm_identity_and_permutation_exact(env):
    """W = I or a permutation makes every output an exact copy of an input element."""
    torch, sptl, ctx = env
    M, K = 300, 264
    a_b = gen(9, (3,), M, K)
    a = to_dev(a_b)
    eye = torch.eye(K, dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(a, eye, out, ctx=ctx)
    perm = np.random.default_rng(0).permutation(K)
    pw = torch.zeros((K, K), dtype=torch.bfloat16, device="cuda")
    pw[torch.from_numpy(perm).cuda(), torch.arange(K, device="cuda")] = 1.0
    out2 = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    sptl.gemm_partial(a, pw, out2, ctx=ctx)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), a_b)
    assert np.array_equal(to_bits(out2), a_b[:, perm])


# ------------------------------------------------------------------------------------------
# reduce + residual + RMSNorm
# ------------------------------------------------------------------------------------------

def epi_inputs(seed, R, H, P):
    parts = [gen(seed, (4, p), R, H, 0.02) for p in range(P)]
    res = gen(seed, (5,), R, H)
    gamma = synth.normal_bf16(seed, (6,), 1, H, 0.1, mean=1.0)[0]
    return parts, res, gamma


@pytest.mark.parametrize("R,H,P", [(256, 256, 2), (37, 4096, 8), (64, 3584, 4), (50, 1024, 4),
                                   (9, 200, 3), (5, 8, 1), (3, 8200, 2), (7, 16392, 5), (12, 512, 16),
                                   (4, 2048, 0), (33, 8192, 16)])
@pytest.mark.parametrize("mode", ["separate", "inplace", "no_h"])
def test_reduce_residual_rmsnorm_parity(env, R, H, P, mode):
    torch, sptl, ctx = env
    parts_b, res_b, g_b = epi_inputs(11 + R + H, R, H, P)
    parts = [to_dev(b) for b in parts_b]
    res = to_dev(res_b)
    y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    h_out = {"separate": torch.empty_like(res), "inplace": res, "no_h": None}[mode]
    sptl.reduce_residual_rmsnorm(parts, res, to_dev(g_b), 1e-6, y, residual_out=h_out, ctx=ctx)
    torch.cuda.synchronize()
    h_want, y_want = O.reduce_residual_rmsnorm(parts_b, res_b, g_b, 1e-6)
    assert_within(dec(y), y_want, bf16_tol(y_want), "y")
    if h_out is not None:
        assert_within(dec(h_out), h_want, bf16_tol(h_want), "h")
    else:
        assert np.array_equal(to_bits(res), res_b), "residual modified although residual_out is NULL"


def test_reduce_row_split_bitwise(env):
    """Rows are independent: any split of the rows gives the same bits (norm commutes with the gather)."""
    torch, sptl, ctx = env
    R, H, P = 96, 4096, 8
    parts_b, res_b, g_b = epi_inputs(13, R, H, P)
    parts = [to_dev(b) for b in parts_b]
    res, g = to_dev(res_b), to_dev(g_b)
    y_all = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    h_all = torch.empty_like(y_all)
    sptl.reduce_residual_rmsnorm(parts, res, g, 1e-6, y_all, residual_out=h_all, ctx=ctx)
    y_sp = torch.empty_like(y_all)
    h_sp = torch.empty_like(y_all)
    for lo, hi in ((0, 17), (17, 64), (64, 96)):
        sptl.reduce_residual_rmsnorm([p[lo:hi] for p in parts], res[lo:hi], g, 1e-6, y_sp[lo:hi],
                                     residual_out=h_sp[lo:hi], ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(y_all.view(torch.int16), y_sp.view(torch.int16))
    assert torch.equal(h_all.view(torch.int16), h_sp.view(torch.int16))


def test_reduce_closed_forms(env):
    """Constant rows give c / sqrt(c^2 + eps) * gamma; zero rows give 0."""
    torch, sptl, ctx = env
    H = 1024
    g_b = synth.normal_bf16(3, (6,), 1, H, 0.1, mean=1.0)[0]
    vals = [0.0, 1.0, -2.5, 0.125, 3.0]
    res = torch.tensor(vals, dtype=torch.float32).repeat_interleave(H).view(len(vals), H)
    res = res.to(torch.bfloat16).cuda()
    y = torch.empty_like(res)
    sptl.reduce_residual_rmsnorm([], res, to_dev(g_b), 1e-6, y, ctx=ctx)
    torch.cuda.synchronize()
    gv = O.bf16_bits_to_f64(g_b)
    want = np.array([[c / np.sqrt(c * c + 1e-6) * g for g in gv] for c in vals])
    assert_within(dec(y), want, bf16_tol(want), "constant rows")
    assert np.all(dec(y)[0] == 0.0)


# ------------------------------------------------------------------------------------------
# delayed tensor parallelism
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,tp", [(64, 1024, 4), (33, 4096, 8), (10, 264, 2)])
def test_dtp_delta0_bitwise_equals_reduce(env, T, H, tp):
    torch, sptl, ctx = env
    seed = 17 + T
    own_b = gen(seed, (7, 0), T, H, 0.02)
    peers_b = [gen(seed, (8, 0, q), T, H, 0.02) for q in range(tp - 1)]
    res_b = gen(seed, (5,), T, H)
    g = to_dev(synth.normal_bf16(seed, (6,), 1, H, 0.1, mean=1.0)[0])
    own, peers = to_dev(own_b), [to_dev(b) for b in peers_b]
    x = to_dev(res_b)
    y_dtp = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    sptl.dtp_accumulate(x, own, peers, g, 1e-6, y_dtp, tp=tp, delta=0, module_idx=0, ctx=ctx)
    res2 = to_dev(res_b)
    y_red = torch.empty_like(y_dtp)
    h_red = torch.empty_like(y_dtp)
    sptl.reduce_residual_rmsnorm([own] + peers, res2, g, 1e-6, y_red, residual_out=h_red, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), h_red.view(torch.int16))
    assert torch.equal(y_dtp.view(torch.int16), y_red.view(torch.int16))


@pytest.mark.parametrize("delta,L,tp", [(1, 4, 4), (2, 3, 2), (0, 2, 3), (3, 2, 4)])
def test_dtp_sequence_parity(env, delta, L, tp):
    """Module by module against the oracle (bf16 residual stream), then the flush steps."""
    torch, sptl, ctx = env
    T, H = 96, 1024
    seed = 23 + delta * 10 + L
    x0_b = gen(seed, (5,), T, H)
    owns_b = [gen(seed, (7, l), T, H, 0.02) for l in range(L)]
    peers_b = [[gen(seed, (8, l, q), T, H, 0.02) for q in range(tp - 1)] for l in range(L)]
    g_b = synth.normal_bf16(seed, (6,), 1, H, 0.1, mean=1.0)[0]
    steps, x_final, x_imm = O.dtp_sequence(x0_b, owns_b, peers_b, delta, g_b, 1e-6, store_bf16=True)
    x = to_dev(x0_b)
    g = to_dev(g_b)
    owns = [to_dev(b) for b in owns_b]
    peers = [[to_dev(b) for b in ps] for ps in peers_b]
    for l in range(L + delta):
        own = owns[l] if l < L else None
        late = peers[l - delta] if l >= delta else None
        if own is None and late is None:  # a flush step with nothing outstanding (L < delta)
            assert np.array_equal(steps[l][0], steps[l - 1][0])
            continue
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda") if l < L else None
        sptl.dtp_accumulate(x, own, late, g if y is not None else None, 1e-6, y, tp=tp, delta=delta,
                            module_idx=l, ctx=ctx)
        torch.cuda.synchronize()
        xs, ys = steps[l]
        assert_within(dec(x), xs, bf16_tol(xs), f"x after step {l}")
        if y is not None:
            assert_within(dec(y), ys, bf16_tol(ys), f"y of module {l}")
    # after the flush every partial has been added once: the immediate all-reduce result,
    # up to the bf16 rounding of the stored residual at each of the L + delta steps (each
    # step may contribute up to the bf16 bound of the value it stores)
    tol = sum(8e-3 * np.abs(xs) for xs, _ in steps) + 1e-2
    assert_within(dec(x), x_imm, tol, "delayed vs immediate")


def test_validation_enqueues_nothing(env):
    """An invalid call returns its status and leaves every buffer untouched."""
    torch, sptl, ctx = env
    R, H = 16, 256
    res = torch.ones((R, H), dtype=torch.bfloat16, device="cuda")
    y = torch.full((R, H), 7.0, dtype=torch.bfloat16, device="cuda")
    g = torch.ones((H,), dtype=torch.bfloat16, device="cuda")
    rc = sptl.raw_reduce_residual_rmsnorm(ctx.handle, R, H, 2, [res.data_ptr(), None], res.data_ptr(),
                                          g.data_ptr(), 1e-6, res.data_ptr(), y.data_ptr(), None)
    assert rc == 1
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(res == 1.0)


# ------------------------------------------------------------------------------------------
# chunk-ordered (SDMA-staged) path
# ------------------------------------------------------------------------------------------

STAGED_CASES = [
    # tp, n_chunks, rows per rank, K, N, rank      (rows per chunk a multiple of 128)
    (4, 4, 256, 512, 384, 1),      # 256-row chunks: 256 x 256 tiles
    (2, 2, 384, 256, 264, 0),      # 384-row chunks: 128 x 128 tiles, ragged N
    (8, 16, 256, 200, 520, 5),     # two chunks per rank, ragged K and N
    (3, 3, 512, 1024, 1024, 2),    # odd TP degree
    # K >= 2048: the four-wave form, one workgroup per tile
    (4, 8, 512, 2048, 520, 2),     # two chunks per rank, ragged N
    (2, 2, 256, 2056, 264, 1),     # K ends on a partial stage
]


@pytest.mark.parametrize("tp,n_chunks,rows,K,N,rank", STAGED_CASES)
def test_agmm_staged_parity_and_cross_path_bits(env, tp, n_chunks, rows, K, N, rank):
    """The staged path matches the oracle and the per-chunk event path bit for bit."""
    torch, sptl, ctx = env
    seed = 300 + rows + N
    shards_b = [gen(seed, (0, q), rows, K) for q in range(tp)]
    w_b = gen(seed, (1,), K, N, 1.0 / K)
    M = tp * rows
    shards = [to_dev(b) for b in shards_b]
    w = to_dev(w_b)
    xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sptl.agmm_chunked(shards, xg, w, y, n_chunks=n_chunks, rank=rank, ctx=ctx)
    ctx.check()
    torch.cuda.synchronize()
    _, y_want = O.agmm(shards_b, w_b)
    assert np.array_equal(to_bits(xg), np.concatenate(shards_b))
    assert_within(y.cpu().numpy().astype(np.float64), y_want, fp32_tol(y_want), "staged y")
    # per-chunk event path (a caller-supplied copy stream selects it)
    xg2 = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    side = torch.cuda.Stream()
    sptl.agmm_chunked(shards, xg2, w, y2, n_chunks=n_chunks, rank=rank, ctx=ctx, copy=side)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def test_agmm_staged_no_stale_data(env):
    """Gathered rows cached by earlier reads, and a previous call's data, are never used."""
    torch, sptl, ctx = env
    tp, rows, K, N = 4, 512, 512, 512
    M = tp * rows
    w_b = gen(41, (1,), K, N, 1.0 / K)
    w = to_dev(w_b)
    xg = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    junk = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sptl.gemm_partial(xg, w, junk, ctx=ctx)  # pulls the poisoned rows through the caches
    for trial in range(3):
        shards_b = [gen(42 + trial, (0, q), rows, K) for q in range(tp)]
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        sptl.agmm_chunked([to_dev(b) for b in shards_b], xg, w, y, n_chunks=tp, rank=trial % tp, ctx=ctx)
        torch.cuda.synchronize()
        ctx.check()
        _, y_want = O.agmm(shards_b, w_b)
        got = y.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), f"trial {trial}: stale poisoned rows were read"
        assert_within(got, y_want, fp32_tol(y_want), f"trial {trial}")


def test_agmm_staged_back_to_back_calls(env):
    """More calls in flight than completion-signal sets: each call still sees its own data."""
    torch, sptl, ctx = env
    tp, rows, K, N = 2, 256, 256, 256
    M = tp * rows
    w_b = gen(51, (1,), K, N, 1.0 / K)
    w = to_dev(w_b)
    outs, wants = [], []
    for i in range(9):
        shards_b = [gen(60 + i, (0, q), rows, K) for q in range(tp)]
        xg = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        sptl.agmm_chunked([to_dev(b) for b in shards_b], xg, w, y, n_chunks=tp, rank=0, ctx=ctx)
        outs.append(y)
        wants.append(O.agmm(shards_b, w_b)[1])
    torch.cuda.synchronize()
    ctx.check()
    for i, (y, want) in enumerate(zip(outs, wants)):
        assert_within(y.cpu().numpy().astype(np.float64), want, fp32_tol(want), f"call {i}")


def test_agmm_staged_wait_timeout_is_reported(env):
    """A chunk wait that runs out of time is reported, and the context stays usable at once.

    The bound on a chunk wait is set to 1 us on one context from the host
    (sptl_ctx_set_wait_timeout_us), so the GEMM's workgroups give up long before 8 MiB chunks
    land; every wave still exits normally.  That call's result is invalid.  The default bound
    is then restored and eight more calls follow back to back, with no host wait: the fifth
    reuses the timed-out call's completion-signal set while that call's copies may still be
    landing, so the set must be drained before it is re-armed (a late copy would otherwise mark
    a chunk of the new call landed before it is).  Every later call gathers fresh shards into a
    NaN-poisoned buffer and must match the oracle.
    """
    torch, sptl, ctx = env
    short = sptl.Context(0)
    tp, rows, K, N = 8, 1024, 4096, 256
    M = tp * rows
    try:
        short.set_wait_timeout_us(1)
        shards = [torch.ones((rows, K), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
        xg = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        w = torch.ones((K, N), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=tp, rank=0, ctx=short)
        short.set_wait_timeout_us(0)
        w2_b = gen(71, (1,), K, N, 1.0 / K)
        w2 = to_dev(w2_b)
        calls = []
        for i in range(8):
            shards_b = [gen(80 + i, (0, q), rows, K) for q in range(tp)]
            xg_i = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
            y_i = torch.empty((M, N), dtype=torch.float32, device="cuda")
            srcs = [to_dev(b) for b in shards_b]
            sptl.agmm_chunked(srcs, xg_i, w2, y_i, n_chunks=tp, rank=0, ctx=short)
            calls.append((shards_b, srcs, xg_i, y_i))
        torch.cuda.synchronize()
        with pytest.raises(sptl.SptlError) as err:
            short.check()  # also waits for the abandoned call's copies
        assert err.value.status == 9, str(err.value)
        short.check()  # the report was cleared
        for i, (shards_b, srcs, xg_i, y_i) in enumerate(calls):
            assert torch.equal(xg_i, torch.cat(srcs)), f"call {i + 1}: x_gathered"
            _, want = O.agmm(shards_b, w2_b)
            got = y_i.cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all(), f"call {i + 1}: read rows that had not landed"
            assert_within(got, want, fp32_tol(want), f"call {i + 1}")
        del xg, y, shards  # the timed-out call's copies have landed (short.check waited)
    finally:
        short.close()
    # the shared context is unaffected
    shards = [torch.ones((rows, K), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
    xg = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((K, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sptl.agmm_chunked(shards, xg, w, y, n_chunks=tp, rank=0, ctx=ctx)
    torch.cuda.synchronize()
    ctx.check()
    assert torch.all(y == float(K))


def test_agmm_overlap_pattern(env):
    """The pipeline's copy/compute overlap pattern, read from the call's device timeline.

    "Add forward all-gather overlap" (Megatron-LM pull request 5513, "Summary") checks its
    pipeline with a profiler test: over n children, the gather of child i + 1 runs while child
    i computes, which gives n - 1 gather/compute overlaps.  Here a child is the own chunk, or a
    batch of peer chunks that land together (the first-round chunks that the launch's own
    workgroups copy land at once; the engines' chunks land one after another), in processing
    order, at the page's shape (M = 8192, dim = 4096, 8 chunks).  A batch is in flight from the
    previous batch's landing (the start, for the first) to its own landing, which is when the
    first tile of its chunks saw them, an upper bound.  At least (batches - 1) of the pairs
    (child i computing, child i + 1 in flight) must overlap.  A pipeline that staged every chunk
    before computing any peer chunk would give one.
    """
    torch, sptl, ctx = env
    wl = synth.WORKLOADS["h100_page_8192x4096"]
    shards = [to_dev(wl.shard(q)) for q in range(wl.tp)]
    w = to_dev(wl.w_col())
    xg = torch.empty((wl.M, wl.K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    n = wl.n_chunks
    best, want = -1, None
    for trial in range(3):
        for _ in range(3):
            sptl.agmm_chunked(shards, xg, w, y, n_chunks=n, rank=0, ctx=ctx)
        sptl.agmm_chunked(shards, xg, w, y, n_chunks=n, rank=0, ctx=ctx, timing=True)
        tl = ctx.timeline(n)
        ctx.check()
        # rank 0, one chunk per rank: own chunk 0, then peers 1, 2, ... in processing order
        staged = [c for c in range(n) if tl[c][1] >= 0]
        assert staged == list(range(1, n))
        batches = []
        for c in staged:  # landings are in processing order; equal ones (within 1 us) batch
            if batches and abs(tl[c][1] - tl[batches[-1][-1]][1]) < 1e-3:
                batches[-1].append(c)
            else:
                batches.append([c])
        children = [[0]] + batches
        gemm = [(min(tl[c][2] for c in ch), max(tl[c][3] for c in ch)) for ch in children]
        flight, prev = [], 0.0
        for b in batches:
            flight.append((prev, tl[b[0]][1]))
            prev = tl[b[0]][1]
        pairs = sum(min(gemm[i][1], flight[i][1]) > max(gemm[i][0], flight[i][0]) for i in range(len(batches)))
        want = len(batches) - 1
        print(f"trial {trial}: {pairs} of {len(batches)} (child i computing, child i + 1 in flight) pairs overlap; "
              f"batches {batches}, landings {[round(tl[b[0]][1], 4) for b in batches]}", flush=True)
        best = max(best, pairs)
        if best >= want:
            break
    assert best >= want, f"only {best} copy/compute overlaps, want {want}"
