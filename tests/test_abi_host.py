"""Host-side checks of the C ABI (no GPU): the library loads, exports every function that
include/sptl.h declares, and rejects invalid arguments before touching the GPU.

Argument validation happens before a NULL context is resolved, so every call here returns
its error status without making a HIP call.
"""
import os
import re

import pytest

from tests.util import ROOT

HEADER = os.path.join(ROOT, "include", "sptl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def sptl():
    from sp_transformer_linear_amd import sptl as mod
    return mod


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("agmm_chunked", "gemm_partial", "reduce_residual_rmsnorm", "dtp_accumulate",
              "sptl_create", "sptl_destroy", "sptl_last_error", "sptl_agmm_timeline", "sptl_version"):
        assert n in names


def test_library_exports_every_declared_symbol(sptl):
    import ctypes
    lib = ctypes.CDLL(sptl.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"libsptl.so does not export {n}"
    assert set(sptl.EXPORTED) == set(declared_functions())
    assert lib.sptl_version() == 100


A = 0x1000  # a 16-byte aligned stand-in address: never dereferenced (validation fails first)


def agmm_args(**kw):
    d = dict(ctx=None, seq_len=256, hidden=256, n_local=512, tp=2, n_chunks=2, rank=0,
             shard_src=[A, A + 0x100000], x_gathered=A, w=A, y=A, y_dtype=0, compute=None, copy=None,
             timing=0)
    d.update(kw)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(shard_src=None), 1), (dict(x_gathered=None), 1), (dict(w=None), 1), (dict(y=None), 1),
    (dict(shard_src=[A, None]), 1),
    (dict(seq_len=-1), 2), (dict(hidden=0), 2), (dict(n_local=-8), 2),
    (dict(tp=0), 6), (dict(tp=65), 6), (dict(rank=2), 6), (dict(rank=-1), 6),
    (dict(n_chunks=0), 6), (dict(n_chunks=513), 6),
    (dict(n_chunks=3), 3), (dict(seq_len=255), 3), (dict(hidden=252), 3), (dict(n_local=500), 3),
    (dict(y_dtype=2), 5), (dict(y_dtype=-1), 5), (dict(timing=2), 6),
    (dict(x_gathered=A + 8), 4), (dict(w=A + 2), 4), (dict(y=A + 4), 4), (dict(shard_src=[A, A + 8]), 4),
    (dict(hidden=2097152 + 8), 2), (dict(n_local=8388608 + 8), 2),
])
def test_agmm_validation(sptl, kw, status):
    rc = sptl.raw_agmm_chunked(**agmm_args(**kw))
    assert rc == status, sptl.last_error()
    assert sptl.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), 1), (dict(w=None), 1), (dict(partial=None), 1),
    (dict(seq_len=-1), 2), (dict(k_local=0), 2), (dict(hidden=0), 2),
    (dict(k_local=12), 3), (dict(hidden=20), 3), (dict(out_dtype=7), 5), (dict(a=A + 2), 4),
    (dict(k_local=2097152 + 8), 2), (dict(hidden=8388608 + 8), 2),
])
def test_gemm_partial_validation(sptl, kw, status):
    d = dict(ctx=None, seq_len=64, k_local=64, hidden=64, a=A, w=A, partial=A, out_dtype=0, stream=None)
    d.update(kw)
    assert sptl.raw_gemm_partial(**d) == status, sptl.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(residual=None), 1), (dict(gamma=None), 1), (dict(y=None), 1), (dict(partials=None), 1),
    (dict(partials=[A, None]), 1), (dict(tp=-1), 6), (dict(tp=17), 6), (dict(hidden=100), 3),
    (dict(hidden=0), 2), (dict(seq_len=-3), 2), (dict(eps=-1.0), 6), (dict(eps=float("nan")), 6),
    (dict(residual=A + 2), 4), (dict(partials=[A, A + 4]), 4), (dict(residual_out=A + 6), 4),
])
def test_reduce_validation(sptl, kw, status):
    d = dict(ctx=None, seq_len=8, hidden=64, tp=2, partials=[A, A], residual=A, gamma=A, eps=1e-6,
             residual_out=None, y=A, stream=None)
    d.update(kw)
    assert sptl.raw_reduce_residual_rmsnorm(**d) == status, sptl.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(residual=None), 1), (dict(tp=0), 6), (dict(tp=17), 6), (dict(delta=-1), 6),
    (dict(module_idx=-1), 6),
    # module < delta: peers must be absent
    (dict(module_idx=0, delta=1), 6),
    # module >= delta: peers required
    (dict(delayed_peers=None), 1), (dict(delayed_peers=[A, None, A]), 1),
    # flush call: no own partial, no norm output
    (dict(own_partial=None), 6), (dict(own_partial=None, y=None, module_idx=0, delta=1, delayed_peers=None), 6),
    (dict(y=None), 1), (dict(gamma=None), 1), (dict(hidden=36), 3), (dict(eps=-2.0), 6),
    (dict(own_partial=A + 2), 4), (dict(y=A + 2), 4),
])
def test_dtp_validation(sptl, kw, status):
    d = dict(ctx=None, seq_len=8, hidden=64, tp=4, delta=1, module_idx=2, residual=A, own_partial=A,
             delayed_peers=[A, A, A], gamma=A, eps=1e-6, y=A, stream=None)
    d.update(kw)
    assert sptl.raw_dtp_accumulate(**d) == status, sptl.last_error()


def test_create_rejects_null_out(sptl):
    assert sptl._lib.sptl_create(None, 0) == 1


def test_wait_timeout_option_rejects_null_ctx(sptl):
    assert sptl._lib.sptl_ctx_set_wait_timeout_us(None, 5) == 1


def test_copy_mode_option_rejects_null_ctx(sptl):
    assert sptl._lib.sptl_ctx_set_copy_mode(None, sptl.COPY_EVENTS, 0) == 1
    assert set(sptl.COPY_MODES.values()) == {0, 1, 2, 3}


def test_staging_option_rejects_null_ctx(sptl):
    assert sptl._lib.sptl_ctx_set_staging(None, sptl.ORDER_INTERLEAVED, 2) == 1
    assert set(sptl.CHUNK_ORDERS.values()) == {0, 1}


@pytest.mark.parametrize("kw,status", [
    (dict(ctx=None), 1),                                   # the set-up lives in the context
    (dict(tp=0), 6), (dict(y_dtype=3), 5), (dict(w=A + 4), 4),
    (dict(seq_len=128 * 128, n_chunks=128), 2),            # more chunks than the scratch holds
    (dict(seq_len=256, n_chunks=4), 8),                    # 64 rows per chunk: no chunk tile fits
])
def test_agmm_noalloc_validation(sptl, kw, status):
    d = dict(ctx=A, seq_len=512, hidden=256, n_local=512, tp=2, n_chunks=2, rank=0,
             shard_src=[A, A + 0x100000], x_gathered=A, w=A, y=A, y_dtype=0, compute=None)
    d.update(kw)
    assert sptl.raw_agmm_chunked_noalloc(**d) == status, sptl.last_error()
    assert "agmm_chunked_noalloc" in sptl.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(shard_src=None), 1), (dict(x_gathered=None), 1), (dict(residual=None), 1), (dict(gamma=None), 1),
    (dict(tp=0), 6), (dict(rank=2), 6), (dict(n_partials=17), 6), (dict(partials=None), 1),
    (dict(partials=[A, None]), 1), (dict(eps=-1.0), 6), (dict(residual=A + 2), 4), (dict(y_dtype=4), 5),
    (dict(shard_src=[None, None]), 1),            # the peer's shard is required (own entry is not)
    (dict(seq_len=301), 3),                       # not a multiple of n_chunks
])
def test_boundary_validation(sptl, kw, status):
    d = dict(ctx=None, n_partials=2, partials=[A, A], residual=A, gamma=A, eps=1e-6, residual_out=None, seq_len=512,
             hidden=256, n_local=512, tp=2, n_chunks=2, rank=0, shard_src=[None, A + 0x100000], x_gathered=A, w=A,
             y=A, y_dtype=0, compute=None)
    d.update(kw)
    assert sptl.raw_reduce_norm_agmm_chunked(**d) == status, sptl.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), 1), (dict(w=None), 1), (dict(partial=None), 1), (dict(dst=None), 1),
    (dict(dst=[None, None]), 1), (dict(tp=0), 6), (dict(tp=65), 6), (dict(rank=2), 6), (dict(seq_len=-2), 2),
    (dict(seq_len=513), 3), (dict(hidden=12), 3), (dict(partial=A + 4), 4), (dict(dst=[None, A + 8]), 4),
    (dict(n_chunks=0), 6), (dict(n_chunks=65), 6), (dict(n_chunks=3), 3), (dict(n_chunks=6), 3),
])
def test_gemm_rs_validation(sptl, kw, status):
    d = dict(ctx=None, seq_len=512, k_local=256, hidden=256, tp=2, n_chunks=2, rank=0, a=A, w=A, partial=A,
             dst=[None, A], compute=None)
    d.update(kw)
    assert sptl.raw_gemm_rs_chunked(**d) == status, sptl.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), 1), (dict(dx=None), 1), (dict(dw=None), 1), (dict(shard_src=[A, None]), 1),
    (dict(tp=0), 6), (dict(tp=65), 6), (dict(rank=2), 6), (dict(hidden=0), 2), (dict(seq_len=-1), 2),
    (dict(seq_len=257), 3), (dict(n_local=12), 3), (dict(hidden=20), 3), (dict(dw_dtype=2), 5),
    (dict(dx=A + 2), 4), (dict(shard_src=[A, A + 8]), 4),
])
def test_agmm_backward_validation(sptl, kw, status):
    d = dict(ctx=None, seq_len=256, hidden=128, n_local=64, tp=2, rank=0, shard_src=[A, A], x_gathered=A, w=A,
             dy=A, dx=A, dw=A, dw_dtype=1, compute=None)
    d.update(kw)
    assert sptl.raw_agmm_backward(**d) == status, sptl.last_error()
