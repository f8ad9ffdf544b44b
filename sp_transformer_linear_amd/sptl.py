"""Thin ctypes binding of libsptl.so (C ABI in include/sptl.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels and
SDMA copies.  torch supplies device memory and streams; tensors are passed by data pointer.
Importing this module loads the library and raises ImportError if it has not been built.

Two levels are offered:
  * ``raw_*``: the C calls with plain integers (device addresses, stream handles), as the C
    ABI takes them;
  * tensor wrappers with the ABI's names, which check device, dtype, contiguity and shape,
    then call the raw function.  Every non-OK status raises SptlError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsptl.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sp_transformer_linear_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

BF16, F32 = 0, 1
STATUS = {0: "SPTL_OK", 1: "SPTL_E_NULL", 2: "SPTL_E_SHAPE", 3: "SPTL_E_DIVISIBILITY",
          4: "SPTL_E_ALIGN", 5: "SPTL_E_DTYPE", 6: "SPTL_E_RANGE", 7: "SPTL_E_HIP",
          8: "SPTL_E_UNSUPPORTED", 9: "SPTL_E_ASYNC"}
MAX_PARTIALS, MAX_TP, MAX_CHUNKS = 16, 64, 512
MAX_K, MAX_N = 2097152, 8388608
COPY_STAGED, COPY_EVENTS, COPY_BLIT, COPY_SERIAL = 0, 1, 2, 3
COPY_MODES = {"staged": COPY_STAGED, "events": COPY_EVENTS, "blit": COPY_BLIT, "serial": COPY_SERIAL}
ORDER_RING, ORDER_INTERLEAVED = 0, 1
CHUNK_ORDERS = {"ring": ORDER_RING, "interleaved": ORDER_INTERLEAVED}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_ptrs = ctypes.POINTER(ctypes.c_void_p)

_SIGS = {
    "sptl_create": ([ctypes.POINTER(ctypes.c_void_p), _int], _int),
    "sptl_destroy": ([_vp], _int),
    "sptl_last_error": ([], ctypes.c_char_p),
    "sptl_version": ([], _int),
    "sptl_ctx_check": ([_vp], _int),
    "sptl_ctx_info": ([_vp], ctypes.c_char_p),
    "sptl_ctx_set_wait_timeout_us": ([_vp, _i64], _int),
    "sptl_ctx_set_copy_mode": ([_vp, _int, _int], _int),
    "sptl_ctx_set_staging": ([_vp, _int, _int], _int),
    "agmm_chunked": ([_vp, _i64, _i64, _i64, _int, _int, _int, _ptrs, _vp, _vp, _vp, _int, _vp, _vp,
                      _int], _int),
    "agmm_chunked_noalloc": ([_vp, _i64, _i64, _i64, _int, _int, _int, _ptrs, _vp, _vp, _vp, _int, _vp], _int),
    "sptl_agmm_timeline": ([_vp, ctypes.POINTER(ctypes.c_double), _int], _int),
    "reduce_norm_agmm_chunked": ([_vp, _int, _ptrs, _vp, _vp, ctypes.c_float, _vp, _i64, _i64, _i64, _int, _int,
                                  _int, _ptrs, _vp, _vp, _vp, _int, _vp], _int),
    "gemm_partial": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _int, _vp], _int),
    "gemm_rs_chunked": ([_vp, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _ptrs, _vp], _int),
    "dtp_affinity_layout": ([ctypes.POINTER(ctypes.c_double), _int, _int, _int, _int, ctypes.POINTER(_int),
                             ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_int)], _int),
    "dtp_colocated_affinity": ([ctypes.POINTER(ctypes.c_double), _int, _int, _int, ctypes.POINTER(_int),
                                ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_double)], _int),
    "dtp_layout_permutation": ([ctypes.POINTER(_int), _int, _int, _int, ctypes.POINTER(ctypes.c_int32)], _int),
    "permute_bf16": ([_vp, _vp, _vp, _i64, _i64, _int, _vp, _vp], _int),
    "agmm_backward": ([_vp, _i64, _i64, _i64, _int, _int, _ptrs, _vp, _vp, _vp, _vp, _vp, _int, _vp], _int),
    "reduce_residual_rmsnorm": ([_vp, _i64, _i64, _int, _ptrs, _vp, _vp, ctypes.c_float, _vp, _vp,
                                 _vp], _int),
    "dtp_accumulate": ([_vp, _i64, _i64, _int, _int, _int, _vp, _vp, _ptrs, _vp, ctypes.c_float, _vp,
                        _vp], _int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class SptlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def last_error() -> str:
    return (_lib.sptl_last_error() or b"").decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise SptlError(rc, last_error())


def _ptr_array(ptrs: Optional[Sequence[Optional[int]]]):
    if ptrs is None:
        return None
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return ctypes.cast(arr, _ptrs)


# ------------------------------------------------------------------------------------------
# raw C calls: integers in, status out (no exceptions)
# ------------------------------------------------------------------------------------------

def raw_agmm_chunked(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, shard_src, x_gathered, w,
                     y, y_dtype, compute, copy, timing=0) -> int:
    return _lib.agmm_chunked(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, _ptr_array(shard_src),
                             x_gathered, w, y, y_dtype, compute, copy, timing)


def raw_agmm_chunked_noalloc(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, shard_src, x_gathered, w,
                             y, y_dtype, compute) -> int:
    return _lib.agmm_chunked_noalloc(ctx, seq_len, hidden, n_local, tp, n_chunks, rank, _ptr_array(shard_src),
                                     x_gathered, w, y, y_dtype, compute)


def _np_ptr(arr, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def dtp_affinity_layout(affinity, tp: int, head_device=None, max_rounds: int = 100):
    """Head and neuron layouts of largest co-located affinity by coordinate ascent (see
    include/sptl.h).  affinity: [n_heads, n_neurons] array; head_device: the starting head layout
    (default: contiguous).  Returns (head_device, neuron_device, score, rounds) as numpy arrays."""
    import numpy as np
    a = np.ascontiguousarray(affinity, dtype=np.float64)
    n_heads, n_neurons = a.shape
    hd = (np.arange(n_heads) // max(1, n_heads // tp) if head_device is None else np.asarray(head_device))
    hd = np.ascontiguousarray(hd, dtype=np.intc).copy()
    nd = np.zeros(n_neurons, dtype=np.intc)
    score = ctypes.c_double()
    rounds = _int()
    _check(_lib.dtp_affinity_layout(_np_ptr(a, ctypes.c_double), n_heads, n_neurons, tp, max_rounds,
                                    _np_ptr(hd, _int), _np_ptr(nd, _int), ctypes.byref(score), ctypes.byref(rounds)))
    return hd, nd, score.value, rounds.value


def dtp_colocated_affinity(affinity, tp: int, head_device, neuron_device) -> float:
    import numpy as np
    a = np.ascontiguousarray(affinity, dtype=np.float64)
    hd = np.ascontiguousarray(head_device, dtype=np.intc)
    nd = np.ascontiguousarray(neuron_device, dtype=np.intc)
    score = ctypes.c_double()
    _check(_lib.dtp_colocated_affinity(_np_ptr(a, ctypes.c_double), a.shape[0], a.shape[1], tp, _np_ptr(hd, _int),
                                       _np_ptr(nd, _int), ctypes.byref(score)))
    return score.value


def dtp_layout_permutation(layout, tp: int, group: int = 1):
    import numpy as np
    lay = np.ascontiguousarray(layout, dtype=np.intc)
    perm = np.empty(lay.size * group, dtype=np.int32)
    _check(_lib.dtp_layout_permutation(_np_ptr(lay, _int), lay.size, tp, group, _np_ptr(perm, ctypes.c_int32)))
    return perm


def permute_bf16(src, dst, perm, *, dim: int, stream=None, ctx: Optional[Context] = None) -> None:
    """dst = src with rows (dim 0) or columns (dim 1) permuted by the device int32 tensor perm."""
    torch = _torch()
    rows, cols = src.shape
    _check(_lib.permute_bf16(_h(ctx), _dev_ptr(src, torch.bfloat16, "src"),
                             _dev_ptr(dst, torch.bfloat16, "dst", (rows, cols)), rows, cols, dim,
                             _dev_ptr(perm, torch.int32, "perm", ((rows if dim == 0 else cols),)), _stream(stream)))


def raw_agmm_backward(ctx, seq_len, hidden, n_local, tp, rank, shard_src, x_gathered, w, dy, dx, dw, dw_dtype,
                      compute) -> int:
    return _lib.agmm_backward(ctx, seq_len, hidden, n_local, tp, rank, _ptr_array(shard_src), x_gathered, w, dy, dx,
                              dw, dw_dtype, compute)


def raw_gemm_rs_chunked(ctx, seq_len, k_local, hidden, tp, n_chunks, rank, a, w, partial, dst, compute) -> int:
    return _lib.gemm_rs_chunked(ctx, seq_len, k_local, hidden, tp, n_chunks, rank, a, w, partial, _ptr_array(dst),
                                compute)


def raw_reduce_norm_agmm_chunked(ctx, n_partials, partials, residual, gamma, eps, residual_out, seq_len, hidden,
                                 n_local, tp, n_chunks, rank, shard_src, x_gathered, w, y, y_dtype, compute) -> int:
    return _lib.reduce_norm_agmm_chunked(ctx, n_partials, _ptr_array(partials), residual, gamma, eps, residual_out,
                                         seq_len, hidden, n_local, tp, n_chunks, rank, _ptr_array(shard_src),
                                         x_gathered, w, y, y_dtype, compute)


def raw_gemm_partial(ctx, seq_len, k_local, hidden, a, w, partial, out_dtype, stream) -> int:
    return _lib.gemm_partial(ctx, seq_len, k_local, hidden, a, w, partial, out_dtype, stream)


def raw_reduce_residual_rmsnorm(ctx, seq_len, hidden, tp, partials, residual, gamma, eps,
                                residual_out, y, stream) -> int:
    return _lib.reduce_residual_rmsnorm(ctx, seq_len, hidden, tp, _ptr_array(partials), residual, gamma,
                                        eps, residual_out, y, stream)


def raw_dtp_accumulate(ctx, seq_len, hidden, tp, delta, module_idx, residual, own_partial,
                       delayed_peers, gamma, eps, y, stream) -> int:
    return _lib.dtp_accumulate(ctx, seq_len, hidden, tp, delta, module_idx, residual, own_partial,
                               _ptr_array(delayed_peers), gamma, eps, y, stream)


# ------------------------------------------------------------------------------------------
# context
# ------------------------------------------------------------------------------------------

class Context:
    """A library context on one device (events + a lazily created copy stream)."""

    def __init__(self, device: int = 0):
        h = ctypes.c_void_p()
        _check(_lib.sptl_create(ctypes.byref(h), device))
        self.handle = h.value
        self.device = device

    def close(self) -> None:
        if self.handle:
            _lib.sptl_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover - interpreter shutdown order
        try:
            self.close()
        except Exception:
            pass

    def check(self) -> None:
        """Wait for this context's staged calls and raise SptlError on a recorded async failure."""
        _check(_lib.sptl_ctx_check(self.handle))

    def set_wait_timeout_us(self, us: int) -> None:
        """Bound on one chunk wait of later staged calls, in microseconds (0: the default 10 s)."""
        _check(_lib.sptl_ctx_set_wait_timeout_us(self.handle, int(us)))

    def set_copy_mode(self, mode, blit_workgroups: int = 0) -> None:
        """How later calls on this context stage their copies: "staged", "events", "blit" or
        "serial" (or the COPY_* value); blit_workgroups sizes the blit mode's copy kernels."""
        m = COPY_MODES[mode] if isinstance(mode, str) else int(mode)
        _check(_lib.sptl_ctx_set_copy_mode(self.handle, m, int(blit_workgroups)))

    def set_staging(self, order="ring", engines_per_peer: int = 0) -> None:
        """Chunk order of the gather ("ring" or "interleaved", or the ORDER_* value) and the link
        model (engines_per_peer > 0: each peer's copies on that many copy engines of their own)."""
        o = CHUNK_ORDERS[order] if isinstance(order, str) else int(order)
        _check(_lib.sptl_ctx_set_staging(self.handle, o, int(engines_per_peer)))

    def info(self) -> str:
        """How agmm_chunked stages chunks on this context (diagnostic)."""
        return (_lib.sptl_ctx_info(self.handle) or b"").decode()

    def timeline(self, n_chunks: int):
        """Per-chunk [copy start, copy end, GEMM start, GEMM end] (ms) of the last timed call."""
        buf = (ctypes.c_double * (4 * n_chunks))()
        _check(_lib.sptl_agmm_timeline(self.handle, buf, n_chunks))
        return [tuple(buf[4 * c:4 * c + 4]) for c in range(n_chunks)]


def _h(ctx) -> Optional[int]:
    return None if ctx is None else ctx.handle


# ------------------------------------------------------------------------------------------
# tensor wrappers
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(s) -> Optional[int]:
    torch = _torch()
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _dev_ptr(t, dtype, name, shape=None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _out_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("output must be bfloat16 or float32")


def agmm_chunked(shards, x_gathered, w, y, *, n_chunks: int, rank: int = 0, compute=None, copy=None,
                 timing: bool = False, ctx: Optional[Context] = None) -> None:
    """x_gathered = concat(shards); y = x_gathered @ w, chunk by chunk (see include/sptl.h)."""
    torch = _torch()
    tp = len(shards)
    M, K = x_gathered.shape
    N = w.shape[1]
    rows = M // tp if tp else 0
    src = [_dev_ptr(s, torch.bfloat16, f"shards[{q}]", (rows, K)) for q, s in enumerate(shards)]
    _check(raw_agmm_chunked(_h(ctx), M, K, N, tp, n_chunks, rank, src,
                            _dev_ptr(x_gathered, torch.bfloat16, "x_gathered"),
                            _dev_ptr(w, torch.bfloat16, "w", (K, N)),
                            _dev_ptr(y, y.dtype, "y", (M, N)), _out_dtype(y), _stream(compute),
                            None if copy is None else _stream(copy), int(bool(timing))))


def reduce_norm_agmm_chunked(partials, residual, gamma, eps: float, shards, x_gathered, w, y, *, n_chunks: int,
                             rank: int = 0, residual_out=None, compute=None, ctx: Optional[Context] = None) -> None:
    """Boundary epilogue of this rank's rows into its slot of x_gathered, then agmm_chunked, with the
    peers' staging started before the epilogue (see include/sptl.h).  shards[rank] is ignored."""
    torch = _torch()
    tp = len(shards)
    M, K = x_gathered.shape
    N = w.shape[1]
    rows = M // tp if tp else 0
    ps = [_dev_ptr(p, torch.bfloat16, f"partials[{i}]", (rows, K)) for i, p in enumerate(partials)]
    src = [None if q == rank else _dev_ptr(s, torch.bfloat16, f"shards[{q}]", (rows, K)) for q, s in enumerate(shards)]
    ro = None if residual_out is None else _dev_ptr(residual_out, torch.bfloat16, "residual_out", (rows, K))
    _check(raw_reduce_norm_agmm_chunked(_h(ctx), len(ps), ps, _dev_ptr(residual, torch.bfloat16, "residual", (rows, K)),
                                        _dev_ptr(gamma, torch.bfloat16, "gamma", (K,)), float(eps), ro, M, K, N, tp,
                                        n_chunks, rank, src, _dev_ptr(x_gathered, torch.bfloat16, "x_gathered"),
                                        _dev_ptr(w, torch.bfloat16, "w", (K, N)), _dev_ptr(y, y.dtype, "y", (M, N)),
                                        _out_dtype(y), _stream(compute)))


def agmm_backward(shards, x_gathered, w, dy, dx, dw, *, rank: int = 0, compute=None,
                  ctx: Optional[Context] = None) -> None:
    """Backward of agmm_chunked: x_gathered = concat(shards) (re-gathered under the dx GEMM),
    dx = dy @ w^T, dw = x_gathered^T @ dy (see include/sptl.h)."""
    torch = _torch()
    tp = len(shards)
    M, K = x_gathered.shape
    N = w.shape[1]
    rows = M // tp if tp else 0
    src = [_dev_ptr(s, torch.bfloat16, f"shards[{q}]", (rows, K)) for q, s in enumerate(shards)]
    _check(raw_agmm_backward(_h(ctx), M, K, N, tp, rank, src, _dev_ptr(x_gathered, torch.bfloat16, "x_gathered"),
                             _dev_ptr(w, torch.bfloat16, "w", (K, N)), _dev_ptr(dy, torch.bfloat16, "dy", (M, N)),
                             _dev_ptr(dx, torch.bfloat16, "dx", (M, K)), _dev_ptr(dw, dw.dtype, "dw", (K, N)),
                             _out_dtype(dw), _stream(compute)))


def gemm_rs_chunked(a, w, partial, dst, *, rank: int = 0, n_chunks: Optional[int] = None, stream=None,
                    ctx: Optional[Context] = None) -> None:
    """partial = a @ w, sub-slice by sub-slice in send order, each peer sub-slice copied into dst[q]
    by the copy engines while later ones compute (n_chunks sub-slices in all, default one per
    slice; dst[rank] is ignored; see include/sptl.h)."""
    torch = _torch()
    M, K = a.shape
    H = w.shape[1]
    tp = len(dst)
    rows = M // tp if tp else 0
    d = [None if (q == rank or t is None) else _dev_ptr(t, torch.bfloat16, f"dst[{q}]", (rows, H))
         for q, t in enumerate(dst)]
    _check(raw_gemm_rs_chunked(_h(ctx), M, K, H, tp, n_chunks or tp, rank, _dev_ptr(a, torch.bfloat16, "a"),
                               _dev_ptr(w, torch.bfloat16, "w", (K, H)),
                               _dev_ptr(partial, torch.bfloat16, "partial", (M, H)), d, _stream(stream)))


def gemm_partial(a, w, partial, *, stream=None, ctx: Optional[Context] = None) -> None:
    """partial = a @ w (row-parallel partial sum)."""
    torch = _torch()
    M, K = a.shape
    H = w.shape[1]
    _check(raw_gemm_partial(_h(ctx), M, K, H, _dev_ptr(a, torch.bfloat16, "a"),
                            _dev_ptr(w, torch.bfloat16, "w", (K, H)),
                            _dev_ptr(partial, partial.dtype, "partial", (M, H)), _out_dtype(partial),
                            _stream(stream)))


def reduce_residual_rmsnorm(partials, residual, gamma, eps: float, y, *, residual_out=None,
                            stream=None, ctx: Optional[Context] = None) -> None:
    """h = residual + sum(partials) -> residual_out (optional); y = RMSNorm(h) * gamma."""
    torch = _torch()
    R, H = residual.shape
    ps = [_dev_ptr(p, torch.bfloat16, f"partials[{i}]", (R, H)) for i, p in enumerate(partials)]
    ro = None if residual_out is None else _dev_ptr(residual_out, torch.bfloat16, "residual_out", (R, H))
    _check(raw_reduce_residual_rmsnorm(_h(ctx), R, H, len(ps), ps,
                                       _dev_ptr(residual, torch.bfloat16, "residual"),
                                       _dev_ptr(gamma, torch.bfloat16, "gamma", (H,)), float(eps), ro,
                                       _dev_ptr(y, torch.bfloat16, "y", (R, H)), _stream(stream)))


def dtp_accumulate(residual, own_partial, delayed_peers, gamma, eps: float, y, *, tp: int, delta: int,
                   module_idx: int, stream=None, ctx: Optional[Context] = None) -> None:
    """Delayed-TP residual update of module `module_idx` (in place on `residual`)."""
    torch = _torch()
    R, H = residual.shape
    own = None if own_partial is None else _dev_ptr(own_partial, torch.bfloat16, "own_partial", (R, H))
    peers = None if delayed_peers is None else [
        _dev_ptr(p, torch.bfloat16, f"delayed_peers[{i}]", (R, H)) for i, p in enumerate(delayed_peers)]
    g = None if gamma is None else _dev_ptr(gamma, torch.bfloat16, "gamma", (H,))
    yy = None if y is None else _dev_ptr(y, torch.bfloat16, "y", (R, H))
    _check(raw_dtp_accumulate(_h(ctx), R, H, tp, delta, module_idx,
                              _dev_ptr(residual, torch.bfloat16, "residual"), own, peers, g, float(eps),
                              yy, _stream(stream)))
