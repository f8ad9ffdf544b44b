"""Seeded synthetic inputs for the SP-TP linear layer workloads.

This module only draws random numbers and stores them as bf16 bits; it holds none of the
layer's arithmetic, so both the HIP path and the float64 oracle can take their inputs from
it.  It imports nothing from the rest of the package.

Recipe (the same for every workload):
  * every tensor has a spawn key (kind, index...) under the workload seed;
  * a tensor is drawn in fixed blocks of BLOCK_ROWS rows; block b is drawn from
    Generator(PCG64(SeedSequence(seed, spawn_key=key + (b,)))), so any subset of rows can
    be regenerated on its own and the result does not depend on the thread count;
  * values are standard_normal float32 * std + mean (float32 arithmetic), then rounded to
    bf16 with round-to-nearest-even on the binary32 bit pattern.

N(mu, v) in a workload description is read as mean mu and *variance* v, so N(0, 1/K) is the
fan-in variance that keeps the GEMM outputs at unit variance.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
from numpy.random import PCG64, Generator, SeedSequence

BLOCK_ROWS = 1024

# spawn-key prefix per tensor kind
_KIND = {
    "shard": 0,      # sequence shard of rank q:            [M/tp, K]
    "w_col": 1,      # column-parallel weight shard:        [K, N]
    "w_row": 2,      # row-parallel weight shard:           [K_row, H]
    "a_row": 3,      # input of the row-parallel GEMM:      [M, K_row]
    "partial": 4,    # partial sum p of the reduce:         [R, H]
    "residual": 5,   # residual stream:                     [R, H]
    "gamma": 6,      # RMSNorm gain:                        [H]
    "own": 7,        # delayed TP: own partial of module l  [R, H]
    "peer": 8,       # delayed TP: partial of peer q, module l
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 storage bits, nearest-even (finite inputs only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: int, key: Sequence[int], rows: int, cols: int, std: float,
                mean: float = 0.0, row_idx: Optional[Sequence[int]] = None) -> np.ndarray:
    """bf16 bits of a [rows, cols] tensor of N(mean, std**2) samples (or of rows ``row_idx``)."""
    key = tuple(int(k) for k in key)
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    if row_idx is None:
        want = None
        blocks = list(range(nblk))
    else:
        want = np.asarray(row_idx, dtype=np.int64)
        if want.size and (want.min() < 0 or want.max() >= rows):
            raise IndexError("row index out of range")
        blocks = sorted(set((want // BLOCK_ROWS).tolist()))

    def draw(b: int) -> np.ndarray:
        r0 = b * BLOCK_ROWS
        n = min(BLOCK_ROWS, rows - r0)
        g = Generator(PCG64(SeedSequence(seed, spawn_key=key + (b,))))
        z = g.standard_normal((n, cols), dtype=np.float32)
        z *= np.float32(std)
        if mean != 0.0:
            z += np.float32(mean)
        return f32_to_bf16_bits(z)

    if want is None:
        out = np.empty((rows, cols), dtype=np.uint16)
        def fill(b: int) -> None:
            r0 = b * BLOCK_ROWS
            blk = draw(b)
            out[r0:r0 + blk.shape[0]] = blk
        if len(blocks) > 1 and rows * cols >= (1 << 22):
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, blocks))
        else:
            for b in blocks:
                fill(b)
        return out
    got = {b: draw(b) for b in blocks}
    out = np.empty((want.size, cols), dtype=np.uint16)
    for i, r in enumerate(want.tolist()):
        out[i] = got[r // BLOCK_ROWS][r % BLOCK_ROWS]
    return out


@dataclass(frozen=True)
class Workload:
    """Shapes and input distributions of one SP-TP linear workload (this rank = 0).

    M: gathered sequence length; K: hidden size entering the column GEMM; N: local width of
    the column GEMM output; K_row: local reduction size of the row GEMM; H: hidden size of the
    row GEMM output and of the reduce + RMSNorm; P: partials summed by the reduce; delta:
    delayed-TP delay (None when the workload has no delayed-TP part).
    """

    name: str
    description: str
    tp: int
    n_chunks: int
    M: int
    K: int
    N: int
    K_row: int
    H: int
    P: int
    eps: float = 1e-6
    delta: Optional[int] = None
    dtp_modules: int = 0
    seed: int = 0
    var_x: float = 1.0
    var_w_col: float = field(default=0.0)   # 0 -> 1/K
    var_w_row: float = field(default=0.0)   # 0 -> 1/K_row
    var_a: float = 1.0
    var_partial: float = 0.02
    var_residual: float = 1.0

    # ---- shapes -------------------------------------------------------------------------
    @property
    def rows_per_rank(self) -> int:
        return self.M // self.tp

    @property
    def rows_per_chunk(self) -> int:
        return self.M // self.n_chunks

    @property
    def R(self) -> int:
        """Rows of the reduce / delayed-TP epilogue."""
        return self.M

    # ---- tensors (bf16 bits) --------------------------------------------------------------
    def _std(self, var: float) -> float:
        return math.sqrt(var)

    def shard(self, q: int, row_idx=None) -> np.ndarray:
        return normal_bf16(self.seed, (_KIND["shard"], q), self.rows_per_rank, self.K,
                           self._std(self.var_x), row_idx=row_idx)

    def w_col(self) -> np.ndarray:
        v = self.var_w_col or 1.0 / self.K
        return normal_bf16(self.seed, (_KIND["w_col"],), self.K, self.N, self._std(v))

    def w_row(self) -> np.ndarray:
        v = self.var_w_row or 1.0 / self.K_row
        return normal_bf16(self.seed, (_KIND["w_row"],), self.K_row, self.H, self._std(v))

    def a_row(self, row_idx=None) -> np.ndarray:
        return normal_bf16(self.seed, (_KIND["a_row"],), self.M, self.K_row,
                           self._std(self.var_a), row_idx=row_idx)

    def partial(self, p: int, row_idx=None) -> np.ndarray:
        return normal_bf16(self.seed, (_KIND["partial"], p), self.R, self.H,
                           self._std(self.var_partial), row_idx=row_idx)

    def residual(self, row_idx=None) -> np.ndarray:
        return normal_bf16(self.seed, (_KIND["residual"],), self.R, self.H,
                           self._std(self.var_residual), row_idx=row_idx)

    def gamma(self) -> np.ndarray:
        """RMSNorm gain: bf16(1 + 0.1 * N(0, 1))."""
        return normal_bf16(self.seed, (_KIND["gamma"],), 1, self.H, 0.1, mean=1.0)[0]

    def own(self, module: int, row_idx=None) -> np.ndarray:
        return normal_bf16(self.seed, (_KIND["own"], module), self.R, self.H,
                           self._std(self.var_partial), row_idx=row_idx)

    def peer(self, module: int, q: int, row_idx=None) -> np.ndarray:
        return normal_bf16(self.seed, (_KIND["peer"], module, q), self.R, self.H,
                           self._std(self.var_partial), row_idx=row_idx)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny_tp2": Workload(
        name="tiny_tp2",
        description="tiny SP-TP linear, tp=2: 2 sequence chunks of 128x256, column shard "
                    "256x512, row shard 512x256, 2 partials of 256x256, seed 0",
        tp=2, n_chunks=2, M=256, K=256, N=512, K_row=512, H=256, P=2),
    "h100_page_8192x4096": Workload(
        name="h100_page_8192x4096",
        description="M=8192 tokens x dim=4096 in 8 chunks of 1024 rows (7 staged), "
                    "4096x4096 weight, then 8 partials + residual + RMSNorm over 4096",
        tp=8, n_chunks=8, M=8192, K=4096, N=4096, K_row=4096, H=4096, P=8),
    "qwen2_7b_tp4_16384": Workload(
        name="qwen2_7b_tp4_16384",
        description="Qwen2-7B-like TP=4 SP shard: seq 16384 x hidden 3584 in 4 chunks, "
                    "column shard 3584x9472, row shard 4736x3584, 4 partials + RMSNorm",
        tp=4, n_chunks=4, M=16384, K=3584, N=9472, K_row=4736, H=3584, P=4),
    "msweep_65536x4096": Workload(
        name="msweep_65536x4096",
        description="M=65536 x dim=4096 in 8 chunks of 8192 rows, 4096x4096 weight, "
                    "8 partials + residual + RMSNorm on 65536x4096",
        tp=8, n_chunks=8, M=65536, K=4096, N=4096, K_row=4096, H=4096, P=8),
    "dtp_qwen3_0p6b_tp4": Workload(
        name="dtp_qwen3_0p6b_tp4",
        description="delayed TP (delta=1), Qwen3-0.6B-shaped shard, tp=4: 32768 tokens, "
                    "hidden 1024, FFN 3072 (768 per device); own partial now, 3 peer "
                    "partials one module later, then RMSNorm",
        tp=4, n_chunks=4, M=32768, K=1024, N=768, K_row=768, H=1024, P=4,
        delta=1, dtp_modules=4),
}


def synthetic_affinity(seed: int, n_heads: int, n_neurons: int, tp: int) -> np.ndarray:
    """Synthetic KV-head / FFN-neuron affinities [n_heads, n_neurons] float64 for the sharding
    optimiser (real ones need a trained model): exp(N(0, 1)), times 3 where a head and a neuron
    share a hidden group (tp balanced groups placed at random), so that there is a layout to find."""
    rng = np.random.default_rng(seed)
    gh = rng.permutation(np.arange(n_heads) % tp)
    gn = rng.permutation(np.arange(n_neurons) % tp)
    return np.exp(rng.standard_normal((n_heads, n_neurons))) * np.where(gh[:, None] == gn[None, :], 3.0, 1.0)

