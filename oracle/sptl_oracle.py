"""Reference oracle for one GPU's share of the sequence-parallel tensor-parallel linear layer.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, obviously correct float64 CPU
statement of what the layer computes.  It exists to check the HIP path, never to stand in
for it: only the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it.  It shares no code with the HIP library (no kernels, headers, helpers or
constant tables) and imports nothing from the product package.

Every function takes bf16 tensors either as raw storage bits (``numpy.uint16``) or as
float64 values, decodes bits exactly, and does all arithmetic in float64 with numpy.  The
only library primitive used as a step is the float64 matrix product ``@``; there is no
chunking, fusion or reordering beyond what each definition states.

Sources (web pages; section named, no line numbers):
  [AReaL] "[Feature] Async Tensor Parallelism for Archon Engine" (AReaL issue), sections
          "TP Communication Is on Activations, Not Weights" and "Potential Solution".
  [DTP]   "Affinity-Aware Sharding for Delayed Tensor Parallelism" (arXiv abstract).
  [MLM]   "Add forward all-gather overlap" (Megatron-LM pull request #5513), "Summary",
          "Scope" and "Observations".

Readings taken where the pages are silent (each is listed, with the reason, in the design
notes of the repository):
  * all-gather order: rank-major blocks of rows (a gather along the sequence dimension);
  * weight orientation: logical [in, out], row-major;
  * RMSNorm: textbook form, mean of squares over the hidden dimension, epsilon inside the
    square root, elementwise gain, no bias and no centring.  The pages only say that the
    norm reduces over the hidden dimension; the formula itself is pinned to the textbook
    definition, not to the pages;
  * delayed TP: a "module" is one attention or FFN sub-layer; module l adds its own partial
    and, when l >= delta, the peers' partials of module l - delta, then normalises; after
    the last module, delta flush steps add the outstanding peer partials without a norm.
"""

from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "round_to_bf16",
    "f64_to_bf16_bits",
    "all_gather_sequence",
    "agmm",
    "agmm_backward",
    "gemm_partial",
    "rmsnorm",
    "reduce_residual_rmsnorm",
    "dtp_accumulate",
    "dtp_sequence",
    "colocated_affinity",
    "balanced_neuron_assignment",
    "best_head_layout",
    "affinity_layout",
    "layout_permutation",
    "permute",
]


# ---------------------------------------------------------------------------------------
# bf16 storage <-> float64 values
# ---------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 storage bits.

    bf16 is the upper half of an IEEE-754 binary32 word (1 sign, 8 exponent, 7 fraction
    bits), so the value is the binary32 whose top 16 bits are ``bits`` and whose low 16 bits
    are zero.  Converting that binary32 to float64 is exact.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 storage bits must be numpy.uint16")
    word = b.astype(np.uint32) << np.uint32(16)
    return word.view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    """Accept bf16 bits (uint16) or real values; return float64 values."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (as float64 values).

    bf16 keeps 8 significant bits.  Writing x = m * 2**e with 0.5 <= |m| < 1 (frexp), the
    bf16 value is rint(m * 2**8) * 2**(e - 8), and numpy's rint rounds halves to even.
    This covers the normal bf16 range, which is the only range the layer's values occupy;
    zero maps to zero.  Overflow and bf16 subnormals are outside the domain of this oracle.
    """
    v = _as_f64(x)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 storage bits of ``round_to_bf16(x)`` (the rounded value is exact in binary32)."""
    r = round_to_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------------------
# (1) sequence all-gather feeding the column-parallel GEMM       [AReaL "Potential Solution"]
# ---------------------------------------------------------------------------------------

def all_gather_sequence(shards: Sequence) -> np.ndarray:
    """All-gather along the sequence dimension.

    Megatron-style sequence parallelism keeps each TP rank's slice of the tokens; the
    all-gather before the column-parallel linear redistributes these activations so every
    rank holds all tokens [AReaL, "TP Communication Is on Activations, Not Weights"].  The
    gathered tensor is the rank-major concatenation of the shards along rows.
    """
    return np.concatenate([_as_f64(s) for s in shards], axis=0)


def agmm(shards: Sequence, w) -> tuple[np.ndarray, np.ndarray]:
    """All-gather then matmul: returns (X, Y) with X = gather(shards), Y = X @ W.

    The page describes splitting all-gather + matmul into chunked, pipelined pieces
    [AReaL, "Potential Solution", intra-layer overlap].  Chunking splits the rows of X only,
    so every element of Y is the same sum; the oracle states the unchunked definition.
    ``w`` is the column-parallel weight shard, logical [in, out].
    """
    x = all_gather_sequence(shards)
    return x, x @ _as_f64(w)


def agmm_backward(shards: Sequence, w, dy) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Backward of Y = gather(shards) @ W for an upstream gradient dY: returns (X, dX, dW).

    The backward pass all-gathers the activation again [MLM, "Scope": backward all-gathers
    are present, not yet overlapped], because the weight gradient needs every token while each
    rank keeps only its shard.  The gradients are those of any linear map Y = X W:
        dX = dY W^T   (this rank's partial sum of the input gradient, since W is its shard of
                       the columns; its sequence slices are reduce-scattered over the ranks)
        dW = X^T dY   (the gradient of this rank's weight shard)
    stated here unchunked and in float64.
    """
    x = all_gather_sequence(shards)
    g = _as_f64(dy)
    wt = _as_f64(w).T
    return x, g @ wt, x.T @ g


# ---------------------------------------------------------------------------------------
# (2) row-parallel GEMM producing this rank's partial sum          [DTP abstract; AReaL]
# ---------------------------------------------------------------------------------------

def gemm_partial(a, w) -> np.ndarray:
    """This rank's partial output of a row-parallel linear: P = A @ W_row.

    A row-parallel linear splits the reduction dimension over the TP ranks; each rank's
    product is a partial sum that the TP all-reduce (or, under delayed TP, the deferred
    gather) completes [DTP abstract: "partial output"; AReaL, "Potential Solution":
    reduce-scatter at the end of a sub-layer].
    """
    return _as_f64(a) @ _as_f64(w)


# ---------------------------------------------------------------------------------------
# (3) reduce + residual + RMSNorm                                   [AReaL "Potential Solution"]
# ---------------------------------------------------------------------------------------

def rmsnorm(h, gamma, eps: float) -> np.ndarray:
    """Textbook RMSNorm over the last (hidden) dimension.

    y[i, j] = h[i, j] / sqrt(mean_j(h[i, j]**2) + eps) * gamma[j].  The page fixes only that
    the norm reduces over the hidden dimension [AReaL, "Potential Solution", sub-layer
    boundary overlap]; rows are independent, which is why the norm commutes with a gather
    along the sequence.
    """
    hv = _as_f64(h)
    g = _as_f64(gamma)
    ms = np.mean(hv * hv, axis=-1, keepdims=True)
    return hv / np.sqrt(ms + float(eps)) * g


def reduce_residual_rmsnorm(partials: Iterable, residual, gamma, eps: float):
    """Sub-layer boundary: h = residual + sum of the TP partials, y = RMSNorm(h).

    The window between one sub-layer's reduce-scatter and the next all-gather holds the
    residual add and the RMSNorm [AReaL, "Potential Solution"].  Partials are added in index
    order.  Returns (h, y) in float64.
    """
    h = _as_f64(residual).copy()
    for p in partials:
        h = h + _as_f64(p)
    return h, rmsnorm(h, gamma, eps)


# ---------------------------------------------------------------------------------------
# (4) delayed tensor parallelism                                    [DTP abstract]
# ---------------------------------------------------------------------------------------

def dtp_accumulate(residual, own, peers: Sequence, gamma=None, eps: float = 0.0):
    """One delayed-TP residual update: x' = x + own + sum(peers); y = RMSNorm(x').

    Under delayed TP each device adds its own partial output to its residual stream at
    once, and adds the other devices' partials delta modules later [DTP abstract].  ``own``
    may be None (a flush step after the last module) and ``peers`` may be empty (a module
    l < delta, whose peers' partials do not exist yet).  With ``gamma`` None no norm is
    taken and y is None.
    """
    x = _as_f64(residual).copy()
    if own is not None:
        x = x + _as_f64(own)
    for p in peers:
        x = x + _as_f64(p)
    y = None if gamma is None else rmsnorm(x, gamma, eps)
    return x, y


def dtp_sequence(x0, owns: Sequence, peers: Sequence[Sequence], delta: int, gamma, eps: float,
                 store_bf16: bool = False):
    """Run delayed TP over L modules followed by delta flush steps.

    ``owns[l]`` is this rank's partial of module l; ``peers[l]`` lists the other ranks'
    partials of module l in ascending rank order.  Module l adds owns[l] and, when
    l >= delta, peers[l - delta], then normalises [DTP abstract].  After module L - 1, the
    flush steps l = L .. L + delta - 1 add peers[l - delta] with no own partial and no norm.

    With ``store_bf16`` the residual stream is rounded to bf16 after every step, as it is
    when it is kept in bf16 storage between modules; each step's arithmetic stays float64.

    Returns (steps, x_final, x_immediate):
      steps[l] = (x after module l, y of module l) for l < L, then (x, None) per flush step;
      x_final  = residual after the last flush step;
      x_immediate = x0 + sum_l (owns[l] + sum_q peers[l][q]), the blocking-all-reduce TP
                    result, which delayed TP reaches once every partial has arrived.
    """
    if delta < 0:
        raise ValueError("delta must be >= 0")
    L = len(owns)
    if len(peers) != L:
        raise ValueError("need one peer list per module")
    x = _as_f64(x0).copy()
    steps = []
    for l in range(L + delta):
        own = owns[l] if l < L else None
        late = peers[l - delta] if l >= delta else []
        x, y = dtp_accumulate(x, own, late, gamma if l < L else None, eps)
        if store_bf16:
            x = round_to_bf16(x)
        steps.append((x, y))
    x_imm = _as_f64(x0).copy()
    for l in range(L):
        x_imm = x_imm + _as_f64(owns[l])
        for p in peers[l]:
            x_imm = x_imm + _as_f64(p)
    return steps, x, x_imm


# ---------------------------------------------------------------------------------------
# (5) affinity-aware sharding for delayed TP                        [DTP abstract]
# ---------------------------------------------------------------------------------------

def colocated_affinity(affinity, head_device, neuron_device) -> float:
    """Co-located affinity of a layout: the sum of affinity[h, j] over every KV head h and FFN
    neuron j placed on the same device [DTP abstract: "maximising the affinity between the KV
    heads and the FFN neurons co-located on a device"]."""
    a = np.asarray(affinity, dtype=np.float64)
    hd = np.asarray(head_device)
    nd = np.asarray(neuron_device)
    return float(np.sum(a * (hd[:, None] == nd[None, :])))


def balanced_neuron_assignment(affinity, head_device, tp: int) -> np.ndarray:
    """For fixed heads, the neuron layout with n_neurons / tp neurons per device of largest
    co-located affinity [DTP abstract: "an exact balanced assignment of neurons"].

    Neuron j placed on device d contributes the sum of its affinities to the heads on d.  The
    balanced assignment is a linear assignment of neurons to device slots (each device repeated
    n_neurons / tp times), solved exactly by scipy's linear_sum_assignment (a library step)."""
    from scipy.optimize import linear_sum_assignment
    a = np.asarray(affinity, dtype=np.float64)
    hd = np.asarray(head_device)
    n = a.shape[1]
    value = np.stack([a[hd == d].sum(axis=0) for d in range(tp)])   # [tp, n_neurons]
    slot_device = np.repeat(np.arange(tp), n // tp)                  # [n_neurons] slots
    rows, cols = linear_sum_assignment(value[slot_device].T, maximize=True)
    out = np.empty(n, dtype=np.int64)
    out[rows] = slot_device[cols]
    return out


def best_head_layout(affinity, neuron_device, tp: int) -> np.ndarray:
    """For fixed neurons, the head layout with n_heads / tp heads per device of largest
    co-located affinity, by trying every one [DTP abstract: "an exhaustive search over the KV
    head partitions"].  Devices are told apart by the neurons they hold, so layouts are
    assignments of heads to devices.  They are tried in lexicographic order of (device of head
    0, device of head 1, ...) and the first best one is kept."""
    import itertools
    a = np.asarray(affinity, dtype=np.float64)
    nd = np.asarray(neuron_device)
    n_heads = a.shape[0]
    t = np.stack([a[:, nd == d].sum(axis=1) for d in range(tp)], axis=1)  # [n_heads, tp]
    best, best_s = None, -np.inf
    for cand in itertools.product(range(tp), repeat=n_heads):
        if any(cand.count(d) != n_heads // tp for d in range(tp)):
            continue
        s = sum(t[h, d] for h, d in enumerate(cand))
        if s > best_s:
            best, best_s = cand, s
    return np.array(best, dtype=np.int64)


def affinity_layout(affinity, tp: int, head_device, max_rounds: int = 100):
    """Coordinate ascent on the co-located affinity [DTP abstract: "a coordinate-ascent optimiser
    that alternates an exact balanced assignment of neurons with an exhaustive search over the
    KV head partitions"], from the head layout given: each round assigns the neurons for the
    current heads, then searches the heads for those neurons; it stops after a round that does
    not raise the score (or after max_rounds).  Returns (heads, neurons, score, rounds)."""
    hd = np.asarray(head_device, dtype=np.int64)
    prev = -np.inf
    rounds = 0
    while rounds < max_rounds:
        nd = balanced_neuron_assignment(affinity, hd, tp)
        hd = best_head_layout(affinity, nd, tp)
        s = colocated_affinity(affinity, hd, nd)
        rounds += 1
        if not s > prev:
            break
        prev = s
    return hd, nd, s, rounds


def layout_permutation(layout, tp: int, group: int = 1) -> np.ndarray:
    """Index order that shards a layout: device 0's items ascending, then device 1's, ...; item
    i stands for the group indices i*group .. i*group + group - 1 [DTP abstract: "permuting the
    dense model before sharding"]."""
    lay = np.asarray(layout)
    items = np.concatenate([np.flatnonzero(lay == d) for d in range(tp)])
    return (items[:, None] * group + np.arange(group)[None, :]).reshape(-1)


def permute(x, perm, dim: int) -> np.ndarray:
    """x with its rows (dim 0) or columns (dim 1) taken in the order perm."""
    return np.take(np.asarray(x), np.asarray(perm), axis=dim)

