"""The library's affinity-aware sharding (host code behind the C ABI) against the oracle.

Layouts of KV heads and FFN neurons for delayed TP ("Affinity-Aware Sharding for Delayed Tensor
Parallelism", abstract): with continuous random affinities every step has one best answer, so the
library and the oracle must agree exactly on the layouts and the number of rounds, and on the
score up to the order of a float64 sum.  Affinities are synthetic (trained models are not used).
"""
import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd.synth import synthetic_affinity


@pytest.fixture(scope="module")
def sptl():
    from sp_transformer_linear_amd import sptl as mod
    return mod


CASES = [  # n_heads, n_neurons, tp, start ("contiguous" or a seed for a random balanced layout)
    (8, 96, 4, "contiguous"), (8, 768, 4, 5), (4, 64, 2, "contiguous"), (6, 30, 3, 7),
    (16, 64, 2, 3), (8, 3072, 4, "contiguous"), (2, 10, 1, "contiguous"),
]


def start_layout(n_heads, tp, start):
    hd = np.arange(n_heads) // (n_heads // tp)
    if start != "contiguous":
        hd = np.random.default_rng(start).permutation(hd)
    return hd


@pytest.mark.parametrize("n_heads,n_neurons,tp,start", CASES)
def test_layout_matches_oracle(sptl, n_heads, n_neurons, tp, start):
    a = synthetic_affinity(100 + n_neurons, n_heads, n_neurons, tp)
    hd0 = start_layout(n_heads, tp, start)
    hd, nd, score, rounds = sptl.dtp_affinity_layout(a, tp, hd0)
    ohd, ond, oscore, orounds = O.affinity_layout(a, tp, hd0)
    assert rounds == orounds
    assert np.array_equal(hd, ohd) and np.array_equal(nd, ond)
    assert abs(score - oscore) <= 1e-12 * abs(oscore)
    assert np.bincount(nd, minlength=tp).tolist() == [n_neurons // tp] * tp
    assert score >= O.colocated_affinity(a, hd0, np.arange(n_neurons) // (n_neurons // tp))  # beats contiguous
    assert sptl.dtp_colocated_affinity(a, tp, hd, nd) == pytest.approx(oscore, rel=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_first_round_matches_oracle(sptl, seed):
    """One round from a random start: the exact neuron step, then the head search."""
    a = np.random.default_rng(seed).standard_normal((6, 48))
    hd0 = start_layout(6, 3, seed)
    hd, nd, score, rounds = sptl.dtp_affinity_layout(a, 3, hd0, max_rounds=1)
    assert rounds == 1
    ond = O.balanced_neuron_assignment(a, hd0, 3)
    assert np.array_equal(nd, ond)
    assert np.array_equal(hd, O.best_head_layout(a, ond, 3))


def test_planted_optimum(sptl):
    rng = np.random.default_rng(9)
    gh = rng.permutation(np.arange(8) % 4)
    gn = rng.permutation(np.arange(256) % 4)
    a = (gh[:, None] == gn[None, :]).astype(np.float64)
    hd, nd, score, _ = sptl.dtp_affinity_layout(a, 4, gh)
    assert score == a.sum() and np.array_equal(nd, gn) and np.array_equal(hd, gh)


def test_layout_permutation_matches_oracle(sptl):
    rng = np.random.default_rng(4)
    lay = rng.permutation(np.arange(16) % 4)
    for group in (1, 128):
        assert np.array_equal(sptl.dtp_layout_permutation(lay, 4, group), O.layout_permutation(lay, 4, group))


def test_affinity_validation(sptl):
    import ctypes
    lib = sptl._lib
    a = np.ones((4, 8))
    hd = np.array([0, 0, 1, 1], dtype=np.intc)
    nd = np.zeros(8, dtype=np.intc)
    s, r = ctypes.c_double(), ctypes.c_int()
    P = sptl._np_ptr
    A = P(a, ctypes.c_double)

    def call(aa=A, nh=4, nn=8, tp=2, mr=10, h=hd):
        h = np.ascontiguousarray(h, dtype=np.intc).copy()
        return lib.dtp_affinity_layout(aa, nh, nn, tp, mr, P(h, ctypes.c_int), P(nd, ctypes.c_int),
                                       ctypes.byref(s), ctypes.byref(r))

    assert call() == 0
    assert lib.dtp_affinity_layout(None, 4, 8, 2, 10, None, None, None, None) == 1
    assert call(tp=0) == 6 and call(tp=65) == 6 and call(mr=0) == 6
    assert call(tp=3) == 3                                   # 4 heads over 3 devices
    assert call(h=[0, 0, 0, 1]) == 6                         # unbalanced start
    assert call(h=[0, 0, 1, 2]) == 6                         # device out of range
    bad = a.copy()
    bad[1, 2] = np.nan
    assert call(aa=P(bad, ctypes.c_double)) == 6
    big = np.ones((32, 64))
    h32 = np.arange(32) // 16
    assert call(aa=P(big, ctypes.c_double), nh=32, nn=64, h=h32) == 8  # C(32, 16) head layouts
    assert lib.dtp_layout_permutation(P(hd, ctypes.c_int), 4, 1, 1, None) == 1
    perm = np.empty(4, dtype=np.int32)
    assert lib.dtp_layout_permutation(P(hd, ctypes.c_int), 4, 1, 1, P(perm, ctypes.c_int32)) == 6  # device 1 >= tp
    assert lib.permute_bf16(None, None, None, 8, 8, 0, None, None) == 1
    assert lib.permute_bf16(None, 0x1000, 0x2000, 8, 12, 0, 0x3000, None) == 3
    assert lib.permute_bf16(None, 0x1000, 0x2000, 8, 16, 2, 0x3000, None) == 6
    assert lib.permute_bf16(None, 0x1000, 0x1000, 8, 16, 0, 0x3000, None) == 6
    assert lib.permute_bf16(None, 0x1008, 0x2000, 8, 16, 0, 0x3000, None) == 4
    assert lib.permute_bf16(None, 0x1000, 0x2000, 8, 16, 0, 0x3002, None) == 4
