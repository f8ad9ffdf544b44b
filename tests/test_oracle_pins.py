"""Pins of the float64 oracle to facts other than itself (CPU only).

Each check is written as a function of the implementation under test, so the same checks
also run against deliberately broken copies of the oracle (bottom of the file): every
planted mistake must make at least one pin fail.

Pins used: hand-worked examples (tests/golden, each with its citation), exact rational
brute force on tiny inputs (tests/brute.py), closed forms of RMSNorm, special weights that
make the product exact (identity, permutation, one-hot rows), the invariants the pages fix
(chunked == unchunked gather-matmul; norm commutes with the sequence gather; delayed TP
after its flush equals the immediate all-reduce sum), the TP identity of a K-split
row-parallel GEMM, and a second, independent bf16 rounding routine.
"""

import ast
import math
import operator
import os
import types

import numpy as np
import pytest

import oracle.sptl_oracle as O
from sp_transformer_linear_amd import synth
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------
# golden-file reader: "key: v v v ; v v v", values are arithmetic expressions with sqrt()
# ----------------------------------------------------------------------------------------

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg, ast.UAdd: operator.pos}


def _eval(expr: str) -> float:
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.BinOp) and type(n.op) in _OPS:
            return _OPS[type(n.op)](ev(n.left), ev(n.right))
        if isinstance(n, ast.UnaryOp) and type(n.op) in _OPS:
            return _OPS[type(n.op)](ev(n.operand))
        if (isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id == "sqrt"
                and len(n.args) == 1):
            return math.sqrt(ev(n.args[0]))
        raise ValueError(f"bad golden expression {expr!r}")
    return ev(ast.parse(expr, mode="eval"))


def load_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows = [[_eval(t) for t in r.split()] for r in val.split(";")]
            out[key.strip()] = np.array(rows, dtype=np.float64)
    return out


def bits(values) -> np.ndarray:
    """bf16 bits of values that are exactly representable (checked)."""
    v = np.asarray(values, dtype=np.float64)
    b = synth.f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f64(b), v), "golden value not exact in bf16"
    return b


def rand_bits(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ----------------------------------------------------------------------------------------
# checks, parameterised by implementation (a module-like object with the oracle's API)
# ----------------------------------------------------------------------------------------

def check_bf16_decode(impl):
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0 + 2.0 ** -7, 0x0000: 0.0,
             0x8000: -0.0, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126,
             0x0001: 2.0 ** -133, 0x4049: 3.140625}
    got = impl.bf16_bits_to_f64(np.array(list(cases), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(cases.values())))
    rng = np.random.default_rng(1)
    b = rng.integers(0, 1 << 16, 4000).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]  # finite patterns only
    want = np.array([float(brute.bf16_value(x)) for x in b.tolist()])
    assert np.array_equal(impl.bf16_bits_to_f64(b), want)


def check_round_to_bf16(impl):
    # ties to even at 1: ulp = 2^-7
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -30,
                  3.0, 0.0, 1 + 2.0 ** -9])
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7, 3.0, 0.0, 1.0])
    assert np.array_equal(impl.round_to_bf16(x), want)
    # agrees with an independent routine (the bit trick on binary32) on binary32 inputs
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    other = O.bf16_bits_to_f64(synth.f32_to_bf16_bits(f))
    assert np.array_equal(impl.round_to_bf16(f.astype(np.float64)), other)


def check_f64_to_bf16_bits(impl):
    # hand-worked patterns: 1/3 = 1.0101010|1010...b * 2^-2 rounds up to fraction 0101011, so
    # 0 01111101 0101011 = 0x3EAB; 1 + 2^-8 and -(1 + 2^-8) are ties that go to the even 1.0;
    # 1 + 3 * 2^-8 ties to the even 1 + 2^-6 (0x3F82); 1 + 2^-8 + 2^-30 is above the tie and
    # rounds up (a double rounding through binary32 would lose the 2^-30 and go down);
    # 65504 = 1.1111111|111b * 2^15 rounds up with a carry into the exponent: 2^16 = 0x4780
    cases = {1.0: 0x3F80, -2.0: 0xC000, 0.0: 0x0000, 3.140625: 0x4049, 1.0 / 3.0: 0x3EAB,
             1 + 2.0 ** -8: 0x3F80, -(1 + 2.0 ** -8): 0xBF80, 1 + 3 * 2.0 ** -8: 0x3F82,
             1 + 2.0 ** -8 + 2.0 ** -30: 0x3F81, 2.0 ** -126: 0x0080, 65504.0: 0x4780}
    got = impl.f64_to_bf16_bits(np.array(list(cases), dtype=np.float64))
    assert np.array_equal(got, np.array(list(cases.values()), dtype=np.uint16))
    # every finite normal bf16 value (and +0) encodes back to its own bits
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    b = b[((exp >= 1) & (exp <= 254)) | (b == 0)]
    assert np.array_equal(impl.f64_to_bf16_bits(O.bf16_bits_to_f64(b)), b)
    # float64 inputs between bf16 values, against the field-by-field brute encoder
    rng = np.random.default_rng(13)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    want = np.array([brute.bf16_bits(brute.Fraction(float(v))) for v in x], dtype=np.uint16)
    assert np.array_equal(impl.f64_to_bf16_bits(x), want)


def check_agmm_golden(impl):
    g = load_golden("agmm_worked_tp3.txt")
    shards = [bits(g[f"shard{q}"]) for q in range(3)]
    x, y = impl.agmm(shards, bits(g["w"]))
    assert np.array_equal(x, g["x"])
    assert np.array_equal(y, g["y"])


def check_agmm_brute(impl):
    rng = np.random.default_rng(3)
    for tp, rows, k, n in ((2, 2, 3, 5), (3, 1, 4, 2), (4, 2, 2, 3), (2, 3, 5, 4)):
        shards = [rand_bits(rng, (rows, k)) for _ in range(tp)]
        w = rand_bits(rng, (k, n), 0.5)
        x, y = impl.agmm(shards, w)
        bx = brute.gather([brute.matrix(s) for s in shards])
        by = brute.matmul(bx, brute.matrix(w))
        assert np.array_equal(x, np.array([[float(v) for v in r] for r in bx]))
        assert np.allclose(y, np.array([[float(v) for v in r] for r in by]), rtol=1e-13, atol=0)


def check_gemm_brute(impl):
    rng = np.random.default_rng(4)
    for m, k, n in ((1, 1, 1), (3, 7, 2), (5, 8, 6), (2, 16, 3)):
        a = rand_bits(rng, (m, k))
        w = rand_bits(rng, (k, n), 0.25)
        want = brute.matmul(brute.matrix(a), brute.matrix(w))
        assert np.allclose(impl.gemm_partial(a, w), np.array([[float(v) for v in r] for r in want]),
                           rtol=1e-13, atol=0)


def check_special_weights(impl):
    rng = np.random.default_rng(5)
    k = 12
    shards = [rand_bits(rng, (3, k)) for _ in range(2)]
    eye = bits(np.eye(k))
    x, y = impl.agmm(shards, eye)
    assert np.array_equal(y, x)
    perm = rng.permutation(k)
    pw = np.zeros((k, k))
    pw[perm, np.arange(k)] = 1.0  # column j picks input feature perm[j]
    x, y = impl.agmm(shards, bits(pw))
    assert np.array_equal(y, x[:, perm])
    # one-hot rows of A select rows of W
    w = rand_bits(rng, (k, 7))
    sel = rng.integers(0, k, 5)
    a = np.zeros((5, k))
    a[np.arange(5), sel] = 1.0
    assert np.array_equal(impl.gemm_partial(bits(a), w), O.bf16_bits_to_f64(w)[sel])


def check_chunked_equals_unchunked(impl):
    rng = np.random.default_rng(6)
    tp, n_chunks, rows, k, n = 4, 8, 6, 64, 40
    shards = [rand_bits(rng, (rows, k)) for _ in range(tp)]
    w = rand_bits(rng, (k, n), 1 / 8)
    x, y = impl.agmm(shards, w)
    per = tp * rows // n_chunks
    ych = np.concatenate([impl.gemm_partial(x[c * per:(c + 1) * per], w) for c in range(n_chunks)])
    assert np.allclose(ych, y, rtol=1e-12, atol=0)


def check_tp_identity(impl):
    rng = np.random.default_rng(7)
    m, k, n, tp = 5, 48, 9, 4
    a = rand_bits(rng, (m, k))
    w = rand_bits(rng, (k, n), 0.2)
    s = k // tp
    parts = [impl.gemm_partial(a[:, q * s:(q + 1) * s], w[q * s:(q + 1) * s]) for q in range(tp)]
    assert np.allclose(sum(parts), impl.gemm_partial(a, w), rtol=1e-12, atol=1e-300)


def _int_bits(rng, shape, lo=-3, hi=4):
    """bf16 bits of small integers: sums of their products are exact in float64."""
    return bits(rng.integers(lo, hi, shape).astype(np.float64))


def check_backward_is_the_gradient(impl):
    """dX and dW are the derivatives of L = <dY, Y> with Y the forward agmm: with integer
    inputs, a unit step of one element of a shard (or of W) changes L by exactly that element
    of dX (or dW).  Pins the backward to the forward and to the definition of a gradient, not
    to a formula (a transposed or misplaced operand fails it)."""
    rng = np.random.default_rng(21)
    for tp, rows, k, n in ((2, 2, 3, 4), (3, 1, 4, 4), (2, 3, 5, 2)):
        shards = [_int_bits(rng, (rows, k)) for _ in range(tp)]
        w = _int_bits(rng, (k, n))
        dy = _int_bits(rng, (tp * rows, n))
        g = O.bf16_bits_to_f64(dy)
        x, dx, dw = impl.agmm_backward(shards, w, dy)
        assert np.array_equal(x, impl.agmm(shards, w)[0])
        loss = lambda sh, ww: float(np.sum(g * impl.agmm(sh, ww)[1]))  # noqa: E731
        base = loss(shards, w)
        for q in range(tp):
            for i in range(rows):
                for j in range(k):
                    v = O.bf16_bits_to_f64(shards[q]).copy()
                    v[i, j] += 1.0
                    step = [bits(v) if p == q else shards[p] for p in range(tp)]
                    assert loss(step, w) - base == dx[q * rows + i, j]
        for i in range(k):
            for j in range(n):
                v = O.bf16_bits_to_f64(w).copy()
                v[i, j] += 1.0
                assert loss(shards, bits(v)) - base == dw[i, j]


def check_backward_brute(impl):
    rng = np.random.default_rng(22)
    for tp, rows, k, n in ((2, 2, 3, 5), (4, 1, 2, 3)):
        shards = [rand_bits(rng, (rows, k)) for _ in range(tp)]
        w = rand_bits(rng, (k, n), 0.5)
        dy = rand_bits(rng, (tp * rows, n), 0.3)
        x, dx, dw = impl.agmm_backward(shards, w, dy)
        bx = brute.gather([brute.matrix(s) for s in shards])
        bw, bdy = brute.matrix(w), brute.matrix(dy)
        tr = lambda m: [list(r) for r in zip(*m)]  # noqa: E731
        f = lambda m: np.array([[float(v) for v in r] for r in m])  # noqa: E731
        assert np.allclose(dx, f(brute.matmul(bdy, tr(bw))), rtol=1e-13, atol=0)
        assert np.allclose(dw, f(brute.matmul(tr(bx), bdy)), rtol=1e-13, atol=0)


def check_backward_special(impl):
    rng = np.random.default_rng(23)
    k = 8
    shards = [rand_bits(rng, (3, k)) for _ in range(2)]
    dy = rand_bits(rng, (6, k))
    x, dx, dw = impl.agmm_backward(shards, bits(np.eye(k)), dy)
    assert np.array_equal(dx, O.bf16_bits_to_f64(dy))       # W = I: the gradient passes through
    one = np.zeros((6, 5))
    one[4, 2] = 1.0                                          # one token, one output feature
    x, dx, dw = impl.agmm_backward(shards, rand_bits(rng, (k, 5)), bits(one))
    want = np.zeros((k, 5))
    want[:, 2] = x[4]
    assert np.array_equal(dw, want)


def _balanced_layouts(n, tp):
    import itertools
    for cand in itertools.product(range(tp), repeat=n):
        if all(cand.count(d) == n // tp for d in range(tp)):
            yield np.array(cand)


def check_affinity_golden(impl):
    g = load_golden("affinity_worked_tp2.txt")
    a = g["affinity"]
    hd, nd = g["heads"][0].astype(int), g["neurons"][0].astype(int)
    assert impl.colocated_affinity(a, hd, nd) == g["score"][0, 0]
    best_nd = impl.balanced_neuron_assignment(a, hd, 2)
    assert np.bincount(best_nd, minlength=2).tolist() == [2, 2]
    assert impl.colocated_affinity(a, hd, best_nd) == g["best_neuron_score"][0, 0]
    best_hd = impl.best_head_layout(a, nd, 2)
    assert np.array_equal(best_hd, g["best_heads"][0].astype(int))
    assert impl.colocated_affinity(a, best_hd, nd) == g["best_head_score"][0, 0]


def check_balanced_assignment_brute(impl):
    """The neuron step against every balanced neuron layout of tiny instances."""
    rng = np.random.default_rng(31)
    for n_heads, n, tp in ((2, 6, 2), (3, 6, 3), (4, 8, 4), (2, 8, 2)):
        a = rng.standard_normal((n_heads, n))
        hd = np.arange(n_heads) % tp
        got = impl.balanced_neuron_assignment(a, hd, tp)
        assert np.bincount(got, minlength=tp).tolist() == [n // tp] * tp
        best = max(O.colocated_affinity(a, hd, nd) for nd in _balanced_layouts(n, tp))
        assert abs(impl.colocated_affinity(a, hd, got) - best) <= 1e-12 * (1 + abs(best))


def check_head_step_is_an_assignment(impl):
    """The head step is itself a balanced assignment of heads to device slots: its optimum must
    match an independent linear-assignment solve (scipy), at head counts past the tiny ones."""
    from scipy.optimize import linear_sum_assignment
    rng = np.random.default_rng(32)
    for n_heads, n, tp in ((8, 40, 4), (6, 30, 3), (8, 16, 2)):
        a = rng.standard_normal((n_heads, n))
        nd = np.arange(n) % tp
        got = impl.best_head_layout(a, nd, tp)
        assert np.bincount(got, minlength=tp).tolist() == [n_heads // tp] * tp
        t = np.stack([a[:, nd == d].sum(axis=1) for d in range(tp)], axis=1)
        slots = np.repeat(np.arange(tp), n_heads // tp)
        r, c = linear_sum_assignment(t[:, slots], maximize=True)
        assert abs(impl.colocated_affinity(a, got, nd) - t[:, slots][r, c].sum()) <= 1e-12 * (1 + abs(t).sum())


def check_affinity_planted(impl):
    """Planted groups (affinity 1 inside a group, 0 across): from the planted head layout the
    ascent reaches the planted layout, whose score (every same-group pair co-located) is the
    largest any layout can have."""
    rng = np.random.default_rng(33)
    n_heads, n, tp = 8, 64, 4
    gh = rng.permutation(np.arange(n_heads) % tp)
    gn = rng.permutation(np.arange(n) % tp)
    a = (gh[:, None] == gn[None, :]).astype(np.float64)
    hd, nd, score, rounds = impl.affinity_layout(a, tp, gh)
    assert score == a.sum()
    assert np.array_equal(nd, gn) and np.array_equal(hd, gh)


def check_affinity_ascent(impl):
    """The ascent ends at a layout that neither step improves, its score is the layout's, and it
    runs until a round brings nothing (this instance needs three rounds)."""
    rng = np.random.default_rng(11)
    a = rng.random((6, 24))
    hd, nd, score, rounds = impl.affinity_layout(a, 3, np.arange(6) // 2)
    assert rounds == 3
    assert score == O.colocated_affinity(a, hd, nd)
    assert O.colocated_affinity(a, hd, impl.balanced_neuron_assignment(a, hd, 3)) <= score + 1e-12
    assert O.colocated_affinity(a, impl.best_head_layout(a, nd, 3), nd) <= score + 1e-12
    # every round's score is at least the last one's
    h = np.arange(6) // 2
    last = -np.inf
    for _ in range(rounds):
        n_ = impl.balanced_neuron_assignment(a, h, 3)
        h = impl.best_head_layout(a, n_, 3)
        s_ = O.colocated_affinity(a, h, n_)
        assert s_ >= last
        last = s_


def check_layout_permutation(impl):
    rng = np.random.default_rng(34)
    lay = rng.permutation(np.arange(12) % 3)
    for group in (1, 4):
        p = impl.layout_permutation(lay, 3, group)
        assert np.array_equal(np.sort(p), np.arange(12 * group))           # a permutation
        blocks = p.reshape(3, -1)
        for d in range(3):                                                  # block d: device d's items
            items = blocks[d].reshape(-1, group)[:, 0] // group
            assert np.all(lay[items] == d) and np.all(np.diff(items) > 0)
            assert np.array_equal(blocks[d].reshape(-1, group), items[:, None] * group + np.arange(group))
    x = rng.standard_normal((5, 12))
    p = rng.permutation(12)
    inv = np.argsort(p)
    assert np.array_equal(impl.permute(impl.permute(x, p, 1), inv, 1), x)
    assert np.array_equal(impl.permute(x, p, 1), impl.permute(x.T, p, 0).T)
    assert np.array_equal(impl.permute(x, np.arange(5), 0), x)
    assert np.array_equal(impl.permute(x, p, 1)[:, 3], x[:, p[3]])


def check_rmsnorm_golden(impl):
    g = load_golden("rmsnorm_worked.txt")
    for case, nparts in (("a", 0), ("b", 2), ("c", 0)):
        parts = [bits(g[f"{case}.partial{p}"]) for p in range(nparts)]
        h, y = impl.reduce_residual_rmsnorm(parts, bits(g[f"{case}.residual"]),
                                            bits(g[f"{case}.gamma"][0]), float(g[f"{case}.eps"][0, 0]))
        assert np.array_equal(h, g[f"{case}.h"])
        assert np.allclose(y, g[f"{case}.y"], rtol=1e-15, atol=0)


def check_rmsnorm_closed_forms(impl):
    rng = np.random.default_rng(8)
    H = 64
    gamma = rand_bits(rng, (H,), 0.3)
    gv = O.bf16_bits_to_f64(gamma)
    for c in (0.5, -2.0, 3.0):
        y = impl.rmsnorm(np.full((1, H), c), gamma, 1e-6)
        assert np.allclose(y[0], c / math.sqrt(c * c + 1e-6) * gv, rtol=1e-15, atol=0)
    assert np.array_equal(impl.rmsnorm(np.zeros((2, H)), gamma, 1e-6), np.zeros((2, H)))
    h = O.bf16_bits_to_f64(rand_bits(rng, (4, H)))
    y1 = impl.rmsnorm(h, gamma, 0.0)
    for alpha in (0.125, 3.0, 1024.0):
        assert np.allclose(impl.rmsnorm(alpha * h, gamma, 0.0), y1, rtol=1e-14, atol=0)
    # with eps = 0 and gamma = 1 every row has mean square 1
    y = impl.rmsnorm(h, np.ones(H), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    # residual only (no partials) is the plain norm
    hh, yy = impl.reduce_residual_rmsnorm([], h, gamma, 1e-6)
    assert np.array_equal(hh, h) and np.array_equal(yy, impl.rmsnorm(h, gamma, 1e-6))


def check_rmsnorm_brute(impl):
    rng = np.random.default_rng(9)
    for rows, H, P in ((1, 3, 0), (2, 5, 2), (3, 8, 3)):
        res = rand_bits(rng, (rows, H))
        parts = [rand_bits(rng, (rows, H), 0.2) for _ in range(P)]
        gamma = rand_bits(rng, (H,), 0.5)
        eps = 1e-6
        h, y = impl.reduce_residual_rmsnorm(parts, res, gamma, eps)
        bh = brute.matrix(res)
        for p in parts:
            bh = brute.add(bh, brute.matrix(p))
        bg = [brute.bf16_value(v) for v in gamma.tolist()]
        assert np.array_equal(h, np.array([[float(v) for v in r] for r in bh]))
        by = np.array([brute.rmsnorm_row(r, bg, eps) for r in bh])
        assert np.allclose(y, by, rtol=1e-14, atol=1e-300)


def check_norm_commutes_with_gather(impl):
    rng = np.random.default_rng(10)
    H = 32
    shards = [rand_bits(rng, (3, H)) for _ in range(4)]
    gamma = rand_bits(rng, (H,), 0.3)
    lhs = impl.rmsnorm(impl.all_gather_sequence(shards), gamma, 1e-6)
    rhs = impl.all_gather_sequence([impl.rmsnorm(s, gamma, 1e-6) for s in shards])
    assert np.array_equal(lhs, rhs)


def check_reduce_uses_each_partial_once(impl):
    H = 4
    res = np.zeros((1, H))
    parts = [np.eye(H)[p:p + 1] * (p + 1) for p in range(H)]  # partial p = (p+1) e_p
    h, _ = impl.reduce_residual_rmsnorm(parts, res, np.ones(H), 1e-6)
    assert np.array_equal(h[0], np.arange(1, H + 1, dtype=np.float64))


def check_dtp_golden(impl):
    g = load_golden("dtp_worked_tp2_delta1.txt")
    owns = [g[f"own{l}"] for l in range(3)]
    peers = [[g[f"peer{l}"]] for l in range(3)]
    steps, xf, ximm = impl.dtp_sequence(g["x0"], owns, peers, int(g["delta"][0, 0]), np.ones(2), 0.0)
    assert len(steps) == 4
    for l in range(3):
        assert np.array_equal(steps[l][0], g[f"x_after{l}"])
        assert np.allclose(steps[l][1], g[f"y{l}"], rtol=1e-15, atol=0)
    assert steps[3][1] is None
    assert np.array_equal(xf, g["x_final"]) and np.array_equal(ximm, g["x_final"])


def check_dtp_invariants(impl):
    rng = np.random.default_rng(11)
    H, T, tp = 16, 3, 4
    gamma = rand_bits(rng, (H,), 0.2)
    for delta in (0, 1, 2, 3):
        for L in (1, 2, 5):
            x0 = rand_bits(rng, (T, H))
            owns = [rand_bits(rng, (T, H), 0.1) for _ in range(L)]
            peers = [[rand_bits(rng, (T, H), 0.1) for _ in range(tp - 1)] for _ in range(L)]
            steps, xf, ximm = impl.dtp_sequence(x0, owns, peers, delta, gamma, 1e-6)
            assert len(steps) == L + delta
            # every partial added exactly once: delayed == immediate after the flush
            assert np.allclose(xf, ximm, rtol=1e-12, atol=1e-12)
            # modules before delta see no peer partials
            x = O.bf16_bits_to_f64(x0)
            for l in range(min(delta, L)):
                x = x + O.bf16_bits_to_f64(owns[l])
                assert np.allclose(steps[l][0], x, rtol=1e-13, atol=1e-13)
            # delta = 0 is the reduce of [own, peers...] at every module
            if delta == 0:
                xr = x0
                for l in range(L):
                    h, y = impl.reduce_residual_rmsnorm([owns[l]] + peers[l], xr, gamma, 1e-6)
                    assert np.array_equal(steps[l][0], h) and np.array_equal(steps[l][1], y)
                    xr = h
            # module l's peers come from module l - delta
            if delta >= 1 and L >= 2:
                l = delta if delta < L else None
                if l is not None:
                    want = steps[l - 1][0] + O.bf16_bits_to_f64(owns[l]) + sum(
                        O.bf16_bits_to_f64(p) for p in peers[l - delta])
                    assert np.allclose(steps[l][0], want, rtol=1e-13, atol=1e-13)


def check_dtp_store_bf16(impl):
    rng = np.random.default_rng(12)
    H, T, tp, L, delta = 8, 2, 2, 3, 1
    x0 = rand_bits(rng, (T, H))
    owns = [rand_bits(rng, (T, H), 0.1) for _ in range(L)]
    peers = [[rand_bits(rng, (T, H), 0.1)] for _ in range(L)]
    steps, _, _ = impl.dtp_sequence(x0, owns, peers, delta, np.ones(H), 1e-6, store_bf16=True)
    x = O.bf16_bits_to_f64(x0)
    for l in range(L + delta):
        x = x + (O.bf16_bits_to_f64(owns[l]) if l < L else 0)
        if l >= delta:
            x = x + O.bf16_bits_to_f64(peers[l - delta][0])
        x = np.array([[float(brute.round_bf16(brute.Fraction(v))) for v in r] for r in x])
        assert np.array_equal(steps[l][0], x)


CHECKS = [check_bf16_decode, check_round_to_bf16, check_f64_to_bf16_bits, check_agmm_golden, check_agmm_brute,
          check_gemm_brute, check_special_weights, check_chunked_equals_unchunked,
          check_tp_identity, check_rmsnorm_golden, check_rmsnorm_closed_forms,
          check_rmsnorm_brute, check_norm_commutes_with_gather,
          check_reduce_uses_each_partial_once, check_dtp_golden, check_dtp_invariants,
          check_dtp_store_bf16, check_backward_is_the_gradient, check_backward_brute, check_backward_special,
          check_affinity_golden, check_balanced_assignment_brute, check_head_step_is_an_assignment,
          check_affinity_planted, check_affinity_ascent, check_layout_permutation]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)


# ----------------------------------------------------------------------------------------
# planted mistakes: each mutant must fail at least one pin
# ----------------------------------------------------------------------------------------

def _mutant(**overrides):
    m = types.SimpleNamespace(**{k: getattr(O, k) for k in O.__all__})
    for k, v in overrides.items():
        setattr(m, k, v)
    # rebind the composite functions to the mutated pieces
    base = m

    def reduce_residual_rmsnorm(partials, residual, gamma, eps):
        h = O._as_f64(residual).copy()
        for p in partials:
            h = h + O._as_f64(p)
        return h, base.rmsnorm(h, gamma, eps)

    def dtp_accumulate(residual, own, peers, gamma=None, eps=0.0):
        x, _ = O.dtp_accumulate(residual, own, peers, None, eps)
        return x, (None if gamma is None else base.rmsnorm(x, gamma, eps))

    if "reduce_residual_rmsnorm" not in overrides:
        m.reduce_residual_rmsnorm = reduce_residual_rmsnorm
    if "dtp_accumulate" not in overrides:
        m.dtp_accumulate = dtp_accumulate
    return m


def _rms_sum(h, gamma, eps):          # sum instead of mean
    hv = O._as_f64(h)
    return hv / np.sqrt(np.sum(hv * hv, -1, keepdims=True) + eps) * O._as_f64(gamma)


def _rms_eps_outside(h, gamma, eps):  # eps added after the square root
    hv = O._as_f64(h)
    return hv / (np.sqrt(np.mean(hv * hv, -1, keepdims=True)) + eps) * O._as_f64(gamma)


def _rms_no_gamma(h, gamma, eps):     # gain dropped
    hv = O._as_f64(h)
    return hv / np.sqrt(np.mean(hv * hv, -1, keepdims=True) + eps)


def _rms_over_rows(h, gamma, eps):    # reduction over the wrong axis
    hv = O._as_f64(h)
    return hv / np.sqrt(np.mean(hv * hv, 0, keepdims=True) + eps) * O._as_f64(gamma)


def _gather_reversed(shards):         # wrong rank order
    return np.concatenate([O._as_f64(s) for s in shards[::-1]], axis=0)


def _agmm_wT(shards, w):              # weight read with swapped indices
    x = O.all_gather_sequence(shards)
    wv = O._as_f64(w)
    if wv.shape[0] == wv.shape[1]:
        return x, x @ wv.T
    return x, x @ wv[:, ::-1]


def _agmm_rev(shards, w):
    x = _gather_reversed(shards)
    return x, x @ O._as_f64(w)


def _reduce_drop_last(partials, residual, gamma, eps):
    parts = list(partials)
    h = O._as_f64(residual).copy()
    for p in parts[:-1]:
        h = h + O._as_f64(p)
    return h, O.rmsnorm(h, gamma, eps)


def _reduce_minus(partials, residual, gamma, eps):
    h = O._as_f64(residual).copy()
    for i, p in enumerate(partials):
        h = h + (-1 if i == 1 else 1) * O._as_f64(p)
    return h, O.rmsnorm(h, gamma, eps)


def _dtp_seq_wrong_module(x0, owns, peers, delta, gamma, eps, store_bf16=False):
    # adds the peers of the current module instead of module l - delta
    L = len(owns)
    x = O._as_f64(x0).copy()
    steps = []
    for l in range(L + delta):
        own = owns[l] if l < L else None
        late = peers[l] if (l >= delta and l < L) else []
        x, y = O.dtp_accumulate(x, own, late, gamma if l < L else None, eps)
        steps.append((x, y))
    return steps, x, O.dtp_sequence(x0, owns, peers, delta, gamma, eps)[2]


def _dtp_seq_no_flush(x0, owns, peers, delta, gamma, eps, store_bf16=False):
    steps, _, ximm = O.dtp_sequence(x0, owns, peers, delta, gamma, eps, store_bf16)
    steps = steps[:len(owns)]
    return steps, steps[-1][0], ximm


def _decode_wrong_bias(b):
    return O.bf16_bits_to_f64(b) * 2.0


def _encode_via_binary32(x):        # rounds to binary32 first: a double rounding
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _round_trunc(x):
    v = O._as_f64(x)
    m, e = np.frexp(v)
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def _bwd_dx_untransposed(shards, w, dy):   # input gradient through W instead of W^T
    x = O.all_gather_sequence(shards)
    wv, g = O._as_f64(w), O._as_f64(dy)
    dx = g @ wv if wv.shape[0] == wv.shape[1] else g @ wv[::-1].T
    return x, dx, x.T @ g


def _bwd_dw_tokens_misaligned(shards, w, dy):  # weight gradient pairs the wrong tokens
    x = O.all_gather_sequence(shards)
    g = O._as_f64(dy)
    return x, g @ O._as_f64(w).T, x.T @ g[::-1]


def _bwd_gather_reversed(shards, w, dy):
    x = _gather_reversed(shards)
    g = O._as_f64(dy)
    return x, g @ O._as_f64(w).T, x.T @ g


def _affinity_cross(affinity, head_device, neuron_device):   # counts pairs on different devices
    a = np.asarray(affinity, dtype=np.float64)
    return float(np.sum(a * (np.asarray(head_device)[:, None] != np.asarray(neuron_device)[None, :])))


def _neurons_unbalanced(affinity, head_device, tp):   # each neuron to its best device, no capacity
    a = np.asarray(affinity, dtype=np.float64)
    hd = np.asarray(head_device)
    value = np.stack([a[hd == d].sum(axis=0) for d in range(tp)])
    return np.argmax(value, axis=0)


def _heads_not_searched(affinity, neuron_device, tp):   # keeps the contiguous head layout
    n_heads = np.asarray(affinity).shape[0]
    return np.arange(n_heads) // (n_heads // tp)


def _ascent_one_round(affinity, tp, head_device, max_rounds=100):
    return O.affinity_layout(affinity, tp, head_device, 1)


def _permutation_interleaved(layout, tp, group=1):     # items in index order, not grouped by device
    lay = np.asarray(layout)
    items = np.argsort(lay, kind="stable")[::-1]
    return (items[:, None] * group + np.arange(group)[None, :]).reshape(-1)


MUTANTS = {
    "rmsnorm_sum_not_mean": dict(rmsnorm=_rms_sum),
    "rmsnorm_eps_outside_sqrt": dict(rmsnorm=_rms_eps_outside),
    "rmsnorm_no_gamma": dict(rmsnorm=_rms_no_gamma),
    "rmsnorm_wrong_axis": dict(rmsnorm=_rms_over_rows),
    "gather_reversed": dict(all_gather_sequence=_gather_reversed, agmm=_agmm_rev),
    "agmm_transposed_weight": dict(agmm=_agmm_wT),
    "reduce_drops_last_partial": dict(reduce_residual_rmsnorm=_reduce_drop_last),
    "reduce_sign_flip": dict(reduce_residual_rmsnorm=_reduce_minus),
    "dtp_peers_of_wrong_module": dict(dtp_sequence=_dtp_seq_wrong_module),
    "dtp_missing_flush": dict(dtp_sequence=_dtp_seq_no_flush),
    "decode_wrong_exponent": dict(bf16_bits_to_f64=_decode_wrong_bias),
    "round_truncates": dict(round_to_bf16=_round_trunc),
    "encode_double_rounding": dict(f64_to_bf16_bits=_encode_via_binary32),
    "backward_dx_untransposed": dict(agmm_backward=_bwd_dx_untransposed),
    "backward_dw_tokens_misaligned": dict(agmm_backward=_bwd_dw_tokens_misaligned),
    "backward_gather_reversed": dict(agmm_backward=_bwd_gather_reversed),
    "affinity_counts_cross_device_pairs": dict(colocated_affinity=_affinity_cross),
    "neuron_step_ignores_balance": dict(balanced_neuron_assignment=_neurons_unbalanced),
    "head_step_does_not_search": dict(best_head_layout=_heads_not_searched),
    "ascent_stops_after_one_round": dict(affinity_layout=_ascent_one_round),
    "permutation_blocks_reversed": dict(layout_permutation=_permutation_interleaved),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    impl = _mutant(**MUTANTS[name])
    failed = []
    for check in CHECKS:
        try:
            check(impl)
        except AssertionError:
            failed.append(check.__name__)
        except Exception:  # a crash also counts as caught
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
