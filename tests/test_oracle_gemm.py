"""Pins for oracle.gemm: exact-rational dot products on tiny shapes,
identity/permutation weights, the low-rank branch reducing to the plain
layer, and exactly representable grid operands."""
from fractions import Fraction

import numpy as np

from oracle import gemm as og
from oracle import quantize as oq


def _exact_linear(a, w, alpha, u, l2):
    m, k = a.shape
    n = w.shape[0]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            s = sum(Fraction(float(a[i, t])) * Fraction(float(w[j, t])) for t in range(k))
            s *= Fraction(float(alpha))
            if u is not None:
                s += sum(Fraction(float(u[i, t])) * Fraction(float(l2[t, j]))
                         for t in range(u.shape[1]))
            out[i, j] = s
    return out


def test_tiny_against_fractions():
    rng = np.random.default_rng(0)
    for (m, n, k, r) in ((3, 5, 64, 0), (8, 8, 256, 4), (1, 2, 32, 2)):
        a = oq.dequantize(oq.quantize(rng.standard_t(3, size=(m, k)).astype(np.float32), "MXFP4"))
        w = oq.dequantize(oq.quantize(rng.normal(0, .02, size=(n, k)).astype(np.float32), "MXFP4"))
        u = rng.standard_normal((m, r)) if r else None
        l2 = rng.standard_normal((r, n)) if r else None
        alpha = 0.75
        y = og.linear(a, w, alpha, u, l2)
        ex = _exact_linear(a, w, alpha, u, l2)
        s = og.abs_sum_bound(a, w, alpha) + (np.abs(u) @ np.abs(l2) if r else 0)
        err = np.abs(y - ex.astype(np.float64))
        assert np.all(err <= 1e-12 * s + 1e-300)


def test_identity_and_permutation_weights():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((4, 32))
    assert np.array_equal(og.linear(a, np.eye(32)), a)
    p = rng.permutation(32)
    assert np.array_equal(og.linear(a, np.eye(32)[p]), a[:, p])


def test_lowrank_zero_reduces_to_plain():
    rng = np.random.default_rng(2)
    a, w = rng.standard_normal((3, 64)), rng.standard_normal((5, 64))
    x, l1 = rng.standard_normal((3, 64)), rng.standard_normal((64, 4))
    u = og.lowrank_down(x, l1)
    assert np.array_equal(og.linear(a, w, 1.0, u, np.zeros((4, 5))), og.linear(a, w))
    assert np.allclose(u, x @ l1)


def test_grid_operands_exact_then_bf16():
    # small integers times powers of two: every partial sum is exact in fp32,
    # so the result equals its bf16 rounding of an exact integer
    a = np.array([[1.0, 2.0, -3.0, 0.5] * 8], np.float64)
    w = np.array([[4.0, -1.0, 1.5, 2.0] * 8, [0.5, 0.5, 0.5, 0.5] * 8])
    y = og.linear(a, w)
    assert y.tolist() == [[8 * (4 - 2 - 4.5 + 1), 8 * (0.5 + 1 - 1.5 + 0.25)]]
    assert og.linear_bf16(np.array([[1.0]]), np.array([[1.0 + 2 ** -8]]))[0, 0] == 1.0
    assert og.linear_bf16(np.array([[1.0]]), np.array([[1.0 + 3 * 2 ** -8]]))[0, 0] == 1.0 + 2 ** -6


def test_tolerance_form():
    y = np.array([[2.0]])
    s = np.array([[10.0]])
    assert og.tolerance(y, s)[0, 0] == 1e-5 * (1 + 2 ** -8) * 10.0 + 2 ** -8 * 2.0 + 2 ** -133


def test_tolerance_covers_bf16_subnormal_rounding():
    # rounding a tiny exact value to bfloat16 (subnormal below 2**-126, quantum
    # 2**-133) errs by up to half a quantum; the tolerance's floor covers it
    ys = np.array([[k * 2.0 ** -141 for k in range(1, 400, 7)] + [2.0 ** -134, 3 * 2.0 ** -134]])
    err = np.abs(og.round_to_bf16(ys) - ys)
    assert err.max() == 2.0 ** -134            # the ties: half a quantum
    assert np.all(err <= og.tolerance(ys, np.zeros_like(ys)))
    # a normal value's rounding stays within 2**-8 |y|
    y = np.array([[1.0 + 2 ** -8]])
    assert abs(og.round_to_bf16(y) - y)[0, 0] <= 2 ** -8 * y[0, 0]


def test_lowrank_terms_against_exact_rationals():
    """u = x L1 and y = a w^T + u L2 + bias on dyadic inputs, against sums of
    Fractions written out element by element (every float64 partial sum is
    exact here, so the oracle must match to the bit); a transposed operand or
    a dropped term fails."""
    from fractions import Fraction as F
    rng = np.random.default_rng(9)
    m, k, r, n = 3, 8, 2, 4
    dy = lambda *s: rng.integers(-8, 9, size=s) * 2.0 ** rng.integers(-4, 4, size=s)
    x, l1, a, w, l2, b = dy(m, k), dy(k, r), dy(m, k), dy(n, k), dy(r, n), dy(n)
    u = og.lowrank_down(x, l1)
    for i in range(m):
        for j in range(r):
            assert u[i, j] == float(sum(F(x[i, t]) * F(l1[t, j]) for t in range(k)))
    y = og.linear(a, w, 1.0, u, l2, b)
    for i in range(m):
        for j in range(n):
            want = (sum(F(a[i, t]) * F(w[j, t]) for t in range(k))
                    + sum(F(u[i, q]) * F(l2[q, j]) for q in range(r)) + F(b[j]))
            assert y[i, j] == float(want)
    # planted slips: L2 used transposed-by-index, or the bias dropped
    assert not np.array_equal(og.linear(a, w, 1.0, u, l2, b), og.linear(a, w, 1.0, u, l2))
    assert not np.array_equal(y, og.linear(a, w, 1.0, u, l2[::-1], b))
