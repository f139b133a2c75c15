"""Pins for oracle.select: rows exactly representable in one format are
chosen with zero error, constructed ties go to the earliest candidate, the
permutation is a stable grouping, and SSE matches exact rationals."""
from fractions import Fraction

import numpy as np

from oracle import quantize as oq
from oracle import select as osel


def test_exactly_representable_rows():
    rng = np.random.default_rng(0)
    k = 64
    # INT4-exact row: integers -7..7 times an fp32 scale with amax 7 in every block
    q = rng.integers(-7, 8, size=k).astype(np.float64)
    q[0], q[32] = 7, -7
    # scale 1.25 * 2**-7: 7 * scale and every q * scale are exact in fp32,
    # so RN_fp32(amax / 7) recovers the scale exactly
    int4_row = (q * (1.25 * 2.0 ** -7)).astype(np.float32)
    # MXFP4-exact row: grid values times 2**-8, a 6 in each block; make it
    # non-representable by NVFP4 by using a different power per 16-block
    g = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mx = rng.choice(g, size=k) * rng.choice([-1, 1], size=k)
    mx[0] = mx[32] = 6.0
    mx_row = (mx * 2.0 ** -8).astype(np.float32)
    w = np.stack([int4_row, mx_row])
    choice, sse, perm = osel.select_formats(w)
    qi = oq.quantize(int4_row[None], "INT4")
    assert np.array_equal(oq.dequantize(qi)[0], int4_row.astype(np.float64))
    assert sse[0, 0] == 0.0 and choice[0] == 0
    assert sse[1, 1] == 0.0 and choice[1] in (0, 1)
    assert choice[1] == (0 if sse[1, 0] == 0.0 else 1)


def test_ties_go_to_earliest_and_perm_is_stable():
    # an all-zero row reconstructs exactly in every format: tie -> INT4 (index 0)
    w = np.zeros((5, 32), np.float32)
    rng = np.random.default_rng(1)
    w[1] = rng.standard_t(2, size=32).astype(np.float32)
    w[3] = rng.uniform(-1, 1, size=32).astype(np.float32)
    choice, sse, perm = osel.select_formats(w)
    for r in (0, 2, 4):
        assert np.all(sse[r] == 0) and choice[r] == 0
    assert sorted(perm.tolist()) == list(range(5))
    groups = [choice[p] for p in perm]
    assert groups == sorted(groups)
    for c in set(choice.tolist()):
        rows = [p for p in perm if choice[p] == c]
        assert rows == sorted(rows)
    # candidate order decides the tie
    c2, _, _ = osel.select_formats(w, ("NVFP4", "MXFP4", "INT4"))
    assert c2[0] == 0


def test_sse_exact_rational():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((3, 32)) * 0.02).astype(np.float32)
    sse = osel.row_sse(w)
    g = oq.nvfp4_tensor_scale(w)
    for j, fmt in enumerate(osel.PALETTE):
        d = oq.dequantize(oq.quantize(w, fmt, tensor_scale=g if fmt == "NVFP4" else None))
        for r in range(3):
            ex = sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(w[r], d[r]))
            assert abs(Fraction(float(sse[r, j])) - ex) <= ex * Fraction(1, 2 ** 45)


def test_distribution_sanity():
    """Not a pin: uniform rows favour the uniform grid, heavy tails favour FP4."""
    rng = np.random.default_rng(3)
    uni = rng.uniform(-1, 1, size=(20, 256)).astype(np.float32)
    heavy = rng.standard_t(2, size=(20, 256)).astype(np.float32)
    cu, _, _ = osel.select_formats(uni)
    ch, _, _ = osel.select_formats(heavy)
    assert np.mean(cu == 0) > 0.5
    assert np.mean(ch != 0) > 0.5
