"""Pins for oracle.hadamard: integer identities, a library routine
(scipy.linalg.hadamard), norm preservation, involution and exact sums."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import hadamard as oh


@pytest.mark.parametrize("n", [1, 2, 4, 16, 32, 128])
def test_sylvester_identities(n):
    h = oh.sylvester(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(h, h.T)
    assert np.all(np.abs(h) == 1) and np.all(h[0] == 1) and np.all(h[:, 0] == 1)


def test_matches_scipy():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    for n in oh.SIZES:
        assert np.array_equal(oh.sylvester(n), scipy_linalg.hadamard(n))
    assert oh.sylvester(2).tolist() == [[1, 1], [1, -1]]


def test_scale_factor_is_nearest():
    for n in (16, 32, 128, 2, 8):
        c = oh.scale_factor(n)
        # c is within half an ulp of 1/sqrt(n): check c**2 * n against 1
        exact = Fraction(c) ** 2 * n
        ulp = Fraction(np.spacing(c))
        lo, hi = (Fraction(c) - ulp / 2) ** 2 * n, (Fraction(c) + ulp / 2) ** 2 * n
        assert lo <= 1 <= hi
    assert oh.scale_factor(16) == 0.25


@pytest.mark.parametrize("n", oh.SIZES)
def test_unit_vectors_and_norm(n):
    x = np.zeros((n, 2 * n), np.float32)
    for j in range(n):
        x[j, n + j] = 1.0
    r = oh.rotate(x, n)
    c = np.float32(oh.scale_factor(n))
    assert np.all(r[:, :n] == 0)
    assert np.array_equal(np.abs(r[:, n:]), np.full((n, n), c, np.float32))
    assert np.array_equal(np.sign(r[:, n:]), oh.sylvester(n).astype(np.float32))
    rng = np.random.default_rng(0)
    y = rng.standard_normal((8, 4 * n)).astype(np.float32)
    ry = oh.rotate(y, n)
    for b in range(4):
        nb = np.linalg.norm(y[:, b * n:(b + 1) * n].astype(np.float64), axis=1)
        nr = np.linalg.norm(ry[:, b * n:(b + 1) * n].astype(np.float64), axis=1)
        assert np.allclose(nr, nb, rtol=1e-6)
    # rotating twice is the identity up to the two float32 roundings
    assert np.allclose(oh.rotate(ry, n), y, rtol=0, atol=1e-5 * np.abs(y).max())


def test_n16_single_rounding_exact():
    rng = np.random.default_rng(1)
    x = (rng.laplace(size=(4, 32)) * 100).astype(np.float32)
    r = oh.rotate(x, 16)
    h = oh.sylvester(16)
    for i in range(4):
        for b in range(2):
            blk = [Fraction(float(v)) for v in x[i, 16 * b:16 * b + 16]]
            for j in range(16):
                s = sum(blk[t] * int(h[t, j]) for t in range(16)) / 4
                assert r[i, 16 * b + j] == np.float32(float(s)) or \
                    Fraction(float(r[i, 16 * b + j])) == Fraction(float(np.float32(s)))


def test_exactness_guard():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 1.0e20
    x[0, 1] = 1.0e-20
    with pytest.raises(ValueError):
        oh.rotate(x, 16)
    # the same range with bf16-width mantissas is exact
    x2 = np.zeros((1, 16), np.float32)
    x2[0, 0], x2[0, 1] = 2.0 ** 20, 2.0 ** -10
    oh.rotate(x2, 16, mant_bits=7)


def test_shape_errors():
    with pytest.raises(ValueError):
        oh.rotate(np.zeros((1, 24), np.float32), 16)
    with pytest.raises(ValueError):
        oh.rotate(np.zeros((1, 64), np.float32), 64)


def test_zero_sum_is_positive_zero():
    # signed zeros and cancelling pairs: every exact-zero output is +0
    x = np.zeros((2, 16), np.float32)
    x[0, 1::2] = -0.0
    x[1, 0], x[1, 1] = 3.0, 3.0          # outputs j with H[0,j] = -H[1,j] cancel
    r = oh.rotate(x, 16)
    zeros = r == 0
    assert zeros.sum() == 16 + 8
    assert not np.signbit(r[zeros]).any()
    # an underflowing nonzero sum keeps its sign
    t = np.zeros((1, 16), np.float32)
    t[0, 0] = -2.0 ** -149
    r = oh.rotate(t, 16)
    assert np.all(r == 0) and np.all(np.signbit(r[0, :]) == (oh.sylvester(16)[0] > 0))


def _nearest_double_inv_sqrt(n):
    """The float64 nearest to 1/sqrt(n), decided with exact rationals: of two
    adjacent doubles c1 < 1/sqrt(n) < c2, c1 is nearer iff n * mid**2 > 1."""
    c = float(1.0 / math.sqrt(n))
    lo, hi = np.nextafter(c, 0.0), np.nextafter(c, 1.0)
    cands = sorted({float(lo), c, float(hi)})
    below = [v for v in cands if Fraction(v) ** 2 * n < 1]
    above = [v for v in cands if Fraction(v) ** 2 * n > 1]
    c1, c2 = max(below), min(above)
    mid = (Fraction(c1) + Fraction(c2)) / 2
    return c1 if mid ** 2 * n > 1 else c2


def _exact_rotation(row, n):
    """r = RN32(RN64(c_n * S)) of one row with S summed in exact rationals;
    float(Fraction) and the float64 -> float32 cast both round to nearest even."""
    h = oh.sylvester(n)
    c = Fraction(_nearest_double_inv_sqrt(n))
    out = []
    for b in range(0, len(row), n):
        blk = [Fraction(float(v)) for v in row[b:b + n]]
        for j in range(n):
            s = sum(blk[t] * int(h[t, j]) for t in range(n))
            out.append(np.float32(0.0) if s == 0 else np.float32(float(c * s)))
    return np.array(out, dtype=np.float32)


def _wide_blocks(n, dtype):
    """Rows whose block sums need more than 24 significant bits: values with
    exponents spread over 2**-16 .. 2**14 (bf16) or 2**0 .. 2**18 (fp32, so
    the float64 sum stays exact), random signs, plus single-outlier blocks."""
    rng = np.random.default_rng(7 + n)
    rows = 6
    span = (-16, 14) if dtype == "bf16" else (0, 18)
    e = rng.integers(span[0], span[1], size=(rows, 2 * n))
    m = 1.0 + rng.random((rows, 2 * n))
    x = (np.where(rng.random((rows, 2 * n)) < 0.5, -1.0, 1.0) * m * 2.0 ** e).astype(np.float32)
    x[0, :n] = 0.0
    x[0, 3] = 2.0 ** span[1]                 # one outlier in an otherwise zero block
    x[1, n:] = 1.0 + 2.0 ** -7               # equal values: only column 0 is nonzero
    if dtype == "bf16":
        from fp8_quantized_linear_mxq_amd.workloads import bf16_to_f32, f32_to_bf16_bits
        x = bf16_to_f32(f32_to_bf16_bits(x))
    return x


@pytest.mark.parametrize("n", [32, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_n32_n128_single_rounding_exact(n, dtype):
    x = _wide_blocks(n, dtype)
    r = oh.rotate(x, n, 7 if dtype == "bf16" else 23)
    bits = []
    for i in range(x.shape[0]):
        want = _exact_rotation(x[i], n)
        assert np.array_equal(r[i].view(np.uint32), want.view(np.uint32)), (n, dtype, i)
        h = oh.sylvester(n)
        for b in range(0, x.shape[1], n):
            for j in range(n):
                s = sum(Fraction(float(v)) * int(h[t, j]) for t, v in enumerate(x[i, b:b + n]))
                if s:
                    bits.append(abs(s).numerator.bit_length())
    # the fixture exercises sums wider than a float32 significand
    assert max(bits) > 24 and np.mean(np.array(bits) > 24) > 0.5


def test_n32_n128_pins_catch_plausible_slips(monkeypatch):
    """Each slip changes at least one output of the exact pins' fixture:
    S rounded to float32 before the multiply, a float32 c_n, and c_n taken
    from the wrong power of two."""
    for n in (32, 128):
        x = _wide_blocks(n, "bf16")
        want = np.stack([_exact_rotation(row, n) for row in x])
        xb = x.astype(np.float64).reshape(x.shape[0], -1, n)
        s = xb @ oh.sylvester(n).astype(np.float64)
        c = oh.scale_factor(n)
        slips = {
            "S rounded to float32": (c * s.astype(np.float32).astype(np.float64)),
            "float32 c_n": (np.float64(np.float32(c)) * s),
            "c_n of 2n": (oh.scale_factor(2 * n if 2 * n in (32, 128) else n // 2) * s),
        }
        for name, v in slips.items():
            got = v.astype(np.float32).reshape(x.shape)
            assert not np.array_equal(got.view(np.uint32), want.view(np.uint32)), (n, name)
        # and the oracle itself is not one of them
        assert np.array_equal(oh.rotate(x, n, 7).view(np.uint32), want.view(np.uint32))
