"""Pins for oracle.formats: closed forms, exhaustive round trips, midpoints,
library routines (numpy float32, torch bfloat16) and exact rationals."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as fm
from tests import exact


def test_e2m1_closed_form():
    mags = [fm.e2m1_value(c) for c in range(8)]
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [fm.e2m1_value(c | 8) for c in range(8)] == [-m for m in mags]
    assert fm.E2M1.max == 6.0 and fm.E2M1.emax == 2
    assert [Fraction(m) for m in mags] == exact.e2m1_grid()


def test_e4m3_closed_form():
    finite = [fm.e4m3_value(c) for c in range(0x7F)]
    assert fm.e4m3_value(0x7F) != fm.e4m3_value(0x7F)          # NaN
    assert fm.e4m3_value(0xFF) != fm.e4m3_value(0xFF)
    pos = [v for v in finite if v > 0]
    assert len(pos) == 126
    assert max(pos) == 448.0 and min(pos) == 2.0 ** -9
    assert fm.e4m3_value(0x7E) == 448.0 and fm.e4m3_value(0x08) == 2.0 ** -6
    assert [Fraction(v) for v in finite] == exact.e4m3_grid()
    assert fm.E4M3.emax == 8


def test_e8m0():
    assert fm.e8m0_value(127) == 1.0
    assert fm.e8m0_value(0) == 2.0 ** -127 and fm.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(fm.e8m0_value(255))


@pytest.mark.parametrize("elem,ncodes", [(fm.E2M1, 16), (fm.E4M3, 256)])
def test_roundtrip_every_code(elem, ncodes):
    codes = np.array([c for c in range(ncodes)
                      if not (elem is fm.E4M3 and (c & 0x7F) == 0x7F)])
    vals = elem.decode(codes)
    # -0.0 must come back as the negative-zero code
    back = elem.encode(vals)
    assert np.array_equal(back, codes.astype(np.uint8))


@pytest.mark.parametrize("elem", [fm.E2M1, fm.E4M3])
def test_midpoints_tie_to_even_and_neighbours(elem):
    grid = exact.e2m1_grid() if elem is fm.E2M1 else exact.e4m3_grid()
    for i in range(len(grid) - 1):
        mid = (grid[i] + grid[i + 1]) / 2
        want = i if i % 2 == 0 else i + 1
        m = float(mid)
        assert elem.encode(np.array([m]))[0] == want
        assert elem.encode(np.array([-m]))[0] == want | elem.sign_bit
        lo, hi = np.nextafter(m, 0.0), np.nextafter(m, np.inf)
        assert elem.encode(np.array([lo]))[0] == i
        assert elem.encode(np.array([hi]))[0] == i + 1


def test_e2m1_midpoint_list():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 1e30])
    assert fm.E2M1.encode(v).tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 7]


def test_saturation_and_signed_zero():
    assert fm.E4M3.encode(np.array([460.0, 464.0, 1e9, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert fm.E2M1.encode(np.array([-0.0, -0.1, 0.0])).tolist() == [8, 8, 0]
    with pytest.raises(ValueError):
        fm.E2M1.encode(np.array([np.nan]))


def test_random_against_exact():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(400) * 3, rng.standard_normal(400) * 100,
                        rng.standard_normal(200) * 0.01])
    for elem, grid in ((fm.E2M1, exact.e2m1_grid()), (fm.E4M3, exact.e4m3_grid())):
        got = elem.encode(v)
        want = [exact.round_to_grid(Fraction(float(x)), grid) | (elem.sign_bit if x < 0 else 0)
                for x in v]
        assert got.tolist() == want


def test_round_to_float32_matches_numpy():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, 300),
                         [1 / 3, 2 / 3, 1e-45, 3e-39]])
    for x in xs:
        # numpy's float64 -> float32 cast is round-to-nearest-even
        assert fm.round_to_float32(Fraction(float(x))) == np.float32(x)
    assert fm.round_to_float32(Fraction(1, 3)) == np.float32(1 / 3)


def test_round_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    x = np.concatenate([x, np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 0.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = fm.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.signbit(got[-2])


def test_floor_log2_exact():
    for k in range(-140, 128):
        a = 2.0 ** k
        assert fm.floor_log2(np.array([a]))[0] == k
        assert fm.floor_log2(np.array([np.nextafter(a, 0.0)]))[0] == k - 1
