"""Pins for oracle.quantize: hand-worked golden blocks, grid round trips,
closed forms, invariants and exact-rational brute force."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as fm
from oracle import quantize as oq
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["mxfp4_block.json", "mxfp8_block.json"])
def test_golden_mx_block(name):
    g = _golden(name)
    x = np.array([g["values"]], dtype=np.float32)
    codes, scales = oq.quantize_mx(x, g["format"])
    assert codes[0].tolist() == g["codes"]
    assert scales.tolist() == [[g["scale_code"]]]
    if "scaled_copy" in g:
        sc = g["scaled_copy"]
        c2, s2 = oq.quantize_mx(x * np.float32(2.0 ** sc["factor_log2"]), g["format"])
        assert c2[0].tolist() == g["codes"] and s2.tolist() == [[sc["scale_code"]]]


def test_golden_nvfp4():
    g = _golden("nvfp4_tensor.json")
    x = np.array(g["rows"], dtype=np.float32)
    codes, s, t = oq.quantize_nvfp4(x)
    assert float(t) == g["tensor_scale"]
    assert s.tolist() == g["scale_codes"]
    assert codes.tolist() == g["codes"]


def test_golden_int4():
    g = _golden("int4_row.json")
    x = np.array([g["values"]], dtype=np.float32)
    codes, s = oq.quantize_int4(x)
    assert oq.int4_code_value(codes)[0].astype(int).tolist() == g["q"]
    assert [hex(v) for v in s.view(np.uint32)[0]] == g["scales_f32_hex"]


@pytest.mark.parametrize("fmt,top", [("MXFP4", [4.0, 6.0]), ("MXFP8", [256.0, 448.0, 320.0])])
def test_grid_roundtrip(fmt, top):
    elem = oq.ELEM[fmt]
    rng = np.random.default_rng(7)
    for t in top:
        for e in (-30, -3, 0, 5, 40):
            mags = rng.choice(elem.mags[elem.mags <= t], size=(4, 32))
            mags[:, 0] = t
            sign = rng.choice([-1.0, 1.0], size=mags.shape)
            x = (sign * mags * 2.0 ** e).astype(np.float32)
            codes, scales = oq.quantize_mx(x, fmt)
            assert np.all(scales == e + 127)
            assert np.array_equal(oq.dequantize_mx(codes, scales, fmt), x.astype(np.float64))


def test_all_zero_block_and_single_outlier():
    x = np.zeros((1, 64), np.float32)
    x[0, 33] = -0.0
    codes, scales = oq.quantize_mx(x, "MXFP4")
    assert scales.tolist() == [[0, 0]]
    assert codes[0, :33].tolist() == [0] * 33 and codes[0, 33] == 8
    for v, e in ((4.0, 3), (6.0, -9)):
        blk = np.zeros((1, 32), np.float32)
        blk[0, 5] = v * 2.0 ** e
        rest = np.arange(1, 32) % 3 - 1.0
        blk[0, np.arange(32) != 5] = rest * 2.0 ** (e - 2)      # |x| <= 2**(e-2): ties to 0
        codes, scales = oq.quantize_mx(blk, "MXFP4")
        assert scales[0, 0] == e + 127
        assert codes[0, 5] == (6 if v == 4.0 else 7)
        others = codes[0, np.arange(32) != 5]
        assert np.all((others & 7) == 0)


def test_mx_saturation():
    # amax * 2**-e in (6, 8) saturates to 6 for FP4; (448, 512) -> 448 for FP8
    x = np.array([[7.5] + [0.0] * 31], np.float32)
    codes, scales = oq.quantize_mx(x, "MXFP4")
    assert scales[0, 0] == 127 and codes[0, 0] == 7
    x = np.array([[500.0] + [0.0] * 31], np.float32)
    codes, scales = oq.quantize_mx(x, "MXFP8")
    assert scales[0, 0] == 127 and codes[0, 0] == 0x7E


def test_mx_scale_clamps():
    x = np.full((1, 32), 2.0 ** -149, np.float32)      # smallest subnormal
    codes, scales = oq.quantize_mx(x, "MXFP4")
    assert scales[0, 0] == 0 and np.all(codes == 0)    # e clamps at -127
    x = np.full((1, 32), 3.0e38, np.float32)
    codes, scales = oq.quantize_mx(x, "MXFP4")
    assert scales[0, 0] == 127 + 125 and np.all(codes == 7)


@pytest.mark.parametrize("fmt", ["MXFP4", "MXFP8"])
def test_mx_invariants(fmt):
    rng = np.random.default_rng(1)
    x = (rng.standard_t(3, size=(6, 96)) * 5).astype(np.float32)
    codes, scales = oq.quantize_mx(x, fmt)
    for k in (-7, 1, 12):
        c2, s2 = oq.quantize_mx(x * np.float32(2.0 ** k), fmt)
        assert np.array_equal(c2, codes) and np.array_equal(s2.astype(int), scales.astype(int) + k)
    sb = oq.ELEM[fmt].sign_bit
    c3, s3 = oq.quantize_mx(-x, fmt)
    assert np.array_equal(c3, codes ^ sb) and np.array_equal(s3, scales)
    perm = rng.permutation(32)
    c4, s4 = oq.quantize_mx(x.reshape(6, 3, 32)[:, :, perm].reshape(6, 96), fmt)
    assert np.array_equal(c4, codes.reshape(6, 3, 32)[:, :, perm].reshape(6, 96))
    # dequant(quant) is monotone within a block
    d = oq.dequantize_mx(codes, scales, fmt)
    order = np.argsort(x[0, :32], kind="stable")
    assert np.all(np.diff(d[0, :32][order]) >= 0)


@pytest.mark.parametrize("fmt", ["MXFP4", "MXFP8"])
def test_mx_against_exact(fmt):
    rng = np.random.default_rng(2)
    x = (rng.standard_t(3, size=(3, 64)) * 10.0 ** rng.integers(-5, 5, size=(3, 1))).astype(np.float32)
    x[1, 3] = -0.0
    codes, scales = oq.quantize_mx(x, fmt)
    grid = exact.e2m1_grid() if fmt == "MXFP4" else exact.e4m3_grid()
    emax = 2 if fmt == "MXFP4" else 8
    sb = 8 if fmt == "MXFP4" else 0x80
    for r in range(3):
        for b in range(2):
            c, s = exact.mx_block(x[r, 32 * b:32 * b + 32], grid, emax, sb)
            assert codes[r, 32 * b:32 * b + 32].tolist() == c and scales[r, b] == s


def _constructed_ties(rng, rows=4):
    """fp32 values placed exactly on E2M1 midpoints of NVFP4 block scales."""
    x = (rng.laplace(size=(rows, 32)) * 3).astype(np.float32)
    x[0, 0] = 2688.0                     # pins g = 1 for the whole tensor
    return x


def test_nvfp4_against_exact():
    rng = np.random.default_rng(4)
    x = _constructed_ties(rng)
    # block (row 1, block 0): amax 6 -> s = 1 -> midpoints are exact ties
    x[1, :16] = [6.0, 5.0, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, -5.0, -0.25, 0.0, -0.0, 1.0, 2.0, 3.0, 4.0]
    codes, s, g = oq.quantize_nvfp4(x)
    ec, es, eg = exact.nvfp4_tensor(x.tolist())
    assert Fraction(float(g)) == eg == 1
    assert s.tolist() == es and codes.tolist() == ec
    # random tensors, dynamic scale (g not a power of two)
    for seed in range(4):
        r = np.random.default_rng(100 + seed)
        x = (r.standard_t(3, size=(3, 48)) * 10.0 ** r.integers(-3, 4)).astype(np.float32)
        codes, s, g = oq.quantize_nvfp4(x)
        ec, es, eg = exact.nvfp4_tensor(x.tolist())
        assert Fraction(float(g)) == eg and s.tolist() == es and codes.tolist() == ec


def test_nvfp4_static_scale_and_zero():
    x = np.zeros((2, 16), np.float32)
    x[1, 2] = -0.0
    codes, s, g = oq.quantize_nvfp4(x)
    assert float(g) == 0.0 and np.all(s == 0) and codes[1, 2] == 8 and codes[0].sum() == 0
    # static g smaller than the data: block scale saturates at 448
    x = np.full((1, 16), 100.0, np.float32)
    codes, s, g = oq.quantize_nvfp4(x, tensor_scale=np.float32(0.01))
    assert s[0, 0] == 0x7E and np.all(codes == 7)


def test_nvfp4_tensor_constant():
    # a tensor whose amax is 2688 * 2**k has g = 2**k and its max block scale 448
    for k in (-12, 0, 9):
        x = np.zeros((1, 32), np.float32)
        x[0, 7] = 2688.0 * 2.0 ** k
        codes, s, g = oq.quantize_nvfp4(x)
        assert float(g) == 2.0 ** k and s[0, 0] == 0x7E and codes[0, 7] == 7
        assert oq.dequantize_nvfp4(codes, s, g)[0, 7] == x[0, 7]


def test_int4_against_exact():
    rng = np.random.default_rng(9)
    x = (rng.uniform(-1, 1, size=(3, 64)) * 10.0 ** rng.integers(-4, 4, size=(3, 1))).astype(np.float32)
    x[2, 0:3] = [7.0, 3.5, -2.5]
    x[2, 3:32] = 0.0
    codes, s = oq.quantize_int4(x)
    for r in range(3):
        q, sc = exact.int4_row(x[r].tolist())
        assert oq.int4_code_value(codes[r]).astype(int).tolist() == q
        assert [Fraction(float(v)) for v in s[r]] == sc


def test_storage_bits_closed_form():
    assert oq.storage_bits_per_element("MXFP4") == 4.25
    assert oq.storage_bits_per_element("MXFP8") == 8.25
    assert oq.storage_bits_per_element("NVFP4") == 4.5
    assert oq.storage_bits_per_element("INT4") == 5.0


def test_pack_low_nibble_first():
    codes = np.array([[1, 2, 3, 15]], np.uint8)
    assert oq.pack_nibbles(codes).tolist() == [[0x21, 0xF3]]
    assert np.array_equal(oq.unpack_nibbles(oq.pack_nibbles(codes)), codes)


def test_shape_errors():
    with pytest.raises(ValueError):
        oq.quantize_mx(np.zeros((1, 48), np.float32), "MXFP4")
    with pytest.raises(ValueError):
        oq.quantize_nvfp4(np.zeros((1, 24), np.float32))
    with pytest.raises(ValueError):
        oq.quantize_mx(np.array([[np.inf] + [0.0] * 31], np.float32), "MXFP8")
