"""Block quantizers: MXFP4, MXFP8, NVFP4 and INT4 (symmetric, per 32).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: MX formats share one power-of-two scale per small block
(Chameleon article, "the format is chosen by the value distribution": blocks
with a common exponent; the MR-GPTQ summary: MXFP4 scales are powers of two),
NVFP4 uses small groups (MR-GPTQ summary, first reason FP4 fails) with a
block scale and a tensor scale (the MSE-grid modification optimises "block
and tensor" scales), and INT4 is the uniform grid (MR-GPTQ summary, INT vs FP
grid paragraph).  Everything below that the pages leave open is read as:

* Blocks run along the reduction axis (K, contiguous): 32 elements for
  MXFP4, MXFP8 and INT4, 16 for NVFP4.  K must be a multiple of the block.
* MX scale: e = floor(log2(amax)) - emax_elem, clamped to [-127, 127],
  stored as E8M0 code e + 127.  amax = 0 gives code 0.  Elements are
  x / 2**e rounded to the element grid (exact real, RNE, saturating).
* NVFP4: tensor scale g = RN_fp32(A / (6 * 448)) with A the tensor's amax
  (A = 0 gives g = 0), or a caller-supplied g.  Block scale
  s = RN_E4M3(a_b / (6 g)) rounded once from the exact quotient, saturating
  at 448 (g = 0 gives s = 0).  Elements are x / (s g) rounded to E2M1 (s = 0
  gives signed zeros).
* INT4: scale s = RN_fp32(a_b / 7) stored as fp32; q = clamp(RNE(x / s), -7, 7)
  as a two's-complement nibble (a_b = 0 gives s = 0, q = 0).

Exactness of the float64 steps: for MX the division by 2**e is exact.  For
NVFP4 and INT4 the float64 quotient can only change a rounding decision if
the exact quotient lies within 2**-53 (relative) of a grid midpoint without
being on it; a float32 dividend over a divisor of at most 28 significant bits
cannot land that close (the gap is at least about 2**-32 relative), so
rounding the float64 quotient gives the same code as rounding the exact one.
The tests pin this against exact rational arithmetic.

Storage (used by the packing helpers): row-major, K contiguous.  4-bit codes
are packed two per byte, element 2i in the low nibble of byte i.  Scales are
row-major [rows][K / block]: uint8 E8M0 (MX), uint8 E4M3 (NVFP4) or float32
(INT4).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .formats import E2M1, E4M3, e8m0_decode, floor_log2, round_to_float32

MXFP4, MXFP8, NVFP4, INT4 = "MXFP4", "MXFP8", "NVFP4", "INT4"
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16, INT4: 32}
ELEM = {MXFP4: E2M1, MXFP8: E4M3, NVFP4: E2M1}
NVFP4_TENSOR_DIVISOR = 6 * 448          # E2M1 max times E4M3 max
INT4_QMAX = 7


def _blocks(x: np.ndarray, block: int) -> np.ndarray:
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array")
    rows, k = x.shape
    if k % block:
        raise ValueError(f"K={k} is not a multiple of the block size {block}")
    xb = x.astype(np.float64).reshape(rows, k // block, block)
    if not np.all(np.isfinite(xb)):
        raise ValueError("non-finite input is outside the contract")
    return xb


# ----------------------------------------------------------------------------
# MXFP4 / MXFP8: E8M0 power-of-two scale per 32 elements
# ----------------------------------------------------------------------------

def mx_scale_exponent(amax: np.ndarray, emax_elem: int) -> np.ndarray:
    """Shared exponent e = floor(log2 amax) - emax_elem, clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    pos = amax > 0
    e[pos] = floor_log2(amax[pos]) - emax_elem
    return np.clip(e, -127, 127)


def quantize_mx(x: np.ndarray, fmt: str):
    """MX quantization of a [rows, K] array.

    Returns (codes uint8 [rows, K] one code per element, scales uint8
    [rows, K/32] E8M0 codes).
    """
    elem = ELEM[fmt]
    xb = _blocks(x, 32)
    amax = np.abs(xb).max(axis=2)
    e = mx_scale_exponent(amax, elem.emax)
    v = xb / np.ldexp(1.0, e)[..., None]           # exact: power of two
    codes = elem.encode(v)
    rows, nb, _ = xb.shape
    return codes.reshape(rows, nb * 32), (e + 127).astype(np.uint8)


def dequantize_mx(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    elem = ELEM[fmt]
    rows, k = codes.shape
    vals = elem.decode(codes).reshape(rows, k // 32, 32)
    return (vals * e8m0_decode(scales)[..., None]).reshape(rows, k)


# ----------------------------------------------------------------------------
# NVFP4: E2M1 elements, E4M3 scale per 16, fp32 tensor scale
# ----------------------------------------------------------------------------

def nvfp4_tensor_scale(x: np.ndarray) -> np.float32:
    """g = RN_fp32(A / 2688), A = max |x| over the whole tensor (exact)."""
    xa = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(xa)):
        raise ValueError("non-finite input is outside the contract")
    amax = float(np.abs(xa).max()) if xa.size else 0.0
    return round_to_float32(Fraction(amax) / NVFP4_TENSOR_DIVISOR)


def quantize_nvfp4(x: np.ndarray, tensor_scale=None):
    """NVFP4 quantization of a [rows, K] array.

    Returns (codes uint8 [rows, K], block-scale E4M3 codes uint8 [rows, K/16],
    tensor scale g as float32).  ``tensor_scale`` None means dynamic (the
    tensor amax of ``x``).
    """
    xb = _blocks(x, 16)
    g = nvfp4_tensor_scale(x) if tensor_scale is None else np.float32(tensor_scale)
    g64 = float(g)
    amax = np.abs(xb).max(axis=2)
    if g64 == 0.0:
        s_codes = np.zeros(amax.shape, dtype=np.uint8)
    else:
        s_codes = E4M3.encode(amax / (6.0 * g64))   # 6*g exact in float64
    s_val = E4M3.decode(s_codes)
    d = s_val * g64                                   # exact: 4 x 24 significant bits
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(d[..., None] > 0, xb / d[..., None], 0.0 * xb)
    codes = E2M1.encode(v)
    rows, nb, _ = xb.shape
    return codes.reshape(rows, nb * 16), s_codes, g


def dequantize_nvfp4(codes, s_codes, g) -> np.ndarray:
    rows, k = codes.shape
    vals = E2M1.decode(codes).reshape(rows, k // 16, 16)
    return (vals * (E4M3.decode(s_codes) * float(g))[..., None]).reshape(rows, k)


# ----------------------------------------------------------------------------
# INT4 symmetric, fp32 scale per 32
# ----------------------------------------------------------------------------

def quantize_int4(x: np.ndarray):
    """INT4 quantization of a [rows, K] array.

    Returns (codes uint8 [rows, K] two's-complement nibbles 0..15,
    scales float32 [rows, K/32]).
    """
    xb = _blocks(x, 32)
    amax = np.abs(xb).max(axis=2)
    # amax / 7 rounded once to float32: the float64 quotient of a float32 by 7
    # rounds correctly to float32 (53 >= 2*24 + 2 bits)
    s = (amax / INT4_QMAX).astype(np.float32)
    s64 = s.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s64[..., None] > 0, np.rint(xb / s64[..., None]), 0.0)
    q = np.clip(q, -INT4_QMAX, INT4_QMAX).astype(np.int64)
    rows, nb, _ = xb.shape
    return (q & 0xF).astype(np.uint8).reshape(rows, nb * 32), s


def int4_code_value(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return np.where(c >= 8, c - 16, c).astype(np.float64)


def dequantize_int4(codes, scales) -> np.ndarray:
    rows, k = codes.shape
    vals = int4_code_value(codes).reshape(rows, k // 32, 32)
    return (vals * np.asarray(scales, dtype=np.float64)[..., None]).reshape(rows, k)


# ----------------------------------------------------------------------------
# Uniform front end, packing
# ----------------------------------------------------------------------------

def quantize(x: np.ndarray, fmt: str, tensor_scale=None) -> dict:
    """Quantize to ``fmt``; returns a dict with codes, scales (and g)."""
    if fmt in (MXFP4, MXFP8):
        codes, scales = quantize_mx(x, fmt)
        return {"fmt": fmt, "codes": codes, "scales": scales, "g": None}
    if fmt == NVFP4:
        codes, scales, g = quantize_nvfp4(x, tensor_scale)
        return {"fmt": fmt, "codes": codes, "scales": scales, "g": g}
    if fmt == INT4:
        codes, scales = quantize_int4(x)
        return {"fmt": fmt, "codes": codes, "scales": scales, "g": None}
    raise ValueError(f"unknown format {fmt}")


def dequantize(q: dict) -> np.ndarray:
    fmt = q["fmt"]
    if fmt in (MXFP4, MXFP8):
        return dequantize_mx(q["codes"], q["scales"], fmt)
    if fmt == NVFP4:
        return dequantize_nvfp4(q["codes"], q["scales"], q["g"])
    if fmt == INT4:
        return dequantize_int4(q["codes"], q["scales"])
    raise ValueError(f"unknown format {fmt}")


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, K] 4-bit codes -> [rows, K/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def storage_bits_per_element(fmt: str) -> float:
    """Bits of codes plus block scales per element (tensor scale excluded)."""
    elem_bits = 8 if fmt == MXFP8 else 4
    scale_bits = 32 if fmt == INT4 else 8
    return elem_bits + scale_bits / BLOCK[fmt]
