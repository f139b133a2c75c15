"""Element and scale formats: E2M1 (FP4), E4M3 (FP8), E8M0 (power-of-two scale).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats -- 4-bit floats supported in hardware by NVIDIA and
AMD, MXFP4 with power-of-two scales, NVFP4 with small groups, FP8 (the
"Bridging the Gap ... Microscaling FP4" summary, the two reasons FP4 fails;
the Chameleon article, "hardware support" paragraph) -- but print no bit
layouts.  The layouts used here are the public OCP microscaling / OCP FP8
definitions, written out from their field meaning:

  E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
        Exponent field 0 is subnormal: value = m * 0.5.  No Inf, no NaN.
  E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
        Exponent field 0 is subnormal: value = m/8 * 2**-6.  S.1111.111 is
        NaN; there is no Inf, so the largest finite magnitude is 448.
  E8M0: unsigned exponent, value = 2**(c - 127); c = 255 is NaN.

Rounding reading (the pages are silent): an exact real value is rounded to
the nearest representable magnitude, ties to the code whose mantissa LSB is
0 ("even"), magnitudes above the largest finite value saturate to it, and the
sign bit is the sign of the input (so -0.0 and small negatives give the
negative-zero code).
"""

from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Decode one E2M1 code (0..15) from its bit fields."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return sign * mag


def e4m3_value(code: int) -> float:
    """Decode one E4M3 code (0..255) from its bit fields (NaN for S.1111.111)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = 2.0 ** (exp - 7) * (1.0 + man / 8.0)
    return sign * mag


def e8m0_value(code: int) -> float:
    """Decode one E8M0 scale code; 255 is NaN."""
    if code == 255:
        return float("nan")
    return 2.0 ** (code - 127)


class ElemFormat:
    """A sign-magnitude element format given by its decoder.

    ``mags[c]`` is the magnitude of positive code ``c`` for c = 0..top; the
    codes are monotone in magnitude, so the mantissa LSB of a code is the
    code's own LSB, which is what ties-to-even looks at.
    """

    def __init__(self, name: str, decode, sign_bit: int, top_code: int,
                 emax: int):
        self.name = name
        self.sign_bit = sign_bit
        self.mags = np.array([decode(c) for c in range(top_code + 1)],
                             dtype=np.float64)
        assert np.all(np.diff(self.mags) > 0)
        self.max = float(self.mags[-1])
        # exponent of the largest power of two <= max (OCP "emax_elem")
        self.emax = emax
        self.table = np.array([decode(c) for c in range(2 * sign_bit)],
                              dtype=np.float64)

    def encode(self, v) -> np.ndarray:
        """Round exact real values ``v`` (float64 array) to codes (uint8).

        Nearest magnitude, ties to the even code, saturating at ``max``;
        the sign bit copies the sign of ``v`` (including -0.0).
        """
        v = np.asarray(v, dtype=np.float64)
        if not np.all(np.isfinite(v)):
            raise ValueError("non-finite input is outside the contract")
        a = np.abs(v)
        mids = (self.mags[:-1] + self.mags[1:]) / 2.0   # exact in float64
        idx = np.searchsorted(mids, a, side="left")      # midpoints strictly below a
        on_mid = np.zeros(a.shape, dtype=bool)
        inside = idx < mids.size
        on_mid[inside] = a[inside] == mids[idx[inside]]
        # a tie sits between codes idx and idx+1: keep whichever is even
        idx = np.where(on_mid & (idx % 2 == 1), idx + 1, idx)
        code = idx.astype(np.int64)
        code |= np.where(np.signbit(v), self.sign_bit, 0)
        return code.astype(np.uint8)

    def decode(self, codes) -> np.ndarray:
        return self.table[np.asarray(codes, dtype=np.int64)]


E2M1 = ElemFormat("E2M1", e2m1_value, sign_bit=0x8, top_code=0x7, emax=2)
E4M3 = ElemFormat("E4M3", e4m3_value, sign_bit=0x80, top_code=0x7E, emax=8)


def e8m0_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    if np.any(codes == 255):
        raise ValueError("E8M0 NaN code")
    return np.ldexp(1.0, codes - 127)


def floor_log2(a) -> np.ndarray:
    """Exact floor(log2(a)) for positive finite float64 values (via frexp)."""
    _, ex = np.frexp(np.asarray(a, dtype=np.float64))
    return ex.astype(np.int64) - 1


def round_to_float32(q) -> np.float32:
    """Correctly rounded (nearest-even) float32 of an exact rational.

    ``q`` is a ``fractions.Fraction`` (or int); used for the few scalar
    quantities the rules define as "rounded once to fp32".
    """
    from fractions import Fraction
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum_exp = max(e, -126) - 23
    n = a / Fraction(2) ** quantum_exp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = float(fl) * 2.0 ** quantum_exp
    if val > float(np.finfo(np.float32).max):
        return np.float32(sign * np.inf)
    return np.float32(sign * val)


def round_to_bf16(y) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 has 8 significant bits and the float32 exponent range
    (subnormal quantum 2**-133).  Overflow goes to +-inf.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    nz = y != 0
    a = np.abs(y[nz])
    e = np.maximum(floor_log2(a), -126)
    quantum = np.ldexp(1.0, e - 7)
    r = np.rint(a / quantum) * quantum          # rint is round-half-even
    r = np.where(r > 3.3895313892515355e38, np.inf, r)
    out[nz] = np.copysign(r, y[nz])
    out[~nz] = y[~nz]                           # keeps -0.0
    return out
