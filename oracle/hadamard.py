"""Block-diagonal Hadamard rotation of activations (and, offline, weights).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the "Bridging the Gap ... Microscaling FP4 Quantization" summary,
modification 3: activations are rotated at inference by block-diagonal
Hadamard rotations, which lowers the quantization error without slowing the
forward pass.  The page gives neither the block size nor the construction;
the readings are:

* H_n is the Sylvester matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]),
  symmetric, with no random sign flips and no sequency reordering.
* The rotation is orthonormal ("rotation"): each consecutive run of n
  elements along K is replaced by r = c_n * (x_block @ H_n), c_n = 1/sqrt(n).
* n is 16, 32 or 128 and must divide K.  The rotation blocks are independent
  of the quantization blocks.
* Rounding: the sum S = x_block @ H_n is exact (see below); c_n is the
  float64 nearest to 1/sqrt(n) (exactly 1/4 for n = 16); r is
  RN_fp32(RN_fp64(c_n * S)).  For n = 16 this is a single rounding.
* An exactly-zero sum is the real number zero and rotates to +0.0 (the sign
  an IEEE sum of signed zeros would give depends on the summation order,
  which the rotation does not define); a nonzero sum that underflows keeps
  its sign.

S is computed in float64 and is exact when every partial sum fits in 53
bits: with M the largest exponent of |x| in the block and L the smallest
exponent of a nonzero input's last mantissa bit, M + 1 + log2(n) - L <= 53.
The oracle checks this condition and refuses inputs that break it.
"""

from __future__ import annotations

import math

import numpy as np

SIZES = (16, 32, 128)


def sylvester(n: int) -> np.ndarray:
    """Integer Sylvester-Hadamard matrix of order n (a power of two)."""
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def scale_factor(n: int) -> float:
    """float64 nearest to 1/sqrt(n) for n a power of two.

    For even log2(n) it is an exact power of two; otherwise 1/sqrt(n) =
    sqrt(2) / 2**((log2 n + 1) / 2), and sqrt(2.0) is correctly rounded, so
    dividing it by a power of two gives the nearest float64.
    """
    k = int(math.log2(n))
    if k % 2 == 0:
        return 2.0 ** (-k // 2)
    return math.sqrt(2.0) / 2.0 ** ((k + 1) // 2)


def _last_bit_exponent(x: np.ndarray, mant_bits: int) -> np.ndarray:
    """Exponent of the last significant bit of each nonzero float value."""
    _, ex = np.frexp(x)
    return ex.astype(np.int64) - 1 - mant_bits


def check_exact(xb: np.ndarray, n: int, mant_bits: int) -> None:
    a = np.abs(xb)
    nz = a > 0
    if not nz.any():
        return
    _, ex = np.frexp(np.where(nz, a, 1.0))
    top = np.where(nz, ex - 1, -100000).max(axis=-1)
    low = np.where(nz, _last_bit_exponent(np.where(nz, a, 1.0), mant_bits),
                   100000).min(axis=-1)
    need = top + 1 + int(math.log2(n)) - low
    has = nz.any(axis=-1)
    if np.any(has & (need > 53)):
        raise ValueError("Hadamard block dynamic range too wide for an exact "
                         "float64 sum (outside the contract)")


def rotate(x: np.ndarray, n: int, mant_bits: int = 23) -> np.ndarray:
    """Rotate each n-block along K of a [rows, K] array; returns float32.

    ``mant_bits`` is the stored mantissa width of the input values (23 for
    float32, 7 for bfloat16); it only enters the exactness check.
    """
    if n not in SIZES:
        raise ValueError(f"Hadamard size {n} not in {SIZES}")
    x = np.asarray(x)
    rows, k = x.shape
    if k % n:
        raise ValueError(f"K={k} is not a multiple of the Hadamard size {n}")
    xb = x.astype(np.float64).reshape(rows, k // n, n)
    if not np.all(np.isfinite(xb)):
        raise ValueError("non-finite input is outside the contract")
    check_exact(xb, n, mant_bits)
    s = xb @ sylvester(n).astype(np.float64)          # exact (checked above)
    s = np.where(s == 0.0, 0.0, s)                    # the real zero is +0
    r = (scale_factor(n) * s).astype(np.float32)
    return r.reshape(rows, k)
