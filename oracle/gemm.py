"""Quantized linear layer in float64, with the low-rank branch and the bound.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: the Nunchaku / SVDQuant article, "main explanation": the layer runs
a 4-bit weight x 4-bit activation product and keeps a 16-bit low-rank part of
the weight next to it, so y = Q(x) Q(R)^T + (x L1) L2.  The Chameleon article
("hardware support" paragraph) notes that channel-wise mixed formats need the
product split into groups or weights unpacked inside the kernel; the value
computed is the same.

Readings (the pages are silent):
* W is stored [N, K] (out x in) and y[m, n] = sum_k a[m, k] w[n, k] over the
  dequantized operands, accumulated exactly (float64 here).
* alpha = g_a * g_w (exact real product) when both operands are NVFP4, else 1.
* The low-rank branch reads the unrotated, unquantized activations:
  u = x @ L1 ([M, r], kept unrounded), added as u @ L2.
* The output is rounded once to bfloat16 (nearest even).
* Tolerance for a GPU result with float32 accumulation:
  |y_gpu - y| <= 1e-5 (1 + 2**-8) S + 2**-8 |y| + 2**-133, with
  S = alpha sum_k |a w| + sum_j sum_k |x L1| |L2|.  The last two terms are
  the bfloat16 output rounding: half an ulp is at most 2**-8 |y| for a
  normal bfloat16 and 2**-134 for a subnormal one (|y| < 2**-126), where
  the float32 value being rounded can also carry up to 2**-150 of
  underflow; 2**-133 bounds that absolute part.
"""

from __future__ import annotations

import numpy as np

from .formats import round_to_bf16

REL_TOL = 1e-5


def lowrank_down(x: np.ndarray, l1: np.ndarray) -> np.ndarray:
    """u = x @ L1 in float64 ([M, K] x [K, r])."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(l1, dtype=np.float64)


def linear(a_deq: np.ndarray, w_deq: np.ndarray, alpha: float = 1.0,
           u: np.ndarray | None = None, l2: np.ndarray | None = None,
           bias: np.ndarray | None = None) -> np.ndarray:
    """Exact-as-float64 pre-rounding output y = alpha a w^T (+ u L2) (+ bias)."""
    a = np.asarray(a_deq, dtype=np.float64)
    w = np.asarray(w_deq, dtype=np.float64)
    y = float(alpha) * (a @ w.T)
    if u is not None:
        y = y + np.asarray(u, dtype=np.float64) @ np.asarray(l2, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def linear_bf16(*args, **kwargs) -> np.ndarray:
    """The layer output rounded once to bfloat16 (returned as float64 values)."""
    return round_to_bf16(linear(*args, **kwargs))


def abs_sum_bound(a_deq, w_deq, alpha=1.0, x=None, l1=None, l2=None) -> np.ndarray:
    """S[m, n] = alpha sum_k |a w| + sum_j sum_k |x| |L1| |L2|."""
    s = abs(float(alpha)) * (np.abs(np.asarray(a_deq, np.float64))
                             @ np.abs(np.asarray(w_deq, np.float64)).T)
    if l1 is not None:
        s = s + (np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(l1, np.float64))) \
            @ np.abs(np.asarray(l2, np.float64))
    return s


BF16_SUBNORMAL_TERM = 2.0 ** -133


def tolerance(y_exact: np.ndarray, s_bound: np.ndarray) -> np.ndarray:
    return (REL_TOL * (1.0 + 2.0 ** -8) * s_bound + 2.0 ** -8 * np.abs(y_exact)
            + BF16_SUBNORMAL_TERM)
