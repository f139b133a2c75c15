"""Least-squared-error block and tensor scales for 4-bit weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the "Bridging the Gap ... Microscaling FP4 Quantization" summary,
MR-GPTQ modification 1: the quantization grid is chosen for least mean
squared error by optimising the scale of every block and the scale of the
tensor in turn; this helps NVFP4 markedly (without rotations).  The same
passage says that for MXFP4 under Hadamard rotations one fixed grid scale
serves every model; it does not give that scale.

Readings (the page gives no candidate sets, criterion arithmetic or number
of rounds):

* Error of a block under a scale: SSE = the sum over the block's elements,
  in element order, of (x - x_hat)**2, every subtraction, product and
  addition rounded to float64 on its own (no fused multiply-add); x_hat is
  the exact dequantized value (element code value times the scale).  The
  element codes under a scale are the ordinary ones (nearest, ties to even,
  saturating; quantize.py).
* Block step: a block's scale code is the one with the smallest SSE among
  every code of its scale format -- E8M0 codes 0..254 (MXFP4, scale
  2**(c - 127)) or E4M3 codes 0..126 times the tensor scale g (NVFP4) --
  ties going to the smaller code.  (So a block the amax rule already fits
  exactly keeps its amax-rule code or a smaller one.)
* Tensor step (NVFP4): with every block's code s_b and element codes q fixed,
  the least-squares tensor scale is P / Q with P = sum x * w, Q = sum w * w,
  w = q_value * E4M3(s_b); each of P and Q is a float64 sum of row sums
  (each row summed over K in order), rows added in order; g = RN_fp32 of the
  float64 quotient.  Q = 0, or a quotient that rounds to 0 in float32, keeps
  the previous g.
* Rounds: NVFP4 starts from the amax-rule g (quantize.nvfp4_tensor_scale),
  then block step, tensor step, block step.  MXFP4 has no tensor scale: one
  block step.
* INT4's float32 scale has no discrete candidate set and keeps the amax rule;
  the rotated-MXFP4 fixed grid scale is not implemented (no value given).

Each x * w product is exact in float64 (24 + 6 significant bits), so only the
additions of P and Q round.
"""

from __future__ import annotations

import numpy as np

from .formats import E2M1, E4M3
from .quantize import _blocks, nvfp4_tensor_scale

E8M0_CODES = 255           # 0..254 (255 is NaN)
E4M3_CODES = 127           # 0..126 (127 is NaN)


def sse_in_order(xb: np.ndarray, x_hat: np.ndarray) -> np.ndarray:
    """Sum over the last axis, in order, of (x - x_hat)**2, each operation
    rounded to float64 separately."""
    s = np.zeros(xb.shape[:-1], dtype=np.float64)
    for i in range(xb.shape[-1]):
        d = xb[..., i] - x_hat[..., i]
        s = s + d * d
    return s


def _e2m1_dequant(xb: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Element codes of x under a positive per-block scale and their exact
    values (code value times scale); a zero scale gives signed zeros."""
    sc = scale[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(sc > 0, xb / np.where(sc > 0, sc, 1.0), 0.0 * xb)
    codes = E2M1.encode(v)
    return codes, E2M1.decode(codes) * sc


def _argmin_codes(xb: np.ndarray, scale_of_code, n_codes: int):
    """Exhaustive block step: the code with the smallest SSE, ties to the
    smaller code; returns (codes [rows, blocks], their SSE)."""
    best = best_code = None
    for c in range(n_codes):
        sc = scale_of_code(c)
        _, x_hat = _e2m1_dequant(xb, sc)
        sse = sse_in_order(xb, x_hat)
        if best is None:
            best, best_code = sse, np.zeros(sse.shape, dtype=np.int64)
        else:
            better = sse < best
            best = np.where(better, sse, best)
            best_code = np.where(better, c, best_code)
    return best_code, best


def mx_block_step(x: np.ndarray):
    """MXFP4 block step over every E8M0 code; returns (E8M0 codes uint8
    [rows, K/32], SSE per block)."""
    xb = _blocks(x, 32)
    ones = np.ones(xb.shape[:-1])
    codes, sse = _argmin_codes(xb, lambda c: ones * np.ldexp(1.0, c - 127), E8M0_CODES)
    return codes.astype(np.uint8), sse


def nvfp4_block_step(x: np.ndarray, g) -> tuple:
    """NVFP4 block step for tensor scale g over every E4M3 code; returns
    (E4M3 codes uint8 [rows, K/16], SSE per block)."""
    xb = _blocks(x, 16)
    g64 = float(np.float32(g))
    ones = np.ones(xb.shape[:-1])
    codes, sse = _argmin_codes(xb, lambda c: ones * (float(E4M3.mags[c]) * g64), E4M3_CODES)
    return codes.astype(np.uint8), sse


def nvfp4_elements(x: np.ndarray, s_codes: np.ndarray, g):
    """Element codes [rows, K] under block codes s_codes and tensor scale g."""
    xb = _blocks(x, 16)
    scale = E4M3.decode(s_codes) * float(np.float32(g))
    codes, _ = _e2m1_dequant(xb, scale)
    return codes.reshape(x.shape)


def nvfp4_tensor_step(x: np.ndarray, s_codes: np.ndarray, g) -> np.float32:
    """Least-squares tensor scale for fixed block and element codes."""
    x64 = np.asarray(x, dtype=np.float64)
    rows, k = x64.shape
    q = nvfp4_elements(x, s_codes, g)
    w = E2M1.decode(q) * np.repeat(E4M3.decode(s_codes), 16, axis=1)   # exact
    p_rows = np.zeros(rows)
    q_rows = np.zeros(rows)
    for j in range(k):                      # each row summed over K in order
        p_rows = p_rows + x64[:, j] * w[:, j]
        q_rows = q_rows + w[:, j] * w[:, j]
    p_tot = q_tot = 0.0
    for r in range(rows):                   # rows added in order
        p_tot = p_tot + float(p_rows[r])
        q_tot = q_tot + float(q_rows[r])
    if q_tot == 0.0:
        return np.float32(g)
    g_new = np.float32(p_tot / q_tot)
    return np.float32(g) if g_new == 0 else g_new


def quantize_mse(x: np.ndarray, fmt: str) -> dict:
    """MSE-scale quantization of float32 weights [rows, K] to MXFP4 or NVFP4;
    the same dict layout as quantize.quantize."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == "MXFP4":
        s_codes, _ = mx_block_step(x)
        xb = _blocks(x, 32)
        codes, _ = _e2m1_dequant(xb, np.ldexp(1.0, s_codes.astype(np.int64) - 127))
        return {"fmt": fmt, "codes": codes.reshape(x.shape), "scales": s_codes, "g": None}
    if fmt == "NVFP4":
        g0 = nvfp4_tensor_scale(x)
        s1, _ = nvfp4_block_step(x, g0)
        g1 = nvfp4_tensor_step(x, s1, g0)
        s2, _ = nvfp4_block_step(x, g1)
        return {"fmt": fmt, "codes": nvfp4_elements(x, s2, g1), "scales": s2, "g": g1}
    raise ValueError(f"MSE scales are defined for MXFP4 and NVFP4, not {fmt}")
