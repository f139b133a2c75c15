"""Per-output-channel weight format choice by least reconstruction error.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the Chameleon article, "the format is chosen by the value
distribution": weights do not depend on the diffusion step, so a format is
chosen separately for every output channel by trying the available variants
and keeping the one with the smallest reconstruction error, with no
retraining.

Readings (the pages are silent):
* The palette is INT4 (symmetric, per 32), MXFP4 and NVFP4; an output
  channel is a row of W [N, K].
* Error = sum_k (w_k - w_hat_k)**2 in float64 over the row (equivalent to MSE
  since K is shared).  w is the float32 master value, w_hat the exact
  dequantized value; each squared difference is exact in float64.
* NVFP4 candidates use one tensor scale computed over the whole W.
* argmin, ties to the earliest candidate in the given order.
* The permutation lists rows grouped by chosen format in candidate order,
  stable (ascending row index) inside each group.
"""

from __future__ import annotations

import numpy as np

from .quantize import NVFP4, dequantize, nvfp4_tensor_scale, quantize

PALETTE = ("INT4", "MXFP4", "NVFP4")


def row_sse(w: np.ndarray, candidates=PALETTE):
    """[N, len(candidates)] float64 reconstruction SSE per row and format."""
    w = np.asarray(w, dtype=np.float32)
    w64 = w.astype(np.float64)
    g = nvfp4_tensor_scale(w) if NVFP4 in candidates else None
    sse = np.empty((w.shape[0], len(candidates)), dtype=np.float64)
    for j, fmt in enumerate(candidates):
        q = quantize(w, fmt, tensor_scale=g if fmt == NVFP4 else None)
        d = w64 - dequantize(q)
        sse[:, j] = np.sum(d * d, axis=1)
    return sse


def select_formats(w: np.ndarray, candidates=PALETTE):
    """Returns (choice index per row [N], sse [N, C], perm [N] int32)."""
    sse = row_sse(w, candidates)
    choice = np.argmin(sse, axis=1)                    # first minimum wins
    perm = np.argsort(choice, kind="stable").astype(np.int32)
    return choice.astype(np.uint8), sse, perm
