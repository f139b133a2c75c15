"""Offline SVDQuant split of a weight: W ~= (L1 L2)^T + R.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the Nunchaku / SVDQuant article, "main explanation": the hardest
part of each weight matrix is kept as a separate low-rank 16-bit branch and
the rest is quantized to 4 bits.

Readings (the page gives no formula):

* W is [N, K] (out x in) and the layer computes y = x W^T, so the branch is
  u = x L1 (L1 [K, r]), y_lr = u L2 (L2 [r, N]), i.e. W ~= (L1 L2)^T + R.
* "The hardest part" is the best rank-r approximation in the least-squares
  (Frobenius) sense, the truncated SVD W_r = U_r S_r V_r^T (Eckart-Young).
* The factors share the singular values evenly: L1 = V_r sqrt(S_r),
  L2 = sqrt(S_r) U_r^T, each rounded once to bfloat16 (the 16-bit branch).
* R = W - (L1 L2)^T with the rounded factors, in float64, rounded once to
  float32 (the residual then goes through any weight quantizer).
* The SVD's factors are unique only up to sign per singular pair (and not at
  all inside a repeated singular value); L1 L2 and R are unique whenever
  sigma_r > sigma_{r+1}, which is what a comparison may rely on.
"""

from __future__ import annotations

import numpy as np

from .formats import round_to_bf16


def svd_split(w: np.ndarray, rank: int):
    """Returns (L1 [K, r], L2 [r, N], R [N, K] float32, sigma [min(N, K)])
    with L1 and L2 bfloat16 values carried in float64."""
    w64 = np.asarray(w, dtype=np.float64)
    u, s, vt = np.linalg.svd(w64, full_matrices=False)   # W = U diag(s) V^T
    r = int(rank)
    root = np.sqrt(s[:r])
    l1 = round_to_bf16(vt[:r].T * root[None, :])          # V_r sqrt(S_r)
    l2 = round_to_bf16(root[:, None] * u[:, :r].T)        # sqrt(S_r) U_r^T
    resid = (w64 - (l1 @ l2).T).astype(np.float32)
    return l1, l2, resid, s
