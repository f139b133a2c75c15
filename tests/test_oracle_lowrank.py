"""Pins for oracle.lowrank (the offline SVD split): a matrix with known
singular structure (signed permutations around exact squares), the
Eckart-Young residual energy, the branch's own singular values, and the
rank-r reconstruction of an exactly low-rank matrix."""
import numpy as np
import pytest

from oracle import lowrank as olr


def _signed_perm(n, rng):
    p = np.zeros((n, n))
    p[np.arange(n), rng.permutation(n)] = rng.choice([-1.0, 1.0], n)
    return p


def test_known_singular_structure_is_split_exactly():
    # W = P diag(s) Q with signed permutations and s exact squares of
    # bfloat16 values: the top-r part is exactly the r largest entries
    rng = np.random.default_rng(0)
    n = 12
    s = np.array([64.0, 16.0, 9.0, 4.0, 2.25, 1.0, 0.25, 0.0625, 0.015625, 0.0, 0.0, 0.0])
    p, q = _signed_perm(n, rng), _signed_perm(n, rng)
    w = p @ np.diag(s) @ q
    for r in (1, 3, 5):
        l1, l2, resid, sig = olr.svd_split(w.astype(np.float32), r)
        assert np.allclose(sig, s, rtol=0, atol=1e-12)
        top = p @ np.diag(np.where(np.arange(n) < r, s, 0.0)) @ q
        assert np.array_equal((l1 @ l2).T, top)            # exact: sqrt(s) are bf16 values
        assert np.array_equal(resid.astype(np.float64), w - top)


def test_eckart_young_energy_and_branch_spectrum():
    rng = np.random.default_rng(1)
    n, k, r = 48, 64, 6
    w = (rng.normal(size=(n, r)) @ rng.normal(size=(r, k)) * 3 + rng.normal(size=(n, k)) * 0.1)
    w = w.astype(np.float32)
    l1, l2, resid, sig = olr.svd_split(w, r)
    # the residual carries the tail energy, up to the factors' bf16 rounding
    tail = float(np.sum(sig[r:] ** 2))
    e = float(np.sum(resid.astype(np.float64) ** 2))
    assert abs(e - tail) <= 0.05 * tail + 1e-3 * float(np.sum(sig[:r] ** 2)) * 2 ** -8
    # the branch's singular values are the top r, to bf16 accuracy
    bs = np.linalg.svd((l1 @ l2), compute_uv=False)[:r]
    assert np.allclose(bs, sig[:r], rtol=2 ** -7)
    # shapes in the layer's orientation
    assert l1.shape == (k, r) and l2.shape == (r, n) and resid.shape == (n, k)


@pytest.mark.parametrize("r", [4, 8])
def test_exactly_low_rank_matrix_leaves_a_bf16_sized_residual(r):
    rng = np.random.default_rng(2)
    n, k = 40, 56
    w = (rng.normal(size=(n, r)) @ rng.normal(size=(r, k))).astype(np.float32)
    l1, l2, resid, sig = olr.svd_split(w, r)
    assert sig[r] <= 1e-5 * sig[0]
    bound = 2 ** -7 * (np.abs(l1) @ np.abs(l2)).T + 1e-5 * sig[0]
    assert np.all(np.abs(resid) <= bound)
    # rank larger than needed changes nothing above rounding
    l1b, l2b, resid_b, _ = olr.svd_split(w, r + 2)
    assert np.max(np.abs(resid_b)) <= np.max(bound)
