"""GPU parity: mxq_lowrank_split (offline SVDQuant split) against the
oracle's truncated SVD (numpy, float64).  What is unique is compared: the
singular values, the branch L1 L2 and the residual R (singular pairs carry
an arbitrary sign); R + (L1 L2)^T must give back W; and the split feeds the
MXFP4 layer (the residual quantized, the branch added in the GEMM epilogue)
with a smaller error than quantizing W itself."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import gemm as og
from oracle import lowrank as olr
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _lowrank_plus_noise(n, k, r, seed, strength=2.0):
    """A weight with a dominant rank-r part (singular values well above the
    noise's) plus N(0, 0.02) noise."""
    rng = np.random.default_rng(seed)
    a = rng.normal(size=(n, r)) * np.linspace(1.0, 0.3, r)[None, :]
    b = rng.normal(size=(r, k))
    w = strength * (a @ b) / np.sqrt(k) + rng.normal(0, 0.02, size=(n, k))
    return w.astype(np.float32)


def _bf16(t):
    return t.float().cpu().numpy().astype(np.float64)


def _compare(w, r, l1t, l2t, resid, sigma, tag):
    l1, l2, res_o, sig_o = olr.svd_split(w, r)
    sig = sigma.cpu().numpy().astype(np.float64)
    assert np.allclose(sig, sig_o[:r], rtol=2e-5, atol=1e-6 * sig_o[0]), (tag, sig[:4], sig_o[:4])
    g1, g2 = _bf16(l1t).T, _bf16(l2t).T           # L1 [k][r], L2 [r][n]
    prod_g, prod_o = (g1 @ g2).T, (l1 @ l2).T
    # each factor element is one bf16 rounding (2**-9 relative) of a value the
    # two sides compute to fp32 accuracy: the products agree to 2**-7 of the
    # absolute sum, plus the subspace's fp32 error
    tol = 2.0 ** -7 * (np.abs(l1) @ np.abs(l2)).T + 2e-5 * sig_o[0] / np.sqrt(min(w.shape))
    assert np.all(np.abs(prod_g - prod_o) <= tol), (tag, float(np.max(np.abs(prod_g - prod_o) / tol)))
    res = resid.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(res - res_o) <= tol + 2.0 ** -22 * np.abs(w)), tag
    # R + (L1 L2)^T = W up to the fp32 roundings of R
    back = res + prod_g
    assert np.all(np.abs(back - w) <= 2.0 ** -22 * (np.abs(w) + (np.abs(g1) @ np.abs(g2)).T) + 1e-30)
    return res, prod_g, sig_o


@pytest.mark.parametrize("n,k,r", [(384, 512, 32), (200, 136, 16), (64, 1024, 8)])
def test_lowrank_split_matches_oracle(n, k, r):
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say(f"lowrank split n={n} k={k} rank={r}")
    w = _lowrank_plus_noise(n, k, r, seed=n + k + r)
    l1t, l2t, resid, sigma = mxq.lowrank_split(gu.to_dev_f32(w), r)
    _compare(w, r, l1t, l2t, resid, sigma, f"{n}x{k} r{r}")


def test_lowrank_split_exact_structure():
    """A signed-permutation matrix around exact squares splits exactly (up to
    the fp32 subspace arithmetic): the top-r part, and a residual holding the
    rest."""
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say("lowrank split: known singular structure")
    rng = np.random.default_rng(0)
    n = 64
    s = np.zeros(n)
    s[:8] = [64.0, 36.0, 16.0, 9.0, 4.0, 2.25, 1.0, 0.25]
    s[8:] = 0.001 * rng.random(n - 8)
    p = np.zeros((n, n)); p[np.arange(n), rng.permutation(n)] = rng.choice([-1, 1], n)
    q = np.zeros((n, n)); q[np.arange(n), rng.permutation(n)] = rng.choice([-1, 1], n)
    w = (p @ np.diag(s) @ q).astype(np.float32)
    l1t, l2t, resid, sigma = mxq.lowrank_split(gu.to_dev_f32(w), 6)
    assert np.allclose(sigma.cpu().numpy(), s[:6], rtol=1e-5)
    top = p @ np.diag(np.where(np.arange(n) < 6, s, 0.0)) @ q
    prod = (_bf16(l1t).T @ _bf16(l2t).T).T
    assert np.max(np.abs(prod - top)) <= 2.0 ** -8 * 64


def test_lowrank_split_full_layer_feeds_the_mxfp4_layer():
    """The 3072 x 3072 layer shape with a dominant rank-32 part: sampled rows
    against the oracle, the residual's energy against Eckart-Young, and the
    split (MXFP4 residual + bf16 branch) beats quantizing W directly."""
    import fp8_quantized_linear_mxq_amd as mxq
    import torch
    n = k = 3072
    r = 32
    gu.say(f"lowrank split full layer {n}x{k} rank {r}")
    w = _lowrank_plus_noise(n, k, r, seed=77, strength=2.0)
    wd = gu.to_dev_f32(w)
    l1t, l2t, resid, sigma = mxq.lowrank_split(wd, r)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    mxq.lowrank_split(wd, r)
    e1.record()
    torch.cuda.synchronize()
    gu.say(f"  split time {e0.elapsed_time(e1):.2f} ms")
    sig_o = np.linalg.svd(w.astype(np.float64), compute_uv=False)
    assert np.allclose(sigma.cpu().numpy(), sig_o[:r], rtol=5e-5)
    res = resid.cpu().numpy().astype(np.float64)
    tail = float(np.sum(sig_o[r:] ** 2))
    assert abs(float(np.sum(res * res)) - tail) <= 0.01 * tail
    # the layer: activations like the SVDQuant workload's, both routes
    x_bits = wl.activations(wl.WORKLOADS["svdq_r32"], rows=256)
    x = wl.bf16_to_f32(x_bits).astype(np.float64)
    xd = gu.to_dev_bf16(x_bits)
    u = torch.empty((256, r), dtype=torch.float32, device="cuda")
    qa = mxq.quantize(xd, mxq.MXFP4, l1t=l1t, u=u)
    y_split = mxq.gemm(qa, mxq.quantize(resid, mxq.MXFP4), u=u, l2t=l2t)
    y_direct = mxq.gemm(mxq.quantize(xd, mxq.MXFP4), mxq.quantize(wd, mxq.MXFP4))
    ref = og.linear(x, w.astype(np.float64))
    e_split = float(np.linalg.norm(y_split.float().cpu().numpy() - ref))
    e_direct = float(np.linalg.norm(y_direct.float().cpu().numpy() - ref))
    gu.say(f"  layer error vs x W^T: split {e_split:.4g}, direct {e_direct:.4g}")
    assert e_split < e_direct
