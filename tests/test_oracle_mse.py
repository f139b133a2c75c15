"""Pins for oracle.mse_scales (least-squared-error block and tensor scales):
exact-rational brute force over every scale code on small blocks, the
least-squares property of the tensor step, never-worse-than-amax, exact
blocks, power-of-two invariance, degenerate blocks, and planted slips."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import mse_scales as om
from oracle import quantize as oq
from oracle.formats import E2M1, E4M3
from tests import exact as ex


def _blocks(kind, n_blocks, size, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.normal(0, 0.02, size=(n_blocks, size))
    elif kind == "student":
        x = rng.standard_t(2, size=(n_blocks, size)) * 0.02
    elif kind == "uniform":
        x = rng.uniform(-0.03, 0.03, size=(n_blocks, size))
    else:  # one outlier per block
        x = rng.normal(0, 0.01, size=(n_blocks, size))
        x[np.arange(n_blocks), rng.integers(0, size, n_blocks)] *= 40
    return x.astype(np.float32)


def _exact_sse(xs, scale):
    """Exact SSE of one block under a scale (Fractions; independent encoder)."""
    grid = ex.e2m1_grid()
    scale = Fraction(scale)
    tot = Fraction(0)
    for x in xs:
        v = Fraction(float(x))
        if scale == 0:
            xh = Fraction(0)
        else:
            c = ex.round_to_grid(v / scale, grid)
            xh = grid[c] * scale * (-1 if v < 0 else 1)
        tot += (v - xh) ** 2
    return tot


def _check_choice(xs, chosen, scales_by_code, sse_fp64_of):
    exact = [_exact_sse(xs, s) for s in scales_by_code]
    best = min(exact)
    want = exact.index(best)                       # ties to the smaller code
    if chosen != want:
        # only a certified near-tie may differ: the two fp64 SSEs agree to 1e-12
        a, b = sse_fp64_of(chosen), sse_fp64_of(want)
        assert abs(a - b) <= 1e-12 * max(a, b), (chosen, want, a, b)
        assert exact[chosen] - best <= Fraction(1, 10 ** 12) * best


@pytest.mark.parametrize("kind", ["normal", "student", "uniform", "outlier"])
def test_mx_block_step_is_the_exact_argmin(kind):
    x = _blocks(kind, 6, 32, seed=len(kind))
    codes, sse = om.mx_block_step(x)
    for b in range(x.shape[0]):
        # every E8M0 code: 2**(c - 127)
        scales = [Fraction(2) ** (c - 127) for c in range(255)]
        xb = x[b:b + 1].astype(np.float64).reshape(1, 1, 32)

        def fp64(c, xb=xb):
            _, xh = om._e2m1_dequant(xb, np.array([[np.ldexp(1.0, c - 127)]]))
            return float(om.sse_in_order(xb, xh)[0, 0])
        _check_choice(x[b], int(codes[b, 0]), scales, fp64)
        assert sse[b, 0] == fp64(int(codes[b, 0]))


@pytest.mark.parametrize("kind", ["normal", "student", "outlier"])
def test_nvfp4_block_step_is_the_exact_argmin(kind):
    x = _blocks(kind, 6, 16, seed=10 + len(kind))
    g = oq.nvfp4_tensor_scale(x)
    codes, _ = om.nvfp4_block_step(x, g)
    e4 = ex.e4m3_grid()
    for b in range(x.shape[0]):
        scales = [Fraction(0)] + [v * Fraction(float(g)) for v in e4[1:]]
        xb = x[b:b + 1].astype(np.float64).reshape(1, 1, 16)

        def fp64(c, xb=xb):
            _, xh = om._e2m1_dequant(xb, np.array([[float(E4M3.mags[c]) * float(g)]]))
            return float(om.sse_in_order(xb, xh)[0, 0])
        _check_choice(x[b], int(codes[b, 0]), scales, fp64)


def _total_sse(x, q):
    xh = oq.dequantize(q).astype(np.float64)
    d = x.astype(np.float64) - xh
    return float(np.sum(d * d))


@pytest.mark.parametrize("fmt", ["MXFP4", "NVFP4"])
def test_never_worse_than_amax_rule(fmt):
    rng = np.random.default_rng(5)
    w = (rng.standard_t(3, size=(24, 256)) * 0.02).astype(np.float32)
    q_mse = om.quantize_mse(w, fmt)
    q_amax = oq.quantize(w, fmt)
    bs = 32 if fmt == "MXFP4" else 16
    xb = w.astype(np.float64).reshape(24, -1, bs)
    e_mse = (w - oq.dequantize(q_mse)).reshape(24, -1, bs)
    e_amx = (w - oq.dequantize(q_amax)).reshape(24, -1, bs)
    if fmt == "MXFP4":
        # the block step alone: blockwise never worse
        s_mse = om.sse_in_order(xb, xb - e_mse)
        s_amx = om.sse_in_order(xb, xb - e_amx)
        assert np.all(s_mse <= s_amx)
        assert np.any(s_mse < s_amx)             # and better somewhere
    t_mse, t_amx = _total_sse(w, q_mse), _total_sse(w, q_amax)
    assert t_mse <= t_amx * (1 + 1e-12)
    assert t_mse < (0.99 if fmt == "MXFP4" else 0.97) * t_amx   # a real improvement


def test_nvfp4_rounds_are_monotone_and_tensor_step_is_least_squares():
    rng = np.random.default_rng(6)
    w = (rng.laplace(size=(16, 128)) * 0.02).astype(np.float32)
    g0 = oq.nvfp4_tensor_scale(w)
    s1, sse1 = om.nvfp4_block_step(w, g0)
    g1 = om.nvfp4_tensor_step(w, s1, g0)
    s2, sse2 = om.nvfp4_block_step(w, g1)
    _, sse0 = om.nvfp4_block_step(w, g0)
    assert sse2.sum() <= sse1.sum() * (1 + 1e-12)
    # least squares for fixed codes: the exact rational optimum of
    # sum (x - g w)^2 over g is P/Q; g1 is its nearest float32
    q = om.nvfp4_elements(w, s1, g0)
    wv = E2M1.decode(q) * np.repeat(E4M3.decode(s1), 16, axis=1)
    P = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(w.ravel(), wv.ravel()))
    Q = sum(Fraction(float(b)) ** 2 for b in wv.ravel())
    g_exact = P / Q
    assert Fraction(float(g1)) == ex.rn_f32(g_exact)
    # and with the codes held fixed, g1 does no worse than g0
    fixed = lambda g: sum((Fraction(float(a)) - Fraction(float(g)) * Fraction(float(b))) ** 2
                          for a, b in zip(w.ravel(), wv.ravel()))
    assert fixed(g1) <= fixed(g0)


def test_exact_blocks_zero_blocks_and_invariance():
    # a block built from E2M1 grid values times 2**-7 is reproduced exactly
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rng = np.random.default_rng(7)
    x = (rng.choice(grid, size=(3, 32)) * rng.choice([-1, 1], size=(3, 32)) * 2.0 ** -7)
    x[:, 0] = 6 * 2.0 ** -7
    x = x.astype(np.float32)
    q = om.quantize_mse(x, "MXFP4")
    assert np.array_equal(oq.dequantize(q), x.astype(np.float64))
    # the amax rule's code fits exactly; no smaller code can (6 * 2**-7 would saturate)
    assert np.all(q["scales"] == oq.quantize(x, "MXFP4")["scales"])
    # all-zero blocks take code 0 (every code ties), NVFP4 of a zero tensor keeps g = 0
    z = np.zeros((2, 64), np.float32)
    assert np.all(om.quantize_mse(z, "MXFP4")["scales"] == 0)
    qz = om.quantize_mse(z, "NVFP4")
    assert float(qz["g"]) == 0.0 and np.all(qz["scales"] == 0)
    # power-of-two invariance of the MX choice (exact scaling)
    y = _blocks("student", 4, 32, seed=8)
    a, b = om.quantize_mse(y, "MXFP4"), om.quantize_mse((y * 2.0 ** 5).astype(np.float32), "MXFP4")
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(b["scales"].astype(int), a["scales"].astype(int) + 5)
    # sign symmetry
    c = om.quantize_mse(-y, "MXFP4")
    assert np.array_equal(c["scales"], a["scales"])
    assert np.array_equal(c["codes"] ^ 8, a["codes"]) or np.all((a["codes"] & 7) == 0)


def test_planted_slips_fail_the_pins(monkeypatch):
    """Ties to the larger code, and a search that only tries the amax-rule
    code, each fail a pin above."""
    x = np.zeros((1, 32), np.float32)
    assert om.mx_block_step(x)[0][0, 0] == 0
    orig = om._argmin_codes

    def ties_to_larger(xb, scale_of_code, n):
        best = best_code = None
        for c in range(n):
            _, xh = om._e2m1_dequant(xb, scale_of_code(c))
            s = om.sse_in_order(xb, xh)
            if best is None:
                best, best_code = s, np.zeros(s.shape, dtype=np.int64)
            else:
                better = s <= best
                best, best_code = np.where(better, s, best), np.where(better, c, best_code)
        return best_code, best
    monkeypatch.setattr(om, "_argmin_codes", ties_to_larger)
    assert om.mx_block_step(x)[0][0, 0] == 254           # the zero-block pin fails
    monkeypatch.setattr(om, "_argmin_codes", orig)

    def amax_only(xw, fmt):
        return oq.quantize(xw, fmt)
    rng = np.random.default_rng(5)
    w = (rng.standard_t(3, size=(24, 256)) * 0.02).astype(np.float32)
    assert not (_total_sse(w, amax_only(w, "NVFP4")) < 0.97 * _total_sse(w, oq.quantize(w, "NVFP4")))
