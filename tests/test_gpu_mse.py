"""GPU parity: mxq_quantize_mse (least-squared-error weight scales) against
oracle.mse_scales, bit-exact on codes, scales and the NVFP4 tensor scale;
at full layer size, sampled rows against the oracle's block step under the
GPU's tensor scale, and the total squared error against the amax rule."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import mse_scales as om
from oracle import quantize as oq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _weights(rows, cols, seed):
    rng = np.random.default_rng(seed)
    w = np.empty((rows, cols))
    for i in range(rows):
        fam = i % 4
        if fam == 0:
            w[i] = rng.normal(0, 0.02, cols)
        elif fam == 1:
            w[i] = rng.standard_t(2, cols) * 0.02
        elif fam == 2:
            w[i] = rng.uniform(-0.03, 0.03, cols)
        else:
            w[i] = rng.laplace(0, 0.01, cols)
            w[i, rng.integers(0, cols, 3)] *= 60
    if rows >= 4:
        w[1] = 0.0                                        # an all-zero row
        w[2] *= 2.0 ** -100                               # tiny blocks
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
        w[3, :64] = rng.choice(grid, 64) * rng.choice([-1, 1], 64) * 2.0 ** -9   # exact blocks
    return w.astype(np.float32)


def _check(q, want, fmt):
    got_codes = gu.unpack_dev_codes(q, fmt)
    got_scales = gu.dev_scales(q, fmt)
    bad = np.argwhere(got_scales != want["scales"])
    assert bad.size == 0, (f"scale mismatch at {bad[:5].tolist()}: got "
                           f"{got_scales[tuple(bad[0])]} want {want['scales'][tuple(bad[0])]}")
    bad = np.argwhere(got_codes != want["codes"])
    assert bad.size == 0, f"code mismatch at {bad[:5].tolist()}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["MXFP4", "NVFP4"])
def test_mse_scales_match_oracle(fmt, dtype):
    import fp8_quantized_linear_mxq_amd as mxq
    rows, cols = 37, 384
    w = _weights(rows, cols, seed=3 if fmt == "MXFP4" else 4)
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(w)
        w, dev = wl.bf16_to_f32(bits), gu.to_dev_bf16(bits)
    else:
        dev = gu.to_dev_f32(w)
    gu.say(f"mse scales fmt={fmt} dtype={dtype} shape={rows}x{cols}")
    q = mxq.quantize_mse(dev, gu.FMT_ID[fmt])
    want = om.quantize_mse(w, fmt)
    if fmt == "NVFP4":
        assert float(q.tensor_scale.cpu()[0]) == float(want["g"])
    _check(q, want, fmt)


def test_mse_zero_tensor_and_ragged_rows():
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say("mse scales: zero tensor, one-row tensor")
    z = np.zeros((3, 64), np.float32)
    for fmt in ("MXFP4", "NVFP4"):
        q = mxq.quantize_mse(gu.to_dev_f32(z), gu.FMT_ID[fmt])
        _check(q, om.quantize_mse(z, fmt), fmt)
    one = _weights(1, 4096, seed=9)
    for fmt in ("MXFP4", "NVFP4"):
        q = mxq.quantize_mse(gu.to_dev_f32(one), gu.FMT_ID[fmt])
        _check(q, om.quantize_mse(one, fmt), fmt)


@pytest.mark.parametrize("name,fmt", [("svdq_r32", "MXFP4"), ("nvfp4_had16", "NVFP4")])
def test_mse_full_layer_sampled(name, fmt):
    """The 3072x3072 residual weight (MXFP4) and the 12288x3072 weight
    (NVFP4): sampled rows match the oracle's block step under the GPU's tensor
    scale, and the total squared error is below the amax rule's."""
    import fp8_quantized_linear_mxq_amd as mxq
    work = wl.WORKLOADS[name]
    w = wl.weights(work)
    gu.say(f"mse scales full layer {name} {fmt} {w.shape}")
    dev = gu.to_dev_f32(w)
    q = mxq.quantize_mse(dev, gu.FMT_ID[fmt])
    qa = mxq.quantize(dev, gu.FMT_ID[fmt])
    codes, scales = gu.unpack_dev_codes(q, fmt), gu.dev_scales(q, fmt)
    g = float(q.tensor_scale.cpu()[0]) if fmt == "NVFP4" else None
    rows = np.random.default_rng(1).choice(w.shape[0], 24, replace=False)
    sub = w[rows]
    if fmt == "MXFP4":
        s_want, _ = om.mx_block_step(sub)
        c_want = om.quantize_mse(sub, fmt)["codes"]
    else:
        s_want, _ = om.nvfp4_block_step(sub, g)
        c_want = om.nvfp4_elements(sub, s_want, g)
    assert np.array_equal(scales[rows], s_want)
    assert np.array_equal(codes[rows], c_want)

    def total(qd):
        x = {"fmt": fmt, "codes": gu.unpack_dev_codes(qd, fmt), "scales": gu.dev_scales(qd, fmt),
             "g": float(qd.tensor_scale.cpu()[0]) if fmt == "NVFP4" else None}
        d = w.astype(np.float64) - oq.dequantize(x)
        return float(np.einsum("ij,ij->", d, d))
    t_mse, t_amax = total(q), total(qa)
    gu.say(f"  squared error: MSE scales {t_mse:.6g}, amax rule {t_amax:.6g} "
           f"({t_mse / t_amax:.4f})")
    assert t_mse <= t_amax
