"""GPU parity of the 4-bit-weight, 16-bit-activation GEMM (mxq_gemm with an
unquantized bf16 activation operand; the Nunchaku article's second kernel
type, for adaptive-normalization layers) against the float64 oracle: the
activations are taken exactly (bf16 values), the weights dequantized from
the oracle's codes; the same bound as every GEMM route."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import quantize as oq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _operands(m, n, k, fw, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_t(3, size=(m, k)) * 2.0
    a[:, rng.choice(k, size=max(1, k // 200), replace=False)] *= 50.0   # hot channels
    a_bits = wl.f32_to_bf16_bits(a.astype(np.float32))
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    return a_bits, oq.quantize(w, fw)


# ragged M/N over 128x128 tiles, one K-tile, slab accumulation past 32 K-tiles
SHAPES = [(200, 300, 640), (130, 129, 128), (96, 160, 8192)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("fw", ["MXFP4", "NVFP4", "INT4"])
def test_w4a16(fw, m, n, k):
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say(f"gemm bf16x{fw} M={m} N={n} K={k}")
    a_bits, qw = _operands(m, n, k, fw, seed=m + n + k + len(fw))
    a_dev = mxq.bf16_operand(gu.to_dev_bf16(a_bits))
    y = mxq.gemm(a_dev, gu.qtensor_from_oracle(qw, n, k))
    a_vals = wl.bf16_to_f32(a_bits).astype(np.float64)
    ratio = gu.check_gemm(y, a_vals, gu.dequant_w_for_gemm(qw), gu.alpha_of({"fmt": "BF16"}, qw),
                          tag=f"bf16x{fw}")
    gu.say(f"  worst err/tol {ratio:.3g}")


@pytest.mark.parametrize("fw", ["MXFP4", "NVFP4", "INT4"])
def test_w4a16_bias_lowrank_colmap_strided(fw):
    """Bias, the rank-32 branch, an output column map and an activation row
    stride wider than K, on one call."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 150, 200, 512
    gu.say(f"gemm bf16x{fw} with bias, low-rank branch, column map, strided rows")
    rng0 = np.random.default_rng(31)
    a_bits = wl.f32_to_bf16_bits((rng0.standard_t(3, size=(m, k + 64)) * 2).astype(np.float32))
    qw = oq.quantize(rng0.normal(0, 0.02, size=(n, k)).astype(np.float32), fw)
    x_full = gu.to_dev_bf16(a_bits)                 # [m, k + 64]: row stride k + 64
    a_dev = mxq.bf16_operand(x_full[:, :k])
    rng = np.random.default_rng(4)
    r = 32
    u = (rng.standard_normal((m, r)) * 4).astype(np.float32)
    l2 = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 0.02, (r, n + 10)).astype(np.float32)))
    bias = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 1, n + 10).astype(np.float32)))
    n_out = n + 10
    perm = rng.permutation(n_out)[:n].astype(np.int32)
    out = torch.full((m, n_out), -7.0, dtype=torch.bfloat16, device="cuda")
    y = mxq.gemm(a_dev, gu.qtensor_from_oracle(qw, n, k), n_out=n_out,
                 w_out_col=torch.from_numpy(perm).cuda(), u=gu.to_dev_f32(u),
                 l2t=gu.to_dev_bf16(wl.f32_to_bf16_bits(np.ascontiguousarray(l2.T))),
                 bias=gu.to_dev_bf16(wl.f32_to_bf16_bits(bias)), out=out)
    untouched = np.setdiff1d(np.arange(n_out), perm)
    assert np.all(y.float().cpu().numpy()[:, untouched] == -7.0)
    a_vals = wl.bf16_to_f32(a_bits[:, :k]).astype(np.float64)
    alpha = gu.alpha_of({"fmt": "BF16"}, qw)
    # the low-rank term enters the bound as sum_j |u_j| |L2_jn| (u given exactly)
    gu.check_gemm(y, np.hstack([a_vals, u.astype(np.float64)]),
                  np.hstack([gu.dequant_w_for_gemm(qw), l2.T[perm].astype(np.float64) / alpha]),
                  alpha, bias=bias[perm], cols=perm, tag=f"bf16x{fw} full epilogue")


def test_w4a16_rejects():
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say("bf16 operand errors")
    a_bits, qw = _operands(8, 8, 128, "MXFP4", seed=1)
    a_dev = mxq.bf16_operand(gu.to_dev_bf16(a_bits))
    with pytest.raises(mxq.MxqError) as ei:          # bf16 is not a weight format
        mxq.gemm(gu.qtensor_from_oracle(qw, 8, 128), a_dev)
    assert ei.value.status == 2
    a96 = mxq.bf16_operand(gu.to_dev_bf16(np.zeros((8, 96), np.uint16)))
    w96 = mxq.empty_qtensor(mxq.MXFP4, 8, 96)
    with pytest.raises(mxq.MxqError) as ei:          # K not a multiple of 128
        mxq.gemm(a96, w96)
    assert ei.value.status == 4


@pytest.mark.parametrize("name", ["w4a16_mlp", "w4a16_mx_mlp"])
def test_w4a16_workload_full_size(name):
    """The benchmarked layers at full size (4096 x 1152 x 4608, bf16
    activations, INT4 or MXFP4 weights quantized on the GPU): weight codes
    and scales bit-exact, outputs checked on sampled rows."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    w = wl.WORKLOADS[name]
    gu.say(f"workload {w.name}: M={w.m} K={w.k} N={w.n} bf16 x {w.w_fmt}")
    act = wl.activations(w)
    wt = wl.weights(w)
    qw = mxq.quantize(gu.to_dev_f32(wt), gu.FMT_ID[w.w_fmt])
    y = mxq.gemm(mxq.bf16_operand(gu.to_dev_bf16(act)), qw)
    torch.cuda.synchronize()
    qw_ref = oq.quantize(wt, w.w_fmt)
    assert np.array_equal(gu.dev_scales(qw, w.w_fmt), qw_ref["scales"])
    assert np.array_equal(gu.unpack_dev_codes(qw, w.w_fmt), qw_ref["codes"])
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(w.m, 96, replace=False), [0, w.m - 1]]))
    a_vals = wl.bf16_to_f32(act[rows]).astype(np.float64)
    r = gu.check_gemm(y, a_vals, gu.dequant_w_for_gemm(qw_ref), 1.0, rows=rows, tag=w.name)
    gu.say(f"  {w.name}: worst err/tol {r:.3g}")
