"""GPU parity: mxq_gemm on every supported (activation, weight) format pair,
with and without bias, low-rank branch and column map, ragged M/N and long
K, against the float64 oracle under the stated error bound.  Operands are the
oracle's own codes, uploaded, so the GEMM is checked in isolation."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import quantize as oq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ROUTES = [(a, w) for a in ("MXFP4", "MXFP8", "NVFP4") for w in ("MXFP4", "NVFP4", "INT4")]


def _operands(m, n, k, fa, fw, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_t(3, size=(m, k)) * 2.0
    a[:, rng.choice(k, size=max(1, k // 200), replace=False)] *= 50.0   # hot channels
    a = a.astype(np.float32)
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    qa = oq.quantize(a, fa)
    qw = oq.quantize(w, fw)
    return qa, qw


@pytest.mark.parametrize("variant", ["plain", "bias_lr", "colmap"])
@pytest.mark.parametrize("fa,fw", ROUTES)
def test_gemm_routes(fa, fw, variant):
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 200, 300, 640
    gu.say(f"gemm {fa}x{fw} {variant} M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, fa, fw, seed=len(fa) * 7 + len(fw) + len(variant))
    a_dev = gu.qtensor_from_oracle(qa, m, k)
    w_dev = gu.qtensor_from_oracle(qw, n, k)
    a_deq = gu.dequant_a_for_gemm(qa)
    w_deq = gu.dequant_w_for_gemm(qw)
    alpha = gu.alpha_of(qa, qw)
    rng = np.random.default_rng(3)
    if variant == "plain":
        y = mxq.gemm(a_dev, w_dev)
        gu.check_gemm(y, a_deq, w_deq, alpha, tag=f"{fa}x{fw}")
    elif variant == "bias_lr":
        r = 32
        u = (rng.standard_normal((m, r)) * 4).astype(np.float32)
        l2 = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 0.02, (r, n)).astype(np.float32)))
        bias = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 1, n).astype(np.float32)))
        y = mxq.gemm(a_dev, w_dev, u=gu.to_dev_f32(u),
                     l2t=gu.to_dev_bf16(wl.f32_to_bf16_bits(np.ascontiguousarray(l2.T))),
                     bias=gu.to_dev_bf16(wl.f32_to_bf16_bits(bias)))
        # the low-rank term's bound: sum_j |u_j| |L2_jn| (u is given exactly here)
        gu.check_gemm(y, np.hstack([a_deq, u.astype(np.float64)]),
                      np.hstack([w_deq, l2.T.astype(np.float64) / alpha]), alpha,
                      bias=bias, tag=f"{fa}x{fw} lr")
    else:
        n_out = n + 20
        perm = rng.permutation(n_out)[:n].astype(np.int32)
        out = torch.full((m, n_out), -7.0, dtype=torch.bfloat16, device="cuda")
        y = mxq.gemm(a_dev, w_dev, n_out=n_out,
                     w_out_col=torch.from_numpy(perm).cuda(), out=out)
        yh = y.float().cpu().numpy()
        untouched = np.setdiff1d(np.arange(n_out), perm)
        assert np.all(yh[:, untouched] == -7.0)
        gu.check_gemm(y, a_deq, w_deq, alpha, cols=perm, tag=f"{fa}x{fw} colmap")


@pytest.mark.parametrize("fa,fw", ROUTES)
def test_gemm_long_k(fa, fw):
    """K = 8192 exercises the fp32 slab accumulation of every route."""
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 64, 96, 8192
    gu.say(f"gemm long K {fa}x{fw} M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, fa, fw, seed=11)
    y = mxq.gemm(gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k))
    r = gu.check_gemm(y, gu.dequant_a_for_gemm(qa), gu.dequant_w_for_gemm(qw),
                      gu.alpha_of(qa, qw), tag=f"{fa}x{fw} longK")
    gu.say(f"  worst err/tol {r:.3g}")


def test_gemm_errors():
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say("gemm argument errors")
    qa, qw = _operands(8, 8, 128, "INT4", "MXFP4", seed=1)
    with pytest.raises(mxq.MxqError) as ei:
        mxq.gemm(gu.qtensor_from_oracle(qa, 8, 128), gu.qtensor_from_oracle(qw, 8, 128))
    assert ei.value.status == 2                      # INT4 activations: unsupported
    a160 = mxq.empty_qtensor(mxq.MXFP4, 8, 160)      # padded, aligned row strides
    w160 = mxq.empty_qtensor(mxq.MXFP4, 8, 160)
    with pytest.raises(mxq.MxqError) as ei:
        mxq.gemm(a160, w160)
    assert ei.value.status == 4                      # K not a multiple of 128
    # M = 0 is a no-op
    qa, qw = _operands(1, 8, 128, "MXFP4", "MXFP4", seed=1)
    a0 = gu.qtensor_from_oracle(qa, 1, 128)
    a0.rows = 0
    out = torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda")
    mxq.gemm(a0, gu.qtensor_from_oracle(qw, 8, 128), out=out)


# Shapes that make the MXFP4 x MXFP4 route pick each of its workgroup tiles
# (64x64 below 128 tiles of 128x128, 128x128, 256x192, 256x256, and the
# slab-accumulating 128x128 past K = 4096 with a half K-tile at the end), all
# with ragged M and N tails.
MX_TILE_SHAPES = [(130, 250, 384), (1500, 1400, 256), (2000, 2300, 256), (4000, 4000, 256),
                  (96, 130, 4224)]


@pytest.mark.parametrize("m,n,k", MX_TILE_SHAPES)
def test_gemm_mx_tiles(m, n, k):
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say(f"gemm MXFP4xMXFP4 tiles M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, "MXFP4", "MXFP4", seed=m + n)
    rng = np.random.default_rng(5)
    r = 32
    u = (rng.standard_normal((m, r)) * 4).astype(np.float32)
    l2 = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 0.02, (r, n)).astype(np.float32)))
    y = mxq.gemm(gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k),
                 u=gu.to_dev_f32(u),
                 l2t=gu.to_dev_bf16(wl.f32_to_bf16_bits(np.ascontiguousarray(l2.T))))
    a_deq = np.hstack([gu.dequant_a_for_gemm(qa), u.astype(np.float64)])
    w_deq = np.hstack([gu.dequant_w_for_gemm(qw), l2.T.astype(np.float64)])
    ratio = gu.check_gemm(y, a_deq, w_deq, 1.0, tag=f"mx tiles {m}x{n}x{k}")
    gu.say(f"  worst err/tol {ratio:.3g}")


# Shapes that make the dequantizing route pick its 256-row workgroup tiles:
# 256x128 (four waves), 256x192 and 256x256 (eight waves) at K = 2048, and
# 256x192 at a short K (9 K-tiles) where it fills whole rounds; ragged M and
# N tails; output rows are checked on a sample.
DQ_TILE_SHAPES = [(2000, 2300, 2048), (4000, 2300, 2048), (4000, 4000, 2048), (4096, 3072, 1152)]
DQ_PAIRS = [(a, w) for a in ("MXFP8", "NVFP4", "MXFP4") for w in ("MXFP4", "NVFP4")
            if (a, w) != ("MXFP4", "MXFP4")]


@pytest.mark.parametrize("m,n,k", DQ_TILE_SHAPES)
@pytest.mark.parametrize("fa,fw", DQ_PAIRS)
def test_gemm_dq_tiles(fa, fw, m, n, k):
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say(f"gemm {fa}x{fw} tiles M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, fa, fw, seed=m + 3 * n + len(fa + fw))
    y = mxq.gemm(gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k))
    rng = np.random.default_rng(m + n)
    rows = np.unique(np.concatenate([rng.choice(m, 96, replace=False), [0, 255, 256, m - 1]]))
    a_deq = gu.dequant_a_for_gemm(qa)[rows]
    ratio = gu.check_gemm(y, a_deq, gu.dequant_w_for_gemm(qw), gu.alpha_of(qa, qw), rows=rows,
                          tag=f"{fa}x{fw} tiles {m}x{n}x{k}")
    gu.say(f"  worst err/tol {ratio:.3g}")


@pytest.mark.parametrize("fa,fw", [("MXFP8", "NVFP4"), ("MXFP4", "NVFP4"), ("MXFP8", "MXFP4")])
def test_gemm_dq_wide_tiles_lowrank(fa, fw):
    """256x256 workgroup tiles (eight waves; 128x64 wave tiles for NVFP4 weights against MX
    activations, 64x128 otherwise) with the low-rank branch and bias in the epilogue; ragged
    M and N; output rows checked on a sample that includes both tile rows of a workgroup."""
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 4000, 4000, 2048
    gu.say(f"gemm {fa}x{fw} 256x256 tiles + low rank M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, fa, fw, seed=17 + len(fa + fw))
    rng = np.random.default_rng(23)
    r = 32
    u = (rng.standard_normal((m, r)) * 4).astype(np.float32)
    l2 = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 0.02, (r, n)).astype(np.float32)))
    bias = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 1, n).astype(np.float32)))
    y = mxq.gemm(gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k),
                 u=gu.to_dev_f32(u),
                 l2t=gu.to_dev_bf16(wl.f32_to_bf16_bits(np.ascontiguousarray(l2.T))),
                 bias=gu.to_dev_bf16(wl.f32_to_bf16_bits(bias)))
    rows = np.unique(np.concatenate([rng.choice(m, 80, replace=False),
                                     [0, 127, 128, 255, 256, 3839, 3840, m - 1]]))
    alpha = gu.alpha_of(qa, qw)
    a_deq = np.hstack([gu.dequant_a_for_gemm(qa)[rows], u[rows].astype(np.float64)])
    w_deq = np.hstack([gu.dequant_w_for_gemm(qw), l2.T.astype(np.float64) / alpha])
    ratio = gu.check_gemm(y, a_deq, w_deq, alpha, bias=bias, rows=rows,
                          tag=f"{fa}x{fw} 256x256 lr")
    gu.say(f"  worst err/tol {ratio:.3g}")


@pytest.mark.parametrize("fa", ["MXFP8", "NVFP4", "MXFP4"])
def test_int4_split_k(fa):
    """Narrow INT4 weight groups (few output tiles) split K into fp32 partial
    sums when a workspace is given, summed in a fixed order by a second
    kernel with the alpha, bias and column map of the epilogue.  Both paths
    meet the tolerance; the split one is deterministic.  K = 4224 gives 66
    K-tiles of 64 over four splits (17, 17, 17, 15)."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 300, 20, 4224
    gu.say(f"gemm {fa}xINT4 split K M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, fa, "INT4", seed=77)
    a_dev, w_dev = gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k)
    assert mxq.workspace_size(mxq.OP_GEMM, m, n, mxq.INT4) == 16 * m * n * 4
    rng = np.random.default_rng(9)
    n_out = 40
    perm = rng.permutation(n_out)[:n].astype(np.int32)
    bias = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 1, n_out).astype(np.float32)))
    bias_dev = gu.to_dev_bf16(wl.f32_to_bf16_bits(bias))
    perm_dev = torch.from_numpy(perm).cuda()
    ys = []
    for ws in (False, None, None):
        out = torch.full((m, n_out), -7.0, dtype=torch.bfloat16, device="cuda")
        ys.append(mxq.gemm(a_dev, w_dev, n_out=n_out, w_out_col=perm_dev, bias=bias_dev, out=out,
                           workspace=ws))
    a_deq, w_deq = gu.dequant_a_for_gemm(qa), gu.dequant_w_for_gemm(qw)
    alpha = gu.alpha_of(qa, qw)
    untouched = np.setdiff1d(np.arange(n_out), perm)
    for y, tag in zip(ys, ("unsplit", "split", "split again")):
        assert np.all(y.float().cpu().numpy()[:, untouched] == -7.0)
        gu.check_gemm(y, a_deq, w_deq, alpha, bias=bias[perm], cols=perm, tag=f"{fa}xINT4 {tag}")
    assert torch.equal(ys[1], ys[2])


@pytest.mark.parametrize("fa,k", [("MXFP8", 256), ("NVFP4", 256), ("MXFP4", 256),
                                  ("MXFP8", 4224)])
def test_int4_wide_grid_lowrank(fa, k):
    """INT4 weights over more than one workgroup per compute unit (288 tiles:
    one K-tile in flight per workgroup, where the small grids above keep two)
    with bias and the rank-32 branch; K = 256 runs without fp32 slabs (two
    workgroups per compute unit), K = 4224 with them; sampled rows."""
    import fp8_quantized_linear_mxq_amd as mxq
    m, n = 2048, 2304
    gu.say(f"gemm {fa}xINT4 wide grid + low rank M={m} N={n} K={k}")
    qa, qw = _operands(m, n, k, fa, "INT4", seed=123)
    rng = np.random.default_rng(6)
    r = 32
    u = (rng.standard_normal((m, r)) * 4).astype(np.float32)
    l2 = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 0.02, (r, n)).astype(np.float32)))
    bias = wl.bf16_to_f32(wl.f32_to_bf16_bits(rng.normal(0, 1, n).astype(np.float32)))
    y = mxq.gemm(gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k),
                 u=gu.to_dev_f32(u),
                 l2t=gu.to_dev_bf16(wl.f32_to_bf16_bits(np.ascontiguousarray(l2.T))),
                 bias=gu.to_dev_bf16(wl.f32_to_bf16_bits(bias)))
    rows = np.unique(np.concatenate([rng.choice(m, 64, replace=False), [0, m - 1]]))
    alpha = gu.alpha_of(qa, qw)
    a_deq = np.hstack([gu.dequant_a_for_gemm(qa)[rows], u[rows].astype(np.float64)])
    w_deq = np.hstack([gu.dequant_w_for_gemm(qw), l2.T.astype(np.float64) / alpha])
    ratio = gu.check_gemm(y, a_deq, w_deq, alpha, bias=bias, rows=rows, tag=f"{fa}xINT4 wide")
    gu.say(f"  worst err/tol {ratio:.3g}")


def _tiny_operands(m, n, k, fa, fw, seed):
    """Activations whose 32-blocks have amax anywhere in 2**-127 .. 2**-110
    (rows 0-15: every block; rows 16-31: every other block, the rest normal;
    row 0's first block at exactly 2**-127, so E4M3 / E2M1 codes reach their
    subnormal and smallest values), and weights with a few such rows."""
    rng = np.random.default_rng(seed)
    a = rng.standard_t(3, size=(m, k)) * 2.0
    nb = k // 32
    e = rng.integers(-127, -109, size=(32, nb)).astype(np.float64)
    blk = a[:32].reshape(32, nb, 32)
    amax = np.abs(blk).max(axis=2, keepdims=True)
    tiny = blk / amax * 2.0 ** e[:, :, None]
    tiny[16:, 1::2] = blk[16:, 1::2]                  # rows 16-31: every other block normal
    tiny[0, 0] = blk[0, 0] / amax[0, 0] * 2.0 ** -127
    a[:32] = tiny.reshape(32, k)
    a = a.astype(np.float32)
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    w[5] *= 2.0 ** -110
    w[7, :64] *= 2.0 ** -100
    return oq.quantize(a, fa), oq.quantize(w, fw)


@pytest.mark.parametrize("fa,fw", ROUTES)
def test_gemm_tiny_block_scales(fa, fw):
    """Blocks with amax down to 2**-127 (E8M0 codes near 0) on every route:
    the MX dequantization must stay exact there (code 0 is 2**-127, and E4M3
    values times a tiny scale must not underflow)."""
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 64, 96, 512
    gu.say(f"gemm tiny scales {fa}x{fw} M={m} N={n} K={k}")
    qa, qw = _tiny_operands(m, n, k, fa, fw, seed=29)
    if fa != "NVFP4":
        assert qa["scales"].min() == 0          # a code-0 block is present
    y = mxq.gemm(gu.qtensor_from_oracle(qa, m, k), gu.qtensor_from_oracle(qw, n, k))
    a_deq = gu.dequant_a_for_gemm(qa)
    ref = np.abs(a_deq[:16] @ gu.dequant_w_for_gemm(qw).T)
    if fa != "NVFP4":
        # the tiny rows' outputs are far above the tolerance's absolute floor
        assert np.median(ref) > 2.0 ** -126
    r = gu.check_gemm(y, a_deq, gu.dequant_w_for_gemm(qw), gu.alpha_of(qa, qw),
                      tag=f"{fa}x{fw} tiny")
    gu.say(f"  worst err/tol {r:.3g}")


def _every_e4m3_scale(rows, k, seed):
    """Values whose 16-blocks, quantized to NVFP4 with the static tensor
    scale g = 1, take every E4M3 block-scale code 0 .. 126 in turn (the
    subnormal codes 1 .. 7 included): block b's amax is 6 * E4M3(b % 127)."""
    from oracle import formats as of
    rng = np.random.default_rng(seed)
    x = rng.uniform(-1.0, 1.0, size=(rows, k // 16, 16))
    code = np.arange(rows * (k // 16)).reshape(rows, k // 16) % 127
    amax = 6.0 * np.vectorize(of.e4m3_value)(code).astype(np.float64)
    x[:, :, 0] = np.where(rng.random((rows, k // 16)) < 0.5, -1.0, 1.0)   # |max| = 1 exactly
    return (x * amax[:, :, None]).reshape(rows, k).astype(np.float32), code


@pytest.mark.parametrize("fa,fw", [("NVFP4", "NVFP4"), ("MXFP8", "NVFP4"), ("MXFP4", "NVFP4"),
                                   ("NVFP4", "MXFP4"), ("NVFP4", "INT4")])
def test_gemm_every_e4m3_block_scale(fa, fw):
    """The NVFP4 operand's block scales cover every E4M3 code (subnormal
    ones too), decoded in the GEMM by the hardware FP8 converts: results
    within the bound on every route that reads NVFP4 scales."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    m, n, k = 48, 40, 512
    gu.say(f"gemm every E4M3 block scale {fa}x{fw} M={m} N={n} K={k}")
    rng = np.random.default_rng(31)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    if fa == "NVFP4":
        a, code = _every_e4m3_scale(m, k, seed=5)
        qa_dev = mxq.quantize(gu.to_dev_f32(a), mxq.NVFP4, static_tensor_scale=one)
        qa = oq.quantize(a, "NVFP4", tensor_scale=1.0)
        assert np.array_equal(qa["scales"], code)            # every code present
    else:
        a = (rng.standard_t(3, size=(m, k)) * 2.0).astype(np.float32)
        qa = oq.quantize(a, fa)
        qa_dev = gu.qtensor_from_oracle(qa, m, k)
    if fw == "NVFP4":
        w, code = _every_e4m3_scale(n, k, seed=6)
        qw_dev = mxq.quantize(gu.to_dev_f32(w), mxq.NVFP4, static_tensor_scale=one)
        qw = oq.quantize(w, "NVFP4", tensor_scale=1.0)
        assert np.array_equal(qw["scales"], code)
    else:
        w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
        qw = oq.quantize(w, fw)
        qw_dev = gu.qtensor_from_oracle(qw, n, k)
    y = mxq.gemm(qa_dev, qw_dev)
    r = gu.check_gemm(y, gu.dequant_a_for_gemm(qa), gu.dequant_w_for_gemm(qw), gu.alpha_of(qa, qw),
                      tag=f"{fa}x{fw} every E4M3 scale")
    gu.say(f"  worst err/tol {r:.3g}")
