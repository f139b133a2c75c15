"""GPU parity of the implicit-im2col 3x3 convolution (mxq_conv3x3_gemm_mixed).

The GPU quantizes only the input's pixel rows and gathers the nine taps
inside the GEMM.  The oracle follows the layer as the Chameleon article
states it for its concatenated-feature convolutions: the explicit im2col
matrix (K index (ky*3 + kx)*C + c, zero padding 1) quantized to the
activation format, times the dequantized weight groups.  Outputs are checked
under the GEMM bound; the activation codes are checked bit for bit against
the oracle on the pixel rows."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import quantize as oq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _latent(images, h, w, c, seed):
    """bf16 bits [images, h, w, c]: Student-t(3) times a per-channel spread
    up to 163x (the concatenated-feature input's shape of distribution)."""
    rng = np.random.default_rng(seed)
    spread = 163.0 ** rng.random(c)
    lat = rng.standard_t(3, size=(images, h, w, c)) * spread
    lat[0, 0, 0, :64] = 0.0                      # all-zero blocks in a corner pixel
    return wl.f32_to_bf16_bits(lat.astype(np.float32))


def _im2col_rows(lat_vals, rows):
    """Rows of the explicit im2col of [images, h, w, c] float values for the
    given output pixels: [len(rows), 9c], zero outside the image."""
    images, h, w, c = lat_vals.shape
    out = np.zeros((len(rows), 9 * c), dtype=np.float32)
    for i, m in enumerate(rows):
        img, rem = divmod(int(m), h * w)
        y, x = divmod(rem, w)
        for ky in range(3):
            for kx in range(3):
                yy, xx = y + ky - 1, x + kx - 1
                if 0 <= yy < h and 0 <= xx < w:
                    out[i, (ky * 3 + kx) * c:(ky * 3 + kx + 1) * c] = lat_vals[img, yy, xx]
    return out


def _groups(wd, wt, assign, fmts):
    """Weight rows grouped by format (row r -> fmts[assign[r]]), quantized on
    the GPU (NVFP4 with its group's own dynamic tensor scale); returns the
    groups, the device permutation and the host row lists."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    groups, idx_all = [], []
    for gi, f in enumerate(fmts):
        idx = np.nonzero(assign == gi)[0]
        idx_all.append(idx)
        if len(idx):
            sub = wd.index_select(0, torch.from_numpy(idx.astype(np.int64)).cuda()).contiguous()
            groups.append(mxq.quantize(sub, gu.FMT_ID[f]))
        else:
            groups.append(mxq.empty_qtensor(gu.FMT_ID[f], 0, wt.shape[1]))
    perm = torch.from_numpy(np.concatenate(idx_all).astype(np.int32)).cuda()
    return groups, perm, idx_all


def _conv_check(lat_bits, wt, act_fmt, fmts, assign, rows=None, bias_bits=None, tag=""):
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    images, h, w, c = lat_bits.shape
    m, n = images * h * w, wt.shape[0]
    assert wt.shape[1] == 9 * c
    xd = gu.to_dev_bf16(lat_bits.reshape(m, c))
    wd = gu.to_dev_f32(wt)
    groups, perm, idx_all = _groups(wd, wt, assign, fmts)
    bias = gu.to_dev_bf16(bias_bits) if bias_bits is not None else None
    gu.say(f"{tag}: conv {images}x{h}x{w}x{c} -> {n}, act {act_fmt}, groups "
           f"{[(f, len(i)) for f, i in zip(fmts, idx_all)]}")
    qx = mxq.quantize(xd, gu.FMT_ID[act_fmt])
    y = mxq.conv3x3_gemm_mixed(qx, h, w, groups, perm, n, bias=bias)
    torch.cuda.synchronize()
    gu.say(f"{tag}: device work done; checking")

    lat_vals = wl.bf16_to_f32(lat_bits)
    rows = np.arange(m) if rows is None else rows
    # activation codes of the pixel rows (the NVFP4 tensor scale is the
    # whole input's, which is also the whole im2col matrix's)
    g_a = oq.nvfp4_tensor_scale(lat_vals.reshape(m, c)) if act_fmt == "NVFP4" else None
    if act_fmt == "NVFP4":
        assert float(qx.tensor_scale.cpu()[0]) == float(g_a)
    qp_ref = oq.quantize(lat_vals.reshape(m, c)[rows], act_fmt, tensor_scale=g_a)
    got_c = gu.unpack_dev_codes(qx, act_fmt)[rows]
    got_s = gu.dev_scales(qx, act_fmt)[rows]
    assert np.array_equal(got_s, qp_ref["scales"]), f"{tag}: input scales differ"
    assert np.array_equal(got_c, qp_ref["codes"]), f"{tag}: input codes differ"
    # the oracle's layer: quantize the explicit im2col rows, then the GEMM
    qa_ref = oq.quantize(_im2col_rows(lat_vals, rows), act_fmt, tensor_scale=g_a)
    a_deq = gu.dequant_a_for_gemm(qa_ref)
    bias_vals = wl.bf16_to_f32(bias_bits).astype(np.float64) if bias_bits is not None else None
    worst = 0.0
    for f, idx in zip(fmts, idx_all):
        if len(idx) == 0:
            continue
        qw_ref = oq.quantize(wt[idx], f)
        r = gu.check_gemm(y, a_deq, gu.dequant_w_for_gemm(qw_ref), gu.alpha_of(qa_ref, qw_ref),
                          bias=None if bias_vals is None else bias_vals[idx],
                          rows=rows, cols=idx, tag=f"{tag} {f}")
        worst = max(worst, r)
    gu.say(f"{tag}: worst err/tol {worst:.3g}")


CASES = [
    # (act, weight formats, images, h, w, c, n, seed)
    ("MXFP8", ("INT4", "MXFP4", "NVFP4"), 2, 11, 13, 256, 150, 1),   # ragged M and N tiles
    ("NVFP4", ("NVFP4", "INT4", "MXFP4"), 1, 9, 17, 256, 70, 2),
    ("MXFP4", ("NVFP4", "INT4"), 2, 5, 7, 128, 40, 3),               # one K-tile per tap
    ("MXFP8", ("MXFP4", "NVFP4", "INT4"), 1, 6, 23, 640, 130, 4),    # K = 5760: slab accumulation
    ("MXFP8", ("NVFP4", "INT4"), 3, 1, 40, 128, 64, 5),              # one image row: dy taps all zero
    ("MXFP8", ("MXFP4",), 2, 12, 1, 256, 33, 6),                     # one image column
    ("MXFP8", ("INT4",), 1, 48, 48, 128, 2000, 7),                   # 288 INT4 tiles: wide grid
    ("MXFP8", ("INT4",), 1, 48, 48, 384, 2000, 8),                   # wide grid, 54 K-tiles: slabs
    ("MXFP8", ("NVFP4", "INT4"), 5, 1, 1, 128, 40, 9),               # 1x1 images: centre tap only
]


@pytest.mark.parametrize("act_fmt,fmts,images,h,w,c,n,seed", CASES)
def test_conv_matches_oracle(act_fmt, fmts, images, h, w, c, n, seed):
    lat = _latent(images, h, w, c, seed)
    wt = wl.mixed_weights(9 * c, n, seed=seed)
    assign = np.arange(n) % len(fmts)
    rng = np.random.default_rng(seed)
    bias = wl.f32_to_bf16_bits(rng.normal(0, 1, size=n).astype(np.float32)) if seed % 2 else None
    m = images * h * w
    rows = None
    if m > 1024:   # sampled pixels, corners and edges included
        rows = np.unique(np.concatenate([[0, w - 1, m - w, m - 1, w, 2 * w - 1],
                                         rng.choice(m, 64, replace=False)]))
    _conv_check(lat, wt, act_fmt, fmts, assign, rows=rows, bias_bits=bias, tag=f"conv{seed}")


def test_conv_single_group_without_permutation():
    """One weight group and no permutation: row j writes column j; an INT4
    group narrow enough to split K over the workspace, run twice (split and
    unsplit) with the same result within the bound."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    lat = _latent(1, 16, 16, 256, 9)
    wt = wl.mixed_weights(9 * 256, 20, seed=9)
    xd = gu.to_dev_bf16(lat.reshape(256, 256))
    qx = mxq.quantize(xd, mxq.MXFP8)
    qw = mxq.quantize(gu.to_dev_f32(wt), mxq.INT4)
    gu.say("conv: single INT4 group, no permutation, split and unsplit K")
    y_split = mxq.conv3x3_gemm_mixed(qx, 16, 16, [qw], None, 20)
    y_plain = mxq.conv3x3_gemm_mixed(qx, 16, 16, [qw], None, 20, workspace=False)
    torch.cuda.synchronize()
    lat_vals = wl.bf16_to_f32(lat)
    rows = np.arange(256)
    qa_ref = oq.quantize(_im2col_rows(lat_vals, rows), "MXFP8")
    qw_ref = oq.quantize(wt, "INT4")
    for y in (y_split, y_plain):
        gu.check_gemm(y, oq.dequantize(qa_ref), oq.dequantize(qw_ref), 1.0, tag="conv int4")


def test_conv_full_layer_sampled():
    """The convolution layer at full size (128 x 128 x 2560 input, 1280
    outputs, K = 23040) through the implicit im2col, with the format groups
    chosen on the GPU; outputs checked on sampled pixels, corners and edges
    included."""
    import fp8_quantized_linear_mxq_amd as mxq
    w = wl.WORKLOADS["chameleon_conv"]
    h, wd_, c = w.extra["latent"]
    lat = wl.conv_latent(w).reshape(1, h, wd_, c)
    wt = wl.weights(w)
    gu.say("conv full layer: selection")
    choice, _, _, _, _ = mxq.select_format(gu.to_dev_f32(wt))
    assign = choice.cpu().numpy().astype(np.int64)
    rng = np.random.default_rng(11)
    edge = [0, wd_ - 1, (h - 1) * wd_, h * wd_ - 1, 5, 7 * wd_, 9 * wd_ + wd_ - 1]
    rows = np.unique(np.concatenate([edge, rng.choice(h * wd_, size=40, replace=False)]))
    _conv_check(lat, wt, "MXFP8", ("INT4", "MXFP4", "NVFP4"), assign, rows=rows, tag="conv full")


def test_conv_rejects():
    """Host-side errors of the convolution entry point (nothing launched)."""
    import fp8_quantized_linear_mxq_amd as mxq
    lat = _latent(1, 4, 4, 128, 12)
    qx = mxq.quantize(gu.to_dev_bf16(lat.reshape(16, 128)), mxq.MXFP4)
    qw4 = mxq.quantize(gu.to_dev_f32(wl.mixed_weights(9 * 128, 8, seed=1)), mxq.MXFP4)
    with pytest.raises(mxq.MxqError) as ei:     # MXFP4 x MXFP4 has no im2col reader
        mxq.conv3x3_gemm_mixed(qx, 4, 4, [qw4], None, 8)
    assert ei.value.status == 2
    with pytest.raises(mxq.MxqError) as ei:     # 16 pixel rows are not whole 3x3 images
        mxq.conv3x3_gemm_mixed(qx, 3, 3, [qw4], None, 8)
    assert ei.value.status == 4
