"""The im2col reading behind the implicit-im2col convolution, pinned on the CPU.

(1) The im2col layout (K index (ky*3 + kx)*C + c, stride 1, zero padding 1)
times the flattened weights is the 3x3 cross-correlation written out by its
definition.  (2) Quantizing the explicit im2col matrix gives, block for block,
the codes and scales of the quantized input pixel rows, and blocks in the
padding dequantize to zero, for every format (NVFP4 with the dynamic tensor
scale), so gathering the quantized input is the same layer."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import quantize as oq
from tests.test_gpu_conv import _im2col_rows


def _direct_conv(lat, wk):
    """y[y, x, n] = sum over ky, kx, c of lat[y+ky-1, x+kx-1, c] wk[n, c, ky, kx]."""
    h, w, c = lat.shape
    n = wk.shape[0]
    y = np.zeros((h, w, n))
    for yy in range(h):
        for xx in range(w):
            for ky in range(3):
                for kx in range(3):
                    sy, sx = yy + ky - 1, xx + kx - 1
                    if 0 <= sy < h and 0 <= sx < w:
                        y[yy, xx] += wk[:, :, ky, kx] @ lat[sy, sx]
    return y


def test_im2col_is_the_convolution():
    rng = np.random.default_rng(0)
    h, w, c, n = 5, 7, 6, 4
    lat = rng.standard_normal((h, w, c))
    wk = rng.standard_normal((n, c, 3, 3))
    wmat = wk.transpose(0, 2, 3, 1).reshape(n, 9 * c)    # K = (ky*3 + kx)*c + ch
    cols = wl.im2col(lat)
    assert cols.shape == (h * w, 9 * c)
    assert np.allclose(cols @ wmat.T, _direct_conv(lat, wk).reshape(h * w, n), rtol=1e-12,
                       atol=1e-12)
    # the sampled-row gather used by the GPU tests is the same layout
    rows = np.array([0, 3, w, h * w - 1])
    assert np.array_equal(_im2col_rows(lat.astype(np.float32)[None], rows),
                          cols[rows].astype(np.float32))


@pytest.mark.parametrize("fmt", ["MXFP8", "MXFP4", "NVFP4", "INT4"])
def test_quantized_im2col_is_gathered_quantized_input(fmt):
    rng = np.random.default_rng(1)
    h, w, c = 4, 5, 64
    lat = (rng.standard_t(3, size=(h, w, c)) * 163.0 ** rng.random(c)).astype(np.float32)
    lat[0, 0, :32] = 0.0
    pix = lat.reshape(h * w, c)
    g = oq.nvfp4_tensor_scale(pix) if fmt == "NVFP4" else None
    qp = oq.quantize(pix, fmt, tensor_scale=g)
    qi = oq.quantize(wl.im2col(lat), fmt)          # its own dynamic tensor scale
    if fmt == "NVFP4":
        assert float(qi["g"]) == float(g)          # every pixel is some output's centre tap
    blk = oq.BLOCK[fmt]
    deq_i = oq.dequantize(qi)
    for m in range(h * w):
        y, x = divmod(m, w)
        for ky in range(3):
            for kx in range(3):
                k0 = (ky * 3 + kx) * c
                sy, sx = y + ky - 1, x + kx - 1
                if 0 <= sy < h and 0 <= sx < w:
                    src = sy * w + sx
                    assert np.array_equal(qi["codes"][m, k0:k0 + c], qp["codes"][src])
                    assert np.array_equal(qi["scales"][m, k0 // blk:(k0 + c) // blk],
                                          qp["scales"][src])
                else:
                    assert not np.any(deq_i[m, k0:k0 + c])
