"""mxq_quantize_noalloc (through the C ABI) against mxq_quantize: identical
codes, scales and NVFP4 tensor scale, on two calls in a row, the second with
a smaller input (the scratch array keeps the first call's partials)."""
import ctypes as C

import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import _lib
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [  # (fmt, hadamard, dtype)
    ("NVFP4", 0, "bf16"), ("NVFP4", 16, "bf16"), ("NVFP4", 128, "f32"), ("MXFP4", 0, "f32"),
    ("MXFP8", 32, "bf16"), ("INT4", 0, "f32"),
]


def _noalloc(lib, x, fmt, had, out, stream):
    import torch
    dt = _lib.DT_BF16 if x.dtype == torch.bfloat16 else _lib.DT_F32
    qc = out.c()
    st = lib.mxq_quantize_noalloc(C.c_void_p(x.data_ptr()), dt, x.shape[0], x.shape[1],
                                  x.stride(0), had, None, None, 0, None, 0, C.byref(qc),
                                  C.c_void_p(stream.cuda_stream))
    assert st == 0, _lib.STATUS.get(st, st)


@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("fmt,had,dtype", CASES)
def test_noalloc_matches_quantize(lib, fmt, had, dtype, two_pass, monkeypatch):
    """Dynamic NVFP4 takes the one-pass kernel (barrier slots) by default; with
    MXQ_NVFP4_TWO_PASS=1 its amax partials go through the scratch array."""
    import torch
    if two_pass:
        if fmt != "NVFP4":
            pytest.skip("the two passes concern the dynamic NVFP4 scale only")
        monkeypatch.setenv("MXQ_NVFP4_TWO_PASS", "1")

    import fp8_quantized_linear_mxq_amd as mxq
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(hash((fmt, had, dtype)) % 997)
    # first a large input (many amax workgroups), then a smaller one whose
    # tensor amax is far below the first's: stale partials would show
    for rows, cols, scale in ((2048, 1024, 1000.0), (40, 256, 0.01)):
        gu.say(f"noalloc fmt={fmt} had={had} dtype={dtype} shape={rows}x{cols}")
        x = (rng.laplace(size=(rows, cols)) * scale).astype(np.float32)
        xd = gu.act_to_dev(wl_bits(x) if dtype == "bf16" else x, dtype)
        want = mxq.quantize(xd, gu.FMT_ID[fmt], hadamard=had)
        got = mxq.empty_qtensor(gu.FMT_ID[fmt], rows, cols)
        _noalloc(lib, xd, fmt, had, got, stream)
        torch.cuda.synchronize()
        assert torch.equal(got.codes, want.codes)
        assert torch.equal(got.scales, want.scales)
        if fmt == "NVFP4":
            assert torch.equal(got.tensor_scale, want.tensor_scale)


def wl_bits(x):
    from fp8_quantized_linear_mxq_amd import workloads as wl
    return wl.f32_to_bf16_bits(x)
