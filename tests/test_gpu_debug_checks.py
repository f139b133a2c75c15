"""MXQ_DEBUG_CHECKS=1: a NaN or Inf input to mxq_quantize or
mxq_select_format sets the device flag, and the next call that would enqueue
work returns MXQ_ERR_NONFINITE (and clears the flag).  Non-finite inputs are
outside the contract: the kernels still only write their outputs."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import _lib
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_env(monkeypatch):
    monkeypatch.setenv("MXQ_DEBUG_CHECKS", "1")
    yield


@pytest.mark.parametrize("fmt,bad", [("MXFP4", np.nan), ("NVFP4", np.inf), ("INT4", -np.inf),
                                     ("MXFP8", np.nan)])
def test_nonfinite_quantize_input_flags_next_call(debug_env, fmt, bad):
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say(f"debug checks: quantize fmt={fmt} bad={bad}")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    good = gu.to_dev_f32(x)
    mxq.quantize(good, gu.FMT_ID[fmt])          # finite: no flag
    mxq.quantize(good, gu.FMT_ID[fmt])
    x[5, 77] = bad
    mxq.quantize(gu.to_dev_f32(x), gu.FMT_ID[fmt])
    with pytest.raises(_lib.MxqError) as ei:
        mxq.quantize(good, gu.FMT_ID[fmt])
    assert ei.value.status == 8
    mxq.quantize(good, gu.FMT_ID[fmt])          # the flag was cleared


def test_nonfinite_weights_flag_selection_then_gemm(debug_env):
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say("debug checks: select_format with a NaN weight, then a GEMM")
    rng = np.random.default_rng(4)
    a = mxq.quantize(gu.to_dev_f32(rng.standard_normal((8, 256)).astype(np.float32)), mxq.MXFP4)
    q = mxq.quantize(gu.to_dev_f32(rng.normal(0, 0.02, size=(16, 256)).astype(np.float32)),
                     mxq.MXFP4)
    w = rng.normal(0, 0.02, size=(16, 256)).astype(np.float32)
    w[3, 100] = np.nan
    mxq.select_format(gu.to_dev_f32(w))
    with pytest.raises(_lib.MxqError) as ei:
        mxq.gemm(a, q)
    assert ei.value.status == 8
    y = mxq.gemm(a, q)
    assert y.shape == (8, 16)


def test_debug_off_ignores_nonfinite(monkeypatch):
    import fp8_quantized_linear_mxq_amd as mxq
    monkeypatch.delenv("MXQ_DEBUG_CHECKS", raising=False)
    gu.say("debug checks off: a NaN input runs and nothing is reported")
    x = np.ones((4, 64), np.float32)
    x[0, 0] = np.nan
    mxq.quantize(gu.to_dev_f32(x), mxq.MXFP4)
    mxq.quantize(gu.to_dev_f32(np.ones((4, 64), np.float32)), mxq.MXFP4)
