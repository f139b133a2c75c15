"""CPU checks of the C ABI: the built library loads, exports every symbol the
header declares, and its host-only entry points and argument validation
behave as documented (no device work is enqueued by any call here)."""
import ctypes as C
import os
import re

import pytest

from fp8_quantized_linear_mxq_amd import _lib
from oracle import route

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mxq.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_exports(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.mxq_version() == 1


def test_status_strings(lib):
    assert lib.mxq_status_string(0) == b"ok"
    assert lib.mxq_status_string(4).startswith(b"shape")
    assert lib.mxq_status_string(99) == b"unknown status"


def test_storage_closed_form(lib):
    for fmt, bits in ((1, 4.25), (2, 8.25), (3, 4.5), (4, 5.0)):
        cb, sb = _lib.storage(fmt, 1152)
        assert (cb + sb) * 8 / 1152 == bits
    with pytest.raises(_lib.MxqError):
        _lib.storage(3, 24)


def test_workspace_sizes(lib):
    assert _lib.workspace_size(_lib.OP_QUANTIZE, 10, 64, _lib.MXFP4) == 0
    assert _lib.workspace_size(_lib.OP_QUANTIZE, 10, 64, _lib.NVFP4) > 0
    assert _lib.workspace_size(_lib.OP_SELECT, 10, 64) >= 10 * 3 * 8
    assert _lib.workspace_size(99, 1, 1) == -1
    # GEMM: only narrow INT4 weight groups (few output tiles) split K
    assert _lib.workspace_size(_lib.OP_GEMM, 4096, 4608, _lib.MXFP4) == 0
    assert _lib.workspace_size(_lib.OP_GEMM, 256, 1152, _lib.MXFP4) == 0
    assert _lib.workspace_size(_lib.OP_GEMM, 4096, 4608, _lib.INT4) == 0
    assert _lib.workspace_size(_lib.OP_GEMM, 16384, 20, _lib.INT4) == 16 * 16384 * 20 * 4
    assert _lib.workspace_size(_lib.OP_GEMM, 200, 300, _lib.INT4) == 16 * 200 * 300 * 4
    assert _lib.workspace_size(_lib.OP_GEMM, 16384, 200, _lib.INT4) == 0   # 256 tiles


def test_act_format_lookup_matches_oracle(lib):
    table = [1, 2, 3, 4, 1, 2, 3, 4, 1, 2] + [2] * 10
    for layer in (0, 1):
        for num_steps in (1, 4, 7, 20, 50):
            for step in range(num_steps):
                assert _lib.act_format_for_step(table, 2, 10, layer, step, num_steps) == \
                    route.act_format(table, 10, layer, step, num_steps)
    assert _lib.act_format_for_step(table, 2, 10, 2, 0, 20) == -1
    assert _lib.act_format_for_step(table, 2, 10, 0, 20, 20) == -1


def test_validation_before_device_work(lib):
    q = _lib.QTensorC(1, 0, 4, 64, None, 32, None, 2, None)
    vp = C.c_void_p
    # null input
    st = lib.mxq_quantize(None, 1, 4, 64, 64, 0, None, None, 0, None, 0, C.byref(q), None, 0, None)
    assert st == 1
    # bad dtype, bad hadamard size, bad rank, K not a multiple of the block
    assert lib.mxq_quantize(vp(16), 9, 4, 64, 64, 0, None, None, 0, None, 0, C.byref(q), None, 0, None) == 1
    assert lib.mxq_quantize(vp(16), 1, 4, 64, 64, 64, None, None, 0, None, 0, C.byref(q), None, 0, None) == 1
    assert lib.mxq_quantize(vp(16), 1, 4, 64, 64, 0, None, None, 8, None, 0, C.byref(q), None, 0, None) == 1
    q48 = _lib.QTensorC(1, 0, 4, 48, None, 32, None, 2, None)
    assert lib.mxq_quantize(vp(16), 1, 4, 48, 48, 0, None, None, 0, None, 0, C.byref(q48), None, 0, None) == 4
    # NVFP4 too: 16-blocks are quantized in pairs, so K must be a multiple of 32
    qn48 = _lib.QTensorC(3, 0, 4, 48, vp(4096), 32, vp(8192), 4, vp(12288))
    assert lib.mxq_quantize(vp(16), 1, 4, 48, 48, 0, None, None, 0, None, 0, C.byref(qn48), vp(65536),
                            4096, None) == 4
    # misaligned input pointer
    qo = _lib.QTensorC(1, 0, 4, 64, vp(4096), 32, vp(8192), 4, None)
    assert lib.mxq_quantize(vp(18), 1, 4, 64, 64, 0, None, None, 0, None, 0, C.byref(qo), None, 0, None) == 3
    # NVFP4 dynamic scale without workspace
    qn = _lib.QTensorC(3, 0, 4, 64, vp(4096), 32, vp(8192), 4, vp(12288))
    assert lib.mxq_quantize(vp(16), 1, 4, 64, 64, 0, None, None, 0, None, 0, C.byref(qn), None, 0, None) == 5
    # empty input: no-op success
    q0 = _lib.QTensorC(1, 0, 0, 64, None, 32, None, 2, None)
    assert lib.mxq_quantize(None, 1, 0, 64, 64, 0, None, None, 0, None, 0, C.byref(q0), None, 0, None) == 0
    # GEMM: unsupported pair (INT4 activations), K mismatch
    a = _lib.QTensorC(4, 0, 8, 128, vp(4096), 64, vp(8192), 16, None)
    w = _lib.QTensorC(1, 0, 8, 128, vp(4096), 64, vp(8192), 4, None)
    assert lib.mxq_gemm(C.byref(a), C.byref(w), None, None, 0, None, 0, None, vp(64), 8, 8, None, 0, None) == 2
    a2 = _lib.QTensorC(1, 0, 8, 256, vp(4096), 128, vp(8192), 8, None)
    assert lib.mxq_gemm(C.byref(a2), C.byref(w), None, None, 0, None, 0, None, vp(64), 8, 8, None, 0, None) == 4
    # convolution: MXFP4 x MXFP4, C not a multiple of 128, pixels not whole
    # images, weight K != 9 C, bad size, two groups without a permutation,
    # empty input
    x4 = _lib.QTensorC(1, 0, 40, 128, vp(4096), 64, vp(8192), 4, None)
    w4 = _lib.QTensorC(1, 0, 8, 1152, vp(4096), 576, vp(8192), 36, None)
    wn = _lib.QTensorC(3, 0, 8, 1152, vp(4096), 576, vp(8192), 72, vp(12288))
    conv = lib.mxq_conv3x3_gemm_mixed
    assert conv(C.byref(x4), 4, 5, C.byref(w4), 1, None, None, vp(64), 8, 8, None, 0, None) == 2
    x64 = _lib.QTensorC(2, 0, 40, 64, vp(4096), 64, vp(8192), 4, None)
    w64 = _lib.QTensorC(3, 0, 8, 576, vp(4096), 288, vp(8192), 36, vp(12288))
    assert conv(C.byref(x64), 4, 5, C.byref(w64), 1, None, None, vp(64), 8, 8, None, 0, None) == 4
    assert conv(C.byref(x4), 3, 5, C.byref(wn), 1, None, None, vp(64), 8, 8, None, 0, None) == 4
    wbad = _lib.QTensorC(3, 0, 8, 1024, vp(4096), 512, vp(8192), 64, vp(12288))
    assert conv(C.byref(x4), 4, 5, C.byref(wbad), 1, None, None, vp(64), 8, 8, None, 0, None) == 4
    assert conv(C.byref(x4), 0, 5, C.byref(wn), 1, None, None, vp(64), 8, 8, None, 0, None) == 1
    two = (_lib.QTensorC * 2)(wn, wn)
    assert conv(C.byref(x4), 4, 5, two, 2, None, None, vp(64), 16, 16, None, 0, None) == 1
    x0 = _lib.QTensorC(1, 0, 0, 128, None, 64, None, 4, None)
    assert conv(C.byref(x0), 4, 5, C.byref(wn), 1, None, None, vp(64), 8, 8, None, 0, None) == 0
    # bf16 activations: not a weight format, not a quantize target, rows
    # misaligned; an empty bf16 operand is a no-op
    ab = _lib.QTensorC(5, 0, 8, 128, vp(4096), 256, None, 0, None)
    assert lib.mxq_gemm(C.byref(w), C.byref(ab), None, None, 0, None, 0, None, vp(64), 8, 8, None, 0, None) == 2
    assert lib.mxq_quantize(vp(16), 1, 8, 128, 128, 0, None, None, 0, None, 0, C.byref(ab), None, 0, None) == 1
    abm = _lib.QTensorC(5, 0, 8, 128, vp(4096), 264, None, 0, None)
    assert lib.mxq_gemm(C.byref(abm), C.byref(w), None, None, 0, None, 0, None, vp(64), 8, 8, None, 0, None) == 3
    ab0 = _lib.QTensorC(5, 0, 0, 128, None, 256, None, 0, None)
    assert lib.mxq_gemm(C.byref(ab0), C.byref(w), None, None, 0, None, 0, None, vp(64), 8, 8, None, 0, None) == 0
    # selection: unsupported candidate, bad K
    cand = (C.c_int32 * 1)(2)
    assert lib.mxq_select_format(vp(16), 1, 4, 64, 64, cand, 1, vp(64), None, None, None, None,
                                 None, 0, None) == 2
    cand = (C.c_int32 * 1)(1)
    assert lib.mxq_select_format(vp(16), 1, 4, 48, 48, cand, 1, vp(64), None, None, None, None,
                                 None, 0, None) == 4


def test_validation_of_packed_lowrank_entry_points(lib):
    """mxq_pack_l1t and mxq_quantize_lrp reject bad arguments before any
    device work (no GPU here): rank, shape, alignment, and the conditions of
    the fused path (bf16 x, no rotation, columns a multiple of 128)."""
    vp = C.c_void_p
    pack = lib.mxq_pack_l1t
    assert pack(vp(4096), 8, 256, vp(8192), None) == 1        # rank not a multiple of 16
    assert pack(vp(4096), 144, 256, vp(8192), None) == 1      # rank above 128
    assert pack(vp(4096), 32, 192, vp(8192), None) == 4       # cols not a multiple of 128
    assert pack(vp(4096), 32, 0, vp(8192), None) == 0         # empty: no-op
    assert pack(None, 32, 256, vp(8192), None) == 1
    assert pack(vp(4100), 32, 256, vp(8192), None) == 3       # misaligned
    lrp = lib.mxq_quantize_lrp
    q = _lib.QTensorC(1, 0, 4, 256, vp(4096), 128, vp(8192), 8, None)
    u = vp(65536)
    # rank 0, f32 input, rotation, cols not a multiple of 128
    assert lrp(vp(16), 2, 4, 256, 256, 0, None, vp(32768), 0, u, 32, C.byref(q), None, 0, None) == 1
    assert lrp(vp(16), 1, 4, 256, 256, 0, None, vp(32768), 32, u, 32, C.byref(q), None, 0, None) == 2
    assert lrp(vp(16), 2, 4, 256, 256, 16, None, vp(32768), 32, u, 32, C.byref(q), None, 0, None) == 2
    q160 = _lib.QTensorC(1, 0, 4, 160, vp(4096), 80, vp(8192), 8, None)
    assert lrp(vp(16), 2, 4, 160, 160, 0, None, vp(32768), 32, u, 32, C.byref(q160), None, 0, None) == 4
    # missing u
    assert lrp(vp(16), 2, 4, 256, 256, 0, None, vp(32768), 32, None, 32, C.byref(q), None, 0, None) == 1
    # an empty input is a no-op after the data-free checks: the low-rank
    # conditions are not looked at, a rank outside [0, 128] still is
    q0 = _lib.QTensorC(1, 0, 0, 256, vp(4096), 128, vp(8192), 8, None)
    assert lrp(None, 2, 0, 256, 256, 0, None, None, 0, None, 32, C.byref(q0), None, 0, None) == 0
    assert lrp(None, 2, 0, 256, 256, 0, None, None, 144, None, 32, C.byref(q0), None, 0, None) == 1


def test_status_codes_and_no_device(lib):
    assert lib.mxq_status_string(8).startswith(b"NaN or Inf")
    assert _lib.STATUS[8] == "MXQ_ERR_NONFINITE"
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call below would enqueue work")
    # valid arguments with aligned stand-in pointers that are never
    # dereferenced: validation passes and the call stops at the device check
    vp = C.c_void_p
    q = _lib.QTensorC(1, 0, 4, 64, 1 << 20, 32, 1 << 21, 4, None)
    st = lib.mxq_quantize(vp(1 << 22), 1, 4, 64, 64, 0, None, None, 0, None, 0, C.byref(q),
                          None, 0, None)
    assert st == 6
    w = _lib.QTensorC(1, 0, 8, 128, 1 << 23, 64, 1 << 24, 4, None)
    a = _lib.QTensorC(1, 0, 4, 128, 1 << 25, 64, 1 << 26, 4, None)
    st = lib.mxq_gemm(C.byref(a), C.byref(w), None, None, 0, None, 0, None, vp(1 << 27), 8, 8,
                      None, 0, None)
    assert st == 6


def test_validation_of_weight_preparation_entry_points(lib):
    """mxq_quantize_mse, mxq_lowrank_split and mxq_quantize_noalloc reject
    bad arguments before any device work (stand-in pointers, never read)."""
    vp = C.c_void_p
    # MSE scales: MXFP8 is a known format without MSE scales, K not a
    # multiple of 32, misaligned input, NVFP4 without its workspace, empty
    q8 = _lib.QTensorC(2, 0, 4, 64, vp(4096), 64, vp(8192), 4, None)
    assert lib.mxq_quantize_mse(vp(16), 1, 4, 64, 64, C.byref(q8), None, 0, None) == 2
    q99 = _lib.QTensorC(99, 0, 4, 64, vp(4096), 32, vp(8192), 4, None)
    assert lib.mxq_quantize_mse(vp(16), 1, 4, 64, 64, C.byref(q99), None, 0, None) == 1
    q48 = _lib.QTensorC(1, 0, 4, 48, vp(4096), 32, vp(8192), 4, None)
    assert lib.mxq_quantize_mse(vp(16), 1, 4, 48, 48, C.byref(q48), None, 0, None) == 4
    q4 = _lib.QTensorC(1, 0, 4, 64, vp(4096), 32, vp(8192), 4, None)
    assert lib.mxq_quantize_mse(vp(18), 1, 4, 64, 64, C.byref(q4), None, 0, None) == 3
    assert lib.mxq_quantize_mse(vp(16), 7, 4, 64, 64, C.byref(q4), None, 0, None) == 1
    qn = _lib.QTensorC(3, 0, 4, 64, vp(4096), 32, vp(8192), 4, vp(12288))
    assert lib.mxq_quantize_mse(vp(16), 1, 4, 64, 64, C.byref(qn), None, 0, None) == 5
    q0 = _lib.QTensorC(1, 0, 0, 64, None, 32, None, 4, None)
    assert lib.mxq_quantize_mse(None, 1, 0, 64, 64, C.byref(q0), None, 0, None) == 0
    # SVD split: rank 0 or above 128, rank above min(n, k), null factor,
    # misaligned residual, workspace missing or too small
    split = lib.mxq_lowrank_split
    args = lambda **o: dict(dict(w=vp(1 << 20), n=64, k=96, ldw=96, rank=8, iters=0, l1t=vp(1 << 21),
                                 l2t=vp(1 << 22), resid=vp(1 << 23), ld_resid=96, sigma=None,
                                 ws=vp(1 << 24), wsb=1 << 30, st=None), **o)
    call = lambda a: split(a["w"], a["n"], a["k"], a["ldw"], a["rank"], a["iters"], a["l1t"], a["l2t"],
                           a["resid"], a["ld_resid"], a["sigma"], a["ws"], a["wsb"], a["st"])
    assert call(args(rank=0)) == 1
    assert call(args(rank=144)) == 1
    assert call(args(rank=80, k=64, ldw=64, ld_resid=64)) == 4
    assert call(args(l1t=None)) == 1
    assert call(args(resid=vp((1 << 23) + 2))) == 3
    assert call(args(ws=None)) == 5
    need = _lib.workspace_size(_lib.OP_LOWRANK_SPLIT, 64, 96, 8)
    assert need > 0 and call(args(wsb=need - 1)) == 5
    # the allocation-free quantize validates like mxq_quantize
    assert lib.mxq_quantize_noalloc(None, 1, 4, 64, 64, 0, None, None, 0, None, 0, C.byref(q4), None) == 1
    assert lib.mxq_quantize_noalloc(vp(16), 1, 4, 48, 48, 0, None, None, 0, None, 0, C.byref(q48), None) == 4
