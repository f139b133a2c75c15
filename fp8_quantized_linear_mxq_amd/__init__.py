"""Block-scaled (microscaling) quantized linear layers for AMD MI355X.

The compute lives in libmxq (HIP kernels for gfx950 behind the C ABI in
include/mxq.h); this package is its thin ctypes binding plus the seeded
synthetic workload generators.  Import is cheap: the library is loaded on
first use and its absence is an error, never a fallback.
"""
from ._lib import (  # noqa: F401
    BF16, DT_BF16, DT_F32, FORMATS, INT4, MXFP4, MXFP8, NVFP4, OP_GEMM, OP_LOWRANK_SPLIT,
    OP_QUANTIZE, OP_QUANTIZE_MSE, OP_SELECT,
    MxqError, QTensor,
    act_format_for_step, bf16_operand, lowrank_split, conv3x3_gemm_mixed, empty_qtensor, gemm, gemm_mixed, load,
    pack_l1t, quantize, quantize_mse,
    select_format, storage, workspace_size,
)
