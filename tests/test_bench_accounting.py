"""The benchmark's algorithmic byte counts for the activation quantize, from
the formats' storage: bf16 in, codes (1/2 byte per element for 4-bit, 1 for
FP8), one scale byte per block (32; 16 for NVFP4), u in fp32; the dynamic
NVFP4 tensor scale reads the input twice."""
import bench
from fp8_quantized_linear_mxq_amd import workloads as wl


def test_quantize_bytes():
    w = wl.WORKLOADS
    # w4a8_mlp: 4096 x 1152 bf16 -> MXFP8
    assert bench.quantize_bytes(w["w4a8_mlp"]) == 4096 * 1152 * 2 + 4096 * 1152 + 4096 * 1152 // 32
    # svdq_r32: 4096 x 3072 bf16 -> MXFP4, plus u = x L1 (rank 32, fp32)
    assert bench.quantize_bytes(w["svdq_r32"]) == (4096 * 3072 * 2 + 4096 * 3072 // 2
                                                   + 4096 * 3072 // 32 + 4096 * 32 * 4)
    # nvfp4_had16: two reads of x, codes, E4M3 scales per 16
    assert bench.quantize_bytes(w["nvfp4_had16"]) == (2 * 4096 * 3072 * 2 + 4096 * 3072 // 2
                                                      + 4096 * 3072 // 16)
    # convolution: the 16384 x 2560 input (implicit im2col) or 16384 x 23040 im2col, to MXFP8
    c = w["chameleon_conv"]
    assert bench.quantize_bytes(c, 2560) == 16384 * 2560 * (2 + 1) + 16384 * 2560 // 32
    assert bench.quantize_bytes(c) == 16384 * 23040 * (2 + 1) + 16384 * 23040 // 32
    # w4a4_small: fp32 in
    assert bench.quantize_bytes(w["w4a4_small"]) == 256 * 1152 * 4 + 256 * 1152 // 2 + 256 * 1152 // 32
