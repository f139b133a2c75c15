"""The benchmark's algorithmic work counts, from the formats' storage and the
layer's shapes: the activation quantize reads bf16 (fp32) x once and writes
codes (1/2 byte per element for 4-bit, 1 for FP8), one scale byte per block
(32; 16 for NVFP4) and u in fp32; the GEMM does 2 M N K plus 2 M N r for a
rank-r branch; each route is judged against its own dense MFMA peak."""
import os

import bench
from fp8_quantized_linear_mxq_amd import workloads as wl


def test_quantize_bytes():
    w = wl.WORKLOADS
    # w4a8_mlp: 4096 x 1152 bf16 -> MXFP8
    assert bench.quantize_bytes(w["w4a8_mlp"]) == 4096 * 1152 * 2 + 4096 * 1152 + 4096 * 1152 // 32
    # svdq_r32: 4096 x 3072 bf16 -> MXFP4, plus u = x L1 (rank 32, fp32)
    assert bench.quantize_bytes(w["svdq_r32"]) == (4096 * 3072 * 2 + 4096 * 3072 // 2
                                                   + 4096 * 3072 // 32 + 4096 * 32 * 4)
    # nvfp4_had16: x once (the tensor-amax re-read is measured, not algorithmic),
    # codes, E4M3 scales per 16: 32.24 MB
    nv = bench.quantize_bytes(w["nvfp4_had16"])
    assert nv == 4096 * 3072 * 2 + 4096 * 3072 // 2 + 4096 * 3072 // 16
    assert round(nv / 1e6, 2) == 32.24
    # convolution: the 16384 x 2560 input (implicit im2col) or 16384 x 23040 im2col, to MXFP8
    c = w["chameleon_conv"]
    assert bench.quantize_bytes(c, 2560, 128 * 128) == 16384 * 2560 * (2 + 1) + 16384 * 2560 // 32
    assert bench.quantize_bytes(c) == 16384 * 23040 * (2 + 1) + 16384 * 23040 // 32
    # w4a4_small: fp32 in
    assert bench.quantize_bytes(w["w4a4_small"]) == 256 * 1152 * 4 + 256 * 1152 // 2 + 256 * 1152 // 32


def test_gemm_flops_and_route_peaks():
    w = wl.WORKLOADS
    # svdq_r32: 2 M N K + 2 M N r (the rank-32 branch counted once, not per bf16 half)
    assert bench.gemm_flops(w["svdq_r32"]) == 2 * 4096 * 3072 * 3072 + 2 * 4096 * 3072 * 32
    assert bench.gemm_flops(w["w4a8_mlp"]) == 2 * 4096 * 1152 * 4608
    assert bench.route_peak_dtype("MXFP4", "MXFP4") == "mxfp4"
    assert bench.route_peak_dtype("MXFP8", "MXFP4") == "fp8"
    assert bench.route_peak_dtype("MXFP8", "MIXED") == "fp8"
    assert bench.route_peak_dtype("NVFP4", "NVFP4") == "bf16"
    assert bench.route_peak_dtype("BF16", "INT4") == "bf16"
    assert bench.PEAK_TFLOPS["mxfp4"] == 10100.0 and bench.PEAK_TFLOPS["fp8"] == 5000.0
    assert bench.DEFAULT_WORKLOAD == "svdq_r32"


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says why,
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
