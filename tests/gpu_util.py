"""Helpers for the GPU parity tests: host<->device marshalling and oracle
packing.  Expected values always come from ``oracle/``; the HIP path's
outputs are only ever compared, never reused as expectations."""
from __future__ import annotations

import sys

import numpy as np

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import gemm as og
from oracle import hadamard as oh
from oracle import quantize as oq

FMT_ID = {"MXFP4": 1, "MXFP8": 2, "NVFP4": 3, "INT4": 4}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev_f32(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_dev_bf16(bits: np.ndarray):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def act_to_dev(act: np.ndarray, dtype: str):
    """Workload activations (fp32 values or bf16 bits) -> device tensor."""
    return to_dev_bf16(act) if dtype == "bf16" else to_dev_f32(act)


def act_values(act: np.ndarray, dtype: str) -> np.ndarray:
    return wl.bf16_to_f32(act) if dtype == "bf16" else np.asarray(act, np.float32)


def unpack_dev_codes(q, fmt: str) -> np.ndarray:
    codes = q.codes.cpu().numpy()
    if fmt == "MXFP8":
        return codes[:, :q.cols]
    return oq.unpack_nibbles(codes[:, :q.cols // 2])


def dev_scales(q, fmt: str) -> np.ndarray:
    s = q.scales.cpu().numpy()
    nb = q.cols // oq.BLOCK[fmt]
    return s[:, :nb]


def oracle_quant(x: np.ndarray, fmt: str, had: int = 0, mant_bits: int = 23, g=None) -> dict:
    """Oracle quantization of fp32 values x (optionally rotated first)."""
    r = oh.rotate(x, had, mant_bits) if had else np.asarray(x, np.float32)
    return oq.quantize(r, fmt, tensor_scale=g)


def qtensor_from_oracle(q: dict, rows: int, cols: int):
    """Upload oracle codes/scales as a device QTensor (packed layout)."""
    torch = torch_mod()
    from fp8_quantized_linear_mxq_amd import QTensor
    fmt = q["fmt"]
    if fmt == "MXFP8":
        codes = q["codes"].astype(np.uint8)
    else:
        codes = oq.pack_nibbles(q["codes"])
    scales = q["scales"]
    if fmt == "INT4":
        sc = torch.from_numpy(np.ascontiguousarray(scales, np.float32)).cuda()
    else:
        sc = torch.from_numpy(np.ascontiguousarray(scales, np.uint8)).cuda()
    ts = None
    if fmt == "NVFP4":
        ts = torch.tensor([float(q["g"])], dtype=torch.float32).cuda()
    return QTensor(FMT_ID[fmt], rows, cols, torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
                   sc, ts)


def alpha_of(qa: dict, qw: dict) -> float:
    """Product of the NVFP4 tensor scales of the operands that are NVFP4."""
    alpha = 1.0
    for q in (qa, qw):
        if q["fmt"] == "NVFP4":
            alpha *= float(q["g"])
    return alpha


def dequant_w_for_gemm(qw: dict) -> np.ndarray:
    """Weights dequantized without the NVFP4 tensor scale (it goes to alpha)."""
    if qw["fmt"] == "NVFP4":
        return oq.dequantize_nvfp4(qw["codes"], qw["scales"], 1.0)
    return oq.dequantize(qw)


def dequant_a_for_gemm(qa: dict) -> np.ndarray:
    if qa["fmt"] == "NVFP4":
        return oq.dequantize_nvfp4(qa["codes"], qa["scales"], 1.0)
    return oq.dequantize(qa)


def check_gemm(y_dev, a_deq, w_deq, alpha, u=None, l2=None, x=None, l1=None, bias=None,
               rows=None, cols=None, tag=""):
    """Compare a device bf16 output with the oracle within the stated bound."""
    torch = torch_mod()
    y = y_dev.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        y = y[rows]
    if cols is not None:
        y = y[:, cols]
    ref = og.linear(a_deq, w_deq, alpha, u, l2, bias)
    s = og.abs_sum_bound(a_deq, w_deq, alpha, x, l1, l2)
    tol = og.tolerance(ref, s)
    err = np.abs(y - ref)
    ratio = float(np.max(err / np.maximum(tol, 1e-300)))
    bad = err > tol
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{tag}: {bad.sum()} outputs out of tolerance; worst err/tol "
                             f"{ratio:.3g}; first ({i},{j}) got {y[i, j]!r} ref {ref[i, j]!r} "
                             f"tol {tol[i, j]!r}")
    return ratio
