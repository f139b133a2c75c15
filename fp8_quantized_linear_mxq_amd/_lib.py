"""ctypes binding of libmxq (include/mxq.h).

Argument marshalling only: every step of the layer runs inside libmxq's HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
built library is missing, ``load()`` raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxq.so")

MXFP4, MXFP8, NVFP4, INT4 = 1, 2, 3, 4
BF16 = 5   # unquantized bf16 activations (GEMM operand only)
FORMATS = {"MXFP4": MXFP4, "MXFP8": MXFP8, "NVFP4": NVFP4, "INT4": INT4}
FORMAT_NAMES = {v: k for k, v in FORMATS.items()}
DT_F32, DT_BF16 = 1, 2
OP_QUANTIZE, OP_GEMM, OP_SELECT, OP_QUANTIZE_MSE, OP_LOWRANK_SPLIT = 1, 2, 3, 4, 5
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16, INT4: 32}

STATUS = {0: "MXQ_OK", 1: "MXQ_ERR_INVALID_ARG", 2: "MXQ_ERR_UNSUPPORTED",
          3: "MXQ_ERR_ALIGNMENT", 4: "MXQ_ERR_SHAPE", 5: "MXQ_ERR_WORKSPACE",
          6: "MXQ_ERR_NO_DEVICE", 7: "MXQ_ERR_LAUNCH", 8: "MXQ_ERR_NONFINITE"}

# Every symbol include/mxq.h declares.
EXPORTS = ("mxq_quantize", "mxq_quantize_noalloc", "mxq_quantize_lrp", "mxq_pack_l1t", "mxq_gemm", "mxq_gemm_mixed", "mxq_conv3x3_gemm_mixed",
           "mxq_select_format", "mxq_quantize_mse", "mxq_lowrank_split",
           "mxq_act_format_for_step", "mxq_workspace_size", "mxq_storage",
           "mxq_status_string", "mxq_version")


class MxqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class QTensorC(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("reserved", C.c_int32),
                ("rows", C.c_int64), ("cols", C.c_int64),
                ("codes", C.c_void_p), ("ld_codes", C.c_int64),
                ("scales", C.c_void_p), ("ld_scales", C.c_int64),
                ("tensor_scale", C.c_void_p)]


_lib = None


def load():
    """Load libmxq.so (built in-tree by ``build.py``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmxq is not built ({LIB_PATH} missing); run "
                           "python -m fp8_quantized_linear_mxq_amd.build")
    try:  # share the HIP runtime torch already mapped (same soname)
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    qp = C.POINTER(QTensorC)
    lib.mxq_quantize.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i32, vp, i64, qp, vp, sz, vp]
    lib.mxq_quantize.restype = i32
    lib.mxq_quantize_lrp.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i32, vp, i64, qp, vp, sz, vp]
    lib.mxq_quantize_lrp.restype = i32
    lib.mxq_pack_l1t.argtypes = [vp, i32, i64, vp, vp]
    lib.mxq_pack_l1t.restype = i32
    lib.mxq_quantize_noalloc.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i32, vp, i64, qp, vp]
    lib.mxq_quantize_noalloc.restype = i32
    lib.mxq_gemm.argtypes = [qp, qp, vp, vp, i64, vp, i32, vp, vp, i64, i64, vp, sz, vp]
    lib.mxq_gemm.restype = i32
    lib.mxq_gemm_mixed.argtypes = [qp, qp, i32, vp, vp, i64, vp, i32, vp, vp, i64, i64, vp, sz, vp]
    lib.mxq_gemm_mixed.restype = i32
    lib.mxq_conv3x3_gemm_mixed.argtypes = [qp, i64, i64, qp, i32, vp, vp, vp, i64, i64, vp, sz,
                                           vp]
    lib.mxq_conv3x3_gemm_mixed.restype = i32
    lib.mxq_select_format.argtypes = [vp, i32, i64, i64, i64, C.POINTER(i32), i32, vp, vp, vp,
                                      vp, vp, vp, sz, vp]
    lib.mxq_select_format.restype = i32
    lib.mxq_quantize_mse.argtypes = [vp, i32, i64, i64, i64, qp, vp, sz, vp]
    lib.mxq_quantize_mse.restype = i32
    lib.mxq_lowrank_split.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, vp, i64, vp, vp, sz, vp]
    lib.mxq_lowrank_split.restype = i32
    lib.mxq_act_format_for_step.argtypes = [C.POINTER(C.c_uint8), i32, i32, i32, i32, i32]
    lib.mxq_act_format_for_step.restype = i32
    lib.mxq_workspace_size.argtypes = [i32, i64, i64, i32]
    lib.mxq_workspace_size.restype = i64
    lib.mxq_storage.argtypes = [i32, i64, C.POINTER(i64), C.POINTER(i64)]
    lib.mxq_storage.restype = i32
    lib.mxq_status_string.argtypes = [i32]
    lib.mxq_status_string.restype = C.c_char_p
    lib.mxq_version.argtypes = []
    lib.mxq_version.restype = i32
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise MxqError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def storage(fmt: int, cols: int):
    """(code bytes, scale bytes) per row for ``cols`` elements."""
    lib = load()
    cb, sb = C.c_int64(), C.c_int64()
    _check("mxq_storage", lib.mxq_storage(fmt, cols, C.byref(cb), C.byref(sb)))
    return cb.value, sb.value


def workspace_size(op: int, rows: int, cols: int, fmt: int = 0) -> int:
    return int(load().mxq_workspace_size(op, rows, cols, fmt))


def act_format_for_step(table, n_layers: int, n_buckets: int, layer: int, step: int,
                        num_steps: int) -> int:
    lib = load()
    buf = (C.c_uint8 * len(table))(*[int(v) for v in table])
    return int(lib.mxq_act_format_for_step(buf, n_layers, n_buckets, layer, step, num_steps))


@dataclass
class QTensor:
    """A quantized [rows, cols] operand in device memory (torch uint8 / fp32)."""
    fmt: int
    rows: int
    cols: int
    codes: "object"
    scales: "object"
    tensor_scale: "object" = None

    def c(self) -> QTensorC:
        return QTensorC(self.fmt, 0, self.rows, self.cols,
                        self.codes.data_ptr() if self.codes is not None else None,
                        self.codes.stride(0) * self.codes.element_size() if self.codes is not None else 0,
                        self.scales.data_ptr() if self.scales is not None else None,
                        self.scales.stride(0) * self.scales.element_size() if self.scales is not None else 0,
                        self.tensor_scale.data_ptr() if self.tensor_scale is not None else None)


def empty_qtensor(fmt: int, rows: int, cols: int, device="cuda") -> QTensor:
    """Allocates (torch) the buffers of a quantized operand."""
    import torch
    cb, sb = storage(fmt, cols)
    # row strides padded to the ABI's alignment (16 B codes; 4 B scales, 16 B
    # for INT4's fp32 scales)
    codes = torch.empty((rows, (cb + 15) // 16 * 16), dtype=torch.uint8, device=device)
    if fmt == INT4:
        scales = torch.empty((rows, (sb // 4 + 3) // 4 * 4), dtype=torch.float32, device=device)
    else:
        scales = torch.empty((rows, (sb + 3) // 4 * 4), dtype=torch.uint8, device=device)
    ts = torch.empty((1,), dtype=torch.float32, device=device) if fmt == NVFP4 else None
    return QTensor(fmt, rows, cols, codes, scales, ts)


def bf16_operand(x) -> QTensor:
    """A 2-D cuda bfloat16 tensor as the GEMM's unquantized activation
    operand (4-bit weights, 16-bit activations)."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("bf16_operand needs a row-major 2-D bfloat16 tensor")
    return QTensor(BF16, x.shape[0], x.shape[1], x, None)


def pack_l1t(l1t, stream=None):
    """mxq_pack_l1t: L1^T [rank, cols] bf16 (cuda) into the packed order the
    fused quantize + low-rank kernel reads; returned with the same shape."""
    import torch
    lib = load()
    rank, cols = l1t.shape
    l1t = l1t.contiguous()
    out = torch.empty_like(l1t)
    _check("mxq_pack_l1t", lib.mxq_pack_l1t(_ptr(l1t), rank, cols, _ptr(out), _stream(stream)))
    return out


def quantize(x, fmt: int, hadamard: int = 0, static_tensor_scale=None, l1t=None, u=None,
             out: QTensor | None = None, workspace=None, stream=None, l1p=None) -> QTensor:
    """mxq_quantize on a 2-D torch tensor (float32 or bfloat16, cuda); with
    ``l1p`` (L1 from pack_l1t) instead of ``l1t``, mxq_quantize_lrp."""
    import torch
    lib = load()
    rows, cols = x.shape
    dt = DT_BF16 if x.dtype == torch.bfloat16 else DT_F32
    if out is None:
        out = empty_qtensor(fmt, rows, cols, x.device)
    if workspace is None:
        n = workspace_size(OP_QUANTIZE, rows, cols, fmt)
        workspace = torch.empty((max(n, 16),), dtype=torch.uint8, device=x.device)
    qc = out.c()
    if l1p is not None:
        st = lib.mxq_quantize_lrp(_ptr(x), dt, rows, cols, x.stride(0), hadamard,
                                  _ptr(static_tensor_scale), _ptr(l1p), l1p.shape[0], _ptr(u),
                                  0 if u is None else u.stride(0), C.byref(qc), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
        _check("mxq_quantize_lrp", st)
        return out
    rank = 0 if l1t is None else l1t.shape[0]
    st = lib.mxq_quantize(_ptr(x), dt, rows, cols, x.stride(0), hadamard,
                          _ptr(static_tensor_scale), _ptr(l1t), rank, _ptr(u),
                          0 if u is None else u.stride(0), C.byref(qc), _ptr(workspace),
                          workspace.numel(), _stream(stream))
    _check("mxq_quantize", st)
    return out


def _gemm_workspace(a: QTensor, ws: list, workspace):
    """The optional GEMM workspace: a given tensor, none (workspace=False),
    or a fresh one sized for the largest of the weight operands ``ws``."""
    import torch
    if workspace is False:
        return None, 0
    if workspace is None:
        n = max([workspace_size(OP_GEMM, a.rows, w.rows, w.fmt) for w in ws] + [0])
        if n <= 0:
            return None, 0
        workspace = torch.empty((n,), dtype=torch.uint8, device=a.codes.device)
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def gemm(a: QTensor, w: QTensor, n_out: int | None = None, w_out_col=None, u=None, l2t=None,
         bias=None, out=None, stream=None, workspace=None):
    """mxq_gemm; returns the bf16 [M, n_out] output tensor.  ``workspace``:
    a device tensor, None (allocated when the route can use one) or False."""
    import torch
    lib = load()
    n_out = w.rows if n_out is None else n_out
    if out is None:
        out = torch.empty((a.rows, n_out), dtype=torch.bfloat16, device=a.codes.device)
    ac, wc = a.c(), w.c()
    rank = 0 if l2t is None else l2t.shape[1]
    wsp, wsn = _gemm_workspace(a, [w], workspace)
    st = lib.mxq_gemm(C.byref(ac), C.byref(wc), _ptr(w_out_col), _ptr(u),
                      0 if u is None else u.stride(0), _ptr(l2t), rank, _ptr(bias), _ptr(out),
                      out.stride(0), n_out, wsp, wsn, _stream(stream))
    _check("mxq_gemm", st)
    return out


def gemm_mixed(a: QTensor, groups: list, w_perm, n_out: int, u=None, l2t=None, bias=None,
               out=None, stream=None, workspace=None):
    """mxq_gemm_mixed over weight groups (QTensor list) and their permutation."""
    import torch
    lib = load()
    if out is None:
        out = torch.empty((a.rows, n_out), dtype=torch.bfloat16, device=a.codes.device)
    ac = a.c()
    arr = (QTensorC * len(groups))(*[g.c() for g in groups])
    rank = 0 if l2t is None else l2t.shape[1]
    wsp, wsn = _gemm_workspace(a, groups, workspace)
    st = lib.mxq_gemm_mixed(C.byref(ac), arr, len(groups), _ptr(w_perm), _ptr(u),
                            0 if u is None else u.stride(0), _ptr(l2t), rank, _ptr(bias),
                            _ptr(out), out.stride(0), n_out, wsp, wsn, _stream(stream))
    _check("mxq_gemm_mixed", st)
    return out


def conv3x3_gemm_mixed(x: QTensor, height: int, width: int, groups: list, w_perm, n_out: int,
                       bias=None, out=None, stream=None, workspace=None):
    """mxq_conv3x3_gemm_mixed: the 3x3 convolution (stride 1, zero padding 1)
    of the quantized pixel rows ``x`` ([images*height*width, C]) with weight
    groups of 9*C columns; returns the bf16 [x.rows, n_out] output tensor."""
    import torch
    lib = load()
    if out is None:
        out = torch.empty((x.rows, n_out), dtype=torch.bfloat16, device=x.codes.device)
    xc = x.c()
    arr = (QTensorC * len(groups))(*[g.c() for g in groups])
    wsp, wsn = _gemm_workspace(x, groups, workspace)
    st = lib.mxq_conv3x3_gemm_mixed(C.byref(xc), height, width, arr, len(groups), _ptr(w_perm),
                                    _ptr(bias), _ptr(out), out.stride(0), n_out, wsp, wsn,
                                    _stream(stream))
    _check("mxq_conv3x3_gemm_mixed", st)
    return out


def select_format(w, candidates=(INT4, MXFP4, NVFP4), stream=None):
    """mxq_select_format; returns (choice u8[n], sse f64[n, c], perm i32[n],
    counts i32[c], g f32[1]) as device tensors."""
    import torch
    lib = load()
    n, k = w.shape
    dt = DT_BF16 if w.dtype == torch.bfloat16 else DT_F32
    dev = w.device
    choice = torch.empty((n,), dtype=torch.uint8, device=dev)
    sse = torch.empty((n, len(candidates)), dtype=torch.float64, device=dev)
    perm = torch.empty((n,), dtype=torch.int32, device=dev)
    counts = torch.empty((len(candidates),), dtype=torch.int32, device=dev)
    g = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty((workspace_size(OP_SELECT, n, k),), dtype=torch.uint8, device=dev)
    cand = (C.c_int32 * len(candidates))(*candidates)
    st = lib.mxq_select_format(_ptr(w), dt, n, k, w.stride(0), cand, len(candidates),
                               _ptr(choice), _ptr(sse), _ptr(perm), _ptr(counts), _ptr(g),
                               _ptr(ws), ws.numel(), _stream(stream))
    _check("mxq_select_format", st)
    return choice, sse, perm, counts, g


def quantize_mse(w, fmt: int, out: QTensor | None = None, workspace=None,
                 stream=None) -> QTensor:
    """mxq_quantize_mse on 2-D torch weights (float32 or bfloat16, cuda):
    MXFP4 or NVFP4 codes with least-squared-error scales."""
    import torch
    lib = load()
    rows, cols = w.shape
    dt = DT_BF16 if w.dtype == torch.bfloat16 else DT_F32
    if out is None:
        out = empty_qtensor(fmt, rows, cols, w.device)
    if workspace is None:
        n = workspace_size(OP_QUANTIZE_MSE, rows, cols, fmt)
        workspace = torch.empty((max(n, 16),), dtype=torch.uint8, device=w.device)
    qc = out.c()
    st = lib.mxq_quantize_mse(_ptr(w), dt, rows, cols, w.stride(0), C.byref(qc),
                              _ptr(workspace), workspace.numel(), _stream(stream))
    _check("mxq_quantize_mse", st)
    return out


def lowrank_split(w, rank: int, iters: int = 0, stream=None):
    """mxq_lowrank_split on 2-D float32 cuda weights [n, k]; returns
    (L1^T bf16 [rank, k], L2^T bf16 [n, rank], R float32 [n, k],
    sigma float32 [rank])."""
    import torch
    lib = load()
    n, k = w.shape
    dev = w.device
    l1t = torch.empty((rank, k), dtype=torch.bfloat16, device=dev)
    l2t = torch.empty((n, rank), dtype=torch.bfloat16, device=dev)
    resid = torch.empty((n, k), dtype=torch.float32, device=dev)
    sigma = torch.empty((rank,), dtype=torch.float32, device=dev)
    ws = torch.empty((max(workspace_size(OP_LOWRANK_SPLIT, n, k, rank), 256),),
                     dtype=torch.uint8, device=dev)
    st = lib.mxq_lowrank_split(_ptr(w), n, k, w.stride(0), rank, iters, _ptr(l1t), _ptr(l2t),
                               _ptr(resid), resid.stride(0), _ptr(sigma), _ptr(ws), ws.numel(),
                               _stream(stream))
    _check("mxq_lowrank_split", st)
    return l1t, l2t, resid, sigma
