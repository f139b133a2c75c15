"""Seeded synthetic inputs shaped like the pages' diffusion-transformer layers.

This module holds random draws and data layout only -- none of the layer's
arithmetic -- so that the CPU oracle and the GPU library can be fed the very
same bits.  Every tensor comes from ``numpy.random.Generator(PCG64)`` with
independent child streams spawned from one base seed per workload.

bfloat16 tensors are carried as ``uint16`` bit patterns (numpy has no
bfloat16); ``bf16_to_f32`` gives their exact float32 values.

Workloads (statistics from the pages; sizes are the library's five layer
shapes):
  w4a4_small   256 x 1152 x 1152, fp32 activations Student-t(4), MXFP4 both
  w4a8_mlp     4096 x 1152 x 4608, bf16 activations Student-t(3) with 0.5% of
               channels x50, MXFP8 activations x MXFP4 weights
  nvfp4_had16  4096 x 3072 x 12288, bf16 Laplace(0,1) activations with 0.3% of
               elements x100 (the outlier share the MixDiT page reports for
               SD3), 16-point Hadamard, NVFP4 both
  svdq_r32     4096 x 3072 x 3072, bf16 Student-t(3) activations with
               per-channel scales 163**u (the channel spread the Chameleon page
               reports), MXFP4 both, rank-32 low-rank branch
  chameleon_conv  3x3 convolution as a GEMM on a 128x128x2560 latent:
               16384 x 23040 x 1280, MXFP8 activations, per-row weight formats
  w4a16_mlp    4096 x 1152 x 4608, the w4a8_mlp activations kept in bf16
               (4-bit weights, 16-bit activations) against INT4 weights
  w4a16_mx_mlp the same against MXFP4 weights
Weights are N(0, 0.02) float32 master copies.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SIGMA_W = 0.02


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


@dataclass
class Workload:
    name: str
    m: int
    k: int
    n: int
    act_dtype: str                  # "f32" or "bf16"
    act_fmt: str
    w_fmt: str                      # "MXFP4", "NVFP4" or "MIXED"
    hadamard: int = 0
    rank: int = 0
    seed: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "w4a4_small": Workload("w4a4_small", 256, 1152, 1152, "f32", "MXFP4", "MXFP4", seed=0),
    "w4a8_mlp": Workload("w4a8_mlp", 4096, 1152, 4608, "bf16", "MXFP8", "MXFP4", seed=1),
    "nvfp4_had16": Workload("nvfp4_had16", 4096, 3072, 12288, "bf16", "NVFP4", "NVFP4",
                            hadamard=16, seed=2),
    "svdq_r32": Workload("svdq_r32", 4096, 3072, 3072, "bf16", "MXFP4", "MXFP4",
                         rank=32, seed=3),
    "chameleon_conv": Workload("chameleon_conv", 16384, 2560 * 9, 1280, "bf16", "MXFP8",
                               "MIXED", seed=4,
                               extra={"latent": (128, 128, 2560), "ksize": 3}),
    "w4a16_mlp": Workload("w4a16_mlp", 4096, 1152, 4608, "bf16", "BF16", "INT4", seed=1),
    "w4a16_mx_mlp": Workload("w4a16_mx_mlp", 4096, 1152, 4608, "bf16", "BF16", "MXFP4", seed=1),
}


def _heavy_activations(rng_a, rng_s, m, k, nu, spread):
    a = rng_a.standard_t(nu, size=(m, k))
    if spread:
        a = a * (spread ** rng_s.random(k))[None, :]
    return a


def activations(wl: Workload, rows: int | None = None) -> np.ndarray:
    """The workload's activations, float32 values or bf16 bit patterns.

    ``rows`` limits the draw to the first rows of the same stream (the
    generator fills row-major, so a prefix is the full tensor's prefix).
    Not available for the convolution workload (see ``conv_latent``).
    """
    m = wl.m if rows is None else rows
    st = _streams(wl.seed, 6)
    if wl.name == "w4a4_small":
        a = st[0].standard_t(4, size=(m, wl.k)) * 1.0
        return a.astype(np.float32)
    if wl.name in ("w4a8_mlp", "w4a16_mlp", "w4a16_mx_mlp"):
        a = st[0].standard_t(3, size=(m, wl.k))
        n_hot = int(round(0.005 * wl.k))
        hot = st[4].choice(wl.k, size=n_hot, replace=False)
        a[:, hot] *= 50.0
        return f32_to_bf16_bits(a.astype(np.float32))
    if wl.name == "nvfp4_had16":
        a = st[0].laplace(0.0, 1.0, size=(m, wl.k))
        mask = st[4].random((m, wl.k)) < 0.003
        a = np.where(mask, a * 100.0, a)
        return f32_to_bf16_bits(a.astype(np.float32))
    if wl.name == "svdq_r32":
        a = _heavy_activations(st[0], st[5], m, wl.k, 3, 163.0)
        return f32_to_bf16_bits(a.astype(np.float32))
    raise ValueError(f"{wl.name}: use conv_latent / im2col")


def weights(wl: Workload, rows: int | None = None) -> np.ndarray:
    """float32 master weights [N, K], N(0, 0.02).

    For the Hadamard workload the values are drawn then rounded to bfloat16
    precision, so that the offline rotation's float64 sums stay exact.
    """
    n = wl.n if rows is None else rows
    st = _streams(wl.seed, 6)
    w = st[1].normal(0.0, SIGMA_W, size=(n, wl.k)).astype(np.float32)
    if wl.hadamard:
        w = bf16_to_f32(f32_to_bf16_bits(w))
    return w


def lowrank_factors(wl: Workload):
    """bf16 bit patterns L1 [K, r], L2 [r, N], N(0, 0.02)."""
    st = _streams(wl.seed, 6)
    l1 = st[2].normal(0.0, SIGMA_W, size=(wl.k, wl.rank)).astype(np.float32)
    l2 = st[3].normal(0.0, SIGMA_W, size=(wl.rank, wl.n)).astype(np.float32)
    return f32_to_bf16_bits(l1), f32_to_bf16_bits(l2)


def conv_latent(wl: Workload, hw: tuple | None = None) -> np.ndarray:
    """bf16 bit patterns of the [H, W, C] latent, Student-t(3) x 163**u_c."""
    h, w, c = wl.extra["latent"] if hw is None else (*hw, wl.extra["latent"][2])
    st = _streams(wl.seed, 6)
    spread = 163.0 ** st[5].random(c)
    lat = st[0].standard_t(3, size=(h, w, c)) * spread[None, None, :]
    return f32_to_bf16_bits(lat.astype(np.float32))


def im2col(latent: np.ndarray, ksize: int = 3) -> np.ndarray:
    """3x3, stride 1, zero padding 1: [H*W, 9*C], K index = (kh*3 + kw)*C + c."""
    h, w, c = latent.shape
    p = ksize // 2
    padded = np.zeros((h + 2 * p, w + 2 * p, c), dtype=latent.dtype)
    padded[p:p + h, p:p + w] = latent
    out = np.empty((h * w, ksize * ksize * c), dtype=latent.dtype)
    for kh in range(ksize):
        for kw in range(ksize):
            tap = kh * ksize + kw
            out[:, tap * c:(tap + 1) * c] = padded[kh:kh + h, kw:kw + w].reshape(h * w, c)
    return out


def mixed_weights(k: int, n: int, seed: int) -> np.ndarray:
    """float32 rows drawn from three families (uniform, normal, Student-t(2))
    so that every format of the palette wins somewhere; row i uses family
    i % 3.  Scale 0.02."""
    rng = _streams(seed, 1)[0]
    w = np.empty((n, k), dtype=np.float64)
    fam = np.arange(n) % 3
    for i in range(n):
        if fam[i] == 0:
            w[i] = rng.uniform(-SIGMA_W * 1.7, SIGMA_W * 1.7, size=k)
        elif fam[i] == 1:
            w[i] = rng.normal(0.0, SIGMA_W, size=k)
        else:
            w[i] = rng.standard_t(2, size=k) * SIGMA_W
    return w.astype(np.float32)


ACT_TABLE_BUCKETS = 10


def chameleon_act_table(n_layers: int = 1, fmt_id: int = 2) -> np.ndarray:
    """Activation-format table u8[layers][10]; the concat convolution's row
    is MXFP8 in every bucket (format id 2 in the library's numbering)."""
    return np.full((n_layers, ACT_TABLE_BUCKETS), fmt_id, dtype=np.uint8)
