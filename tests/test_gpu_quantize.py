"""GPU parity: mxq_quantize (all formats, both input dtypes, every Hadamard
size) against the oracle, bit-exact on codes, scales and tensor scale."""
import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd import workloads as wl
from oracle import quantize as oq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

FORMATS = ["MXFP4", "MXFP8", "NVFP4", "INT4"]


def _inputs(rows, cols, dtype, seed, had):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols))
    x *= 2.0 ** rng.integers(-12, 12, size=(rows, 1))
    hot = rng.random((rows, cols)) < 0.003
    x = np.where(hot, x * 100.0, x)
    if had:
        # keep each rotation block's dynamic range inside the exact-sum contract
        scale = 2.0 ** np.floor(np.log2(np.abs(x).max(axis=1, keepdims=True)))
        x = np.sign(x) * np.maximum(np.abs(x), scale * 2.0 ** -12)
    x[0, :] = 0.0
    x[0, 1::3] = -0.0
    x[1, :] = (1.0 + rng.random(cols)) * 2.0 ** -128 * rng.choice([-1, 1], cols)  # subnormals
    if had == 0:
        # exact grid midpoints and saturation cases in MX blocks (scale 2**0)
        x[2, :32] = [6.0, 5.0, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25] * 4
        x[2, 32:64] = [448.0, 464.0, 460.0, 1.0625, 1.1875, 17.0, 0.0009765625, 300.0] * 4
        x[3, :] = rng.standard_normal(cols) * 1e30
    x = x.astype(np.float32)
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(x)
        return bits, wl.bf16_to_f32(bits)
    return x, x


@pytest.mark.parametrize("had", [0, 16, 32, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_quantize_matches_oracle(fmt, dtype, had):
    import fp8_quantized_linear_mxq_amd as mxq
    rows, cols = 37, 384
    raw, vals = _inputs(rows, cols, dtype, seed=hash((fmt, dtype, had)) % 1000, had=had)
    gu.say(f"quantize fmt={fmt} dtype={dtype} had={had} shape={rows}x{cols}")
    xd = gu.act_to_dev(raw, dtype)
    q = mxq.quantize(xd, gu.FMT_ID[fmt], hadamard=had)
    want = gu.oracle_quant(vals, fmt, had, mant_bits=7 if dtype == "bf16" else 23)
    got_codes = gu.unpack_dev_codes(q, fmt)
    got_scales = gu.dev_scales(q, fmt)
    if fmt == "NVFP4":
        assert float(q.tensor_scale.cpu()[0]) == float(want["g"])
    bad = np.argwhere(got_scales != want["scales"])
    assert bad.size == 0, f"scale mismatch at {bad[:5].tolist()}"
    bad = np.argwhere(got_codes != want["codes"])
    assert bad.size == 0, (f"code mismatch at {bad[:5].tolist()}: got "
                           f"{got_codes[tuple(bad[0])]} want {want['codes'][tuple(bad[0])]}")


def test_nvfp4_static_scale_and_strided_rows():
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    rng = np.random.default_rng(5)
    x = (rng.laplace(size=(50, 256 + 64)) * 3).astype(np.float32)
    xd = gu.to_dev_f32(x)[:, :256]                    # row stride 320 elements
    g = np.float32(0.0017)
    gd = torch.tensor([g], dtype=torch.float32).cuda()
    gu.say("quantize NVFP4 static g, strided rows")
    q = mxq.quantize(xd, mxq.NVFP4, static_tensor_scale=gd)
    want = oq.quantize(x[:, :256], "NVFP4", tensor_scale=g)
    assert np.array_equal(gu.dev_scales(q, "NVFP4"), want["scales"])
    assert np.array_equal(gu.unpack_dev_codes(q, "NVFP4"), want["codes"])
    assert float(q.tensor_scale.cpu()[0]) == float(g)


def test_edge_shapes():
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    gu.say("quantize edge shapes")
    # one block, one row
    x = np.array([[7.5] + [0.0] * 30 + [-0.3]], np.float32)
    q = mxq.quantize(gu.to_dev_f32(x), mxq.MXFP4)
    want = oq.quantize(x, "MXFP4")
    assert np.array_equal(gu.unpack_dev_codes(q, "MXFP4"), want["codes"])
    # empty input is a no-op
    e = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    q = mxq.quantize(e, mxq.MXFP8)
    assert q.rows == 0
    # shape errors are reported, nothing is launched
    with pytest.raises(mxq.MxqError) as ei:
        mxq.quantize(gu.to_dev_f32(np.zeros((2, 48), np.float32)), mxq.MXFP4)
    assert ei.value.status == 4
    with pytest.raises(mxq.MxqError):
        mxq.quantize(gu.to_dev_f32(np.zeros((2, 96), np.float32)), mxq.MXFP4, hadamard=64)


@pytest.mark.parametrize("fmt,r,had,k", [("MXFP4", 32, 0, 640), ("MXFP8", 16, 0, 640),
                                          ("NVFP4", 128, 0, 640), ("INT4", 32, 0, 640),
                                          ("NVFP4", 48, 0, 1152), ("MXFP4", 32, 16, 640),
                                          ("NVFP4", 16, 32, 640), ("MXFP8", 32, 0, 608)])
def test_lowrank_down(fmt, r, had, k):
    """Quantize with the low-rank down projection u = x L1 (fused into the
    quantize pass without rotation and with columns a multiple of 128, else
    a separate pass): codes and scales bit-exact, u within 1e-5 of
    sum |x| |L1|; ragged rows (100 = 6 * 16 + 4)."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    rng = np.random.default_rng(8 + r + had + k)
    m = 100
    xb = wl.f32_to_bf16_bits((rng.standard_t(3, size=(m, k)) * 3).astype(np.float32))
    xb[7, :64] = 0                                   # all-zero blocks
    l1 = wl.f32_to_bf16_bits(rng.normal(0, 0.02, size=(k, r)).astype(np.float32))
    l1t = np.ascontiguousarray(l1.T)
    u = torch.empty((m, r), dtype=torch.float32, device="cuda")
    gu.say(f"quantize {fmt} had={had} + low-rank down projection rank {r}")
    q = mxq.quantize(gu.to_dev_bf16(xb), gu.FMT_ID[fmt], hadamard=had, l1t=gu.to_dev_bf16(l1t), u=u)
    xv = wl.bf16_to_f32(xb)
    want = gu.oracle_quant(xv, fmt, had=had, mant_bits=7)
    assert np.array_equal(gu.dev_scales(q, fmt), want["scales"])
    assert np.array_equal(gu.unpack_dev_codes(q, fmt), want["codes"])
    if fmt == "NVFP4":
        assert float(q.tensor_scale.cpu()[0]) == float(want["g"])
    x64 = xv.astype(np.float64)
    lv = wl.bf16_to_f32(l1).astype(np.float64)
    ref = x64 @ lv
    bound = np.abs(x64) @ np.abs(lv)
    err = np.abs(u.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * bound), float(np.max(err / bound))


@pytest.mark.parametrize("exp2", [-30, -50, -62, -80, -110])
def test_nvfp4_small_tensor_scales(exp2):
    """NVFP4 on tensors scaled by 2**exp2: the element thresholds s * g *
    midpoint take the float32 error-free path while s * g >= 2**-60 and the
    float64 path below; both must match the oracle bit for bit."""
    import fp8_quantized_linear_mxq_amd as mxq
    rng = np.random.default_rng(40 - exp2)
    x = (rng.standard_t(3, size=(24, 256)) * 2.0 ** rng.integers(-6, 6, size=(24, 1))
         * 2.0 ** exp2).astype(np.float32)
    gu.say(f"NVFP4 small tensor scale 2**{exp2}")
    q = mxq.quantize(gu.to_dev_f32(x), mxq.NVFP4)
    want = gu.oracle_quant(x, "NVFP4")
    assert float(q.tensor_scale.cpu()[0]) == float(want["g"])
    assert np.array_equal(gu.dev_scales(q, "NVFP4"), want["scales"])
    assert np.array_equal(gu.unpack_dev_codes(q, "NVFP4"), want["codes"])


def test_nvfp4_thresholds_just_above_a_midpoint():
    """Values a hair above a rounding midpoint of x / (s g): 75 / (18 g) is
    3.5 + 1e-8 for g = 1.1904761791229248, so it must round up to 4.  The
    threshold 3.5 * s * g is not a float32 and the float32 just above it is
    75 itself, which the encoder finds only if each step of its error-free
    threshold arithmetic rounds on its own (a multiply fused into a later add
    moved these thresholds one ulp up)."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    g = np.float32(1.1904761791229248)
    x = np.zeros((2, 32), np.float32)
    x[0, :5] = [128.0, 75.0, -75.0, 37.5, -37.5]      # s = 18: 3.5+ and 1.75+
    x[0, 16:19] = [64.0, 18.75, -18.75]                # s = 9: 1.75+
    x[1, :3] = [107.0, 62.5, -62.5]                    # s = 15: 3.5+
    x[1, 16:19] = [424.0, 125.0, -125.0]               # s = 60: 1.75+
    gu.say("NVFP4 values just above a midpoint (static g)")
    gd = torch.tensor([g], dtype=torch.float32).cuda()
    want = oq.quantize(x, "NVFP4", tensor_scale=g)
    assert want["codes"][0, 1] == 6 and want["codes"][1, 17] == 4   # 4.0 and 2.0: rounded up
    for dtype in ("f32", "bf16"):
        xd = gu.act_to_dev(wl.f32_to_bf16_bits(x) if dtype == "bf16" else x, dtype)
        q = mxq.quantize(xd, mxq.NVFP4, static_tensor_scale=gd)
        assert np.array_equal(gu.dev_scales(q, "NVFP4"), want["scales"])
        assert np.array_equal(gu.unpack_dev_codes(q, "NVFP4"), want["codes"]), dtype


def _packed_l1t(l1t: np.ndarray) -> np.ndarray:
    """The packed order of mxq_pack_l1t written out: 16-byte piece
    i = ((g * rank/16 + t) * 4 + j) * 64 + l holds
    L1^T[16 t + l % 16][128 g + 32 (l // 16) + 8 j + (0..7)]."""
    rank, cols = l1t.shape
    nt, pieces = rank // 16, rank * cols // 8
    i = np.arange(pieces)
    lane, j, rest = i & 63, (i >> 6) & 3, i >> 8
    t, g = rest % nt, rest // nt
    row = t * 16 + lane % 16
    col0 = g * 128 + (lane // 16) * 32 + 8 * j
    return l1t[row[:, None], col0[:, None] + np.arange(8)].reshape(rank, cols)


@pytest.mark.parametrize("rank,cols", [(16, 128), (32, 640), (48, 1152), (128, 256), (32, 3072)])
def test_pack_l1t_layout(rank, cols):
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    rng = np.random.default_rng(rank + cols)
    bits = rng.integers(0, 1 << 16, size=(rank, cols), dtype=np.uint16)
    gu.say(f"pack L1^T rank {rank} cols {cols}")
    got = mxq.pack_l1t(gu.to_dev_bf16(bits))
    torch.cuda.synchronize()
    got = got.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _packed_l1t(bits))


@pytest.mark.parametrize("fmt,r,m,k", [("MXFP4", 32, 4096, 3072), ("MXFP4", 16, 100, 640),
                                        ("MXFP8", 32, 37, 256), ("NVFP4", 48, 100, 1152),
                                        ("INT4", 128, 21, 384), ("NVFP4", 32, 300, 1024)])
def test_quantize_with_packed_l1(fmt, r, m, k):
    """mxq_quantize_lrp (L1 in the packed order) equals mxq_quantize (L1^T
    rows) bit for bit: codes, scales, tensor scale and u; ragged rows and the
    SVDQuant layer's 4096 x 3072 activation.  Against the oracle on every row
    of the small cases and on 64 sampled rows of the full one."""
    import torch
    import fp8_quantized_linear_mxq_amd as mxq
    rng = np.random.default_rng(3 * r + m + k)
    xb = wl.f32_to_bf16_bits((rng.standard_t(3, size=(m, k)) * 3).astype(np.float32))
    l1 = wl.f32_to_bf16_bits(rng.normal(0, 0.02, size=(r, k)).astype(np.float32))
    xd, l1d = gu.to_dev_bf16(xb), gu.to_dev_bf16(l1)
    gu.say(f"quantize {fmt} with packed L1, rank {r}, {m}x{k}")
    ua = torch.empty((m, r), dtype=torch.float32, device="cuda")
    ub = torch.empty((m, r), dtype=torch.float32, device="cuda")
    qa = mxq.quantize(xd, gu.FMT_ID[fmt], l1t=l1d, u=ua)
    qb = mxq.quantize(xd, gu.FMT_ID[fmt], l1p=mxq.pack_l1t(l1d), u=ub)
    torch.cuda.synchronize()
    assert torch.equal(ua, ub)
    assert np.array_equal(gu.dev_scales(qa, fmt), gu.dev_scales(qb, fmt))
    assert np.array_equal(gu.unpack_dev_codes(qa, fmt), gu.unpack_dev_codes(qb, fmt))
    if fmt == "NVFP4":
        assert torch.equal(qa.tensor_scale, qb.tensor_scale)
    # every row up to 512, else 64 sampled rows (MX formats: per-row scales,
    # so a row's codes depend on that row alone)
    rows = np.arange(m) if m <= 512 else np.sort(np.random.default_rng(m).choice(m, 64, replace=False))
    if m <= 512 or fmt != "NVFP4":
        want = gu.oracle_quant(wl.bf16_to_f32(xb[rows]), fmt, mant_bits=7)
        assert np.array_equal(gu.unpack_dev_codes(qb, fmt)[rows], want["codes"])
        assert np.array_equal(gu.dev_scales(qb, fmt)[rows], want["scales"])
    x64 = wl.bf16_to_f32(xb[rows]).astype(np.float64)
    lv = wl.bf16_to_f32(l1).astype(np.float64).T
    err = np.abs(ub.cpu().numpy()[rows].astype(np.float64) - x64 @ lv)
    assert np.all(err <= 1e-5 * (np.abs(x64) @ np.abs(lv)))
