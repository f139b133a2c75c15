"""Matrix-core probes behind two design decisions (GPU only):

  python -m fp8_quantized_linear_mxq_amd.probe.mfma_probe [--rate-only|--sum-only|--layout|--gemm-data]

1. Summation: single MFMAs on operands whose exact results the host computes
   with rationals -- random finite codes and block scales, and a
   "one large product plus 63 small same-sign ones" sweep -- for the scaled
   E4M3 x E2M1, E2M1 x E2M1 and E4M3 x E4M3 32x32x64 MFMAs, the plain
   E4M3 32x32x16 MFMA and the bf16 32x32x16 MFMA.  Reported per kind: the
   worst error over the largest product's magnitude, and the worst error in
   units of the fp32 spacing at the exact result (a single fp32 rounding of
   the exact sum is at most 0.5).
2. Rate: independent MFMAs from registers on one workgroup per compute unit
   (4 or 8 waves), random or all-zero operands; TFLOP/s against the
   published dense peaks (MXFP4 10.1, FP8 5.0, bf16 2.5 PFLOP/s).
3. GEMM operand data (--gemm-data): the library's MXFP4 GEMM timed on
   random, sparse and all-zero codes.
Prints one JSON line per measurement.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmxq_probe.so")

SUM_KINDS = {0: "scaled E4M3 x E2M1 32x32x64", 1: "scaled E2M1 x E2M1 32x32x64",
             2: "scaled E4M3 x E4M3 32x32x64", 3: "E4M3 x E4M3 32x32x16", 4: "bf16 x bf16 32x32x16"}
RATE_KINDS = {0: ("scaled E2M1 x E2M1 32x32x64", 2 * 32 * 32 * 64, 10100.0),
              1: ("scaled E4M3 x E2M1 32x32x64", 2 * 32 * 32 * 64, 5000.0),
              2: ("bf16 32x32x16", 2 * 32 * 32 * 16, 2500.0)}


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (python -m fp8_quantized_linear_mxq_amd.build)")
    lib = C.CDLL(LIB)
    lib.probe_mfma_rate.argtypes = [C.c_int] * 5 + [C.c_void_p, C.c_void_p]
    lib.probe_mfma_sum.argtypes = [C.c_int] + [C.c_void_p] * 6
    lib.probe_cvt_scale.argtypes = [C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]
    return lib


# ---- operand values (exact) -------------------------------------------------

_E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def e2m1(c):
    v = _E2M1[c & 7]
    return -v if c & 8 else v


def e4m3(c):
    e, m = (c >> 3) & 15, c & 7
    assert (c & 0x7F) != 0x7F, "E4M3 NaN code"
    v = Fraction(m, 512) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return -v if c & 0x80 else v


def bf16(bits):
    return Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))


def e4m3_code(v: Fraction):
    """The E4M3 code of an exactly representable power of two 2**-9 .. 256."""
    e = math.floor(math.log2(v))
    return (e + 7) << 3 if e >= -6 else 1 << (e + 9)


def bf16_code(v: float):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0]) >> 16


# ---- lane packing -----------------------------------------------------------

def _kmap(fp8, h, t):
    """Logical K of slot t in lane half h for the 32x32x64 scaled MFMA (as
    the --layout probe finds it): E2M1 operands hold K = 32h + t; E4M3
    operands hold K = 16h + t for t < 16 and K = 32 + 16h + (t - 16) after,
    so each lane's E4M3 values straddle both 32-blocks.  The scale of block
    b comes from lane 32b of the row for both formats."""
    if not fp8:
        return 32 * h + t
    return 16 * h + t if t < 16 else 32 + 16 * h + (t - 16)


def _pack(kind, codes, is_a):
    """codes: [32][K] ints in logical K order -> [64][8] int32 operand
    dwords (lane l carries row l % 32, lane half l // 32)."""
    ops = np.zeros((64, 8), dtype=np.uint64)
    fp4 = (kind == 1) or (kind == 0 and not is_a)
    for lane in range(64):
        row, h = lane % 32, lane // 32
        if kind in (0, 1, 2):
            ks = [codes[row][_kmap(not fp4, h, t)] for t in range(32)]
            if fp4:
                for d in range(4):
                    ops[lane, d] = sum(int(ks[8 * d + t]) << (4 * t) for t in range(8))
            else:
                for d in range(8):
                    ops[lane, d] = sum(int(ks[4 * d + t]) << (8 * t) for t in range(4))
        elif kind == 3:
            ks = codes[row][8 * h:8 * h + 8]
            for d in range(2):
                ops[lane, d] = sum(int(ks[4 * d + t]) << (8 * t) for t in range(4))
        else:
            ks = codes[row][8 * h:8 * h + 8]
            for d in range(4):
                ops[lane, d] = int(ks[2 * d]) | (int(ks[2 * d + 1]) << 16)
    return ops.astype(np.uint32).view(np.int32)


def _value_fns(kind):
    if kind == 0:
        return e4m3, e2m1
    if kind == 1:
        return e2m1, e2m1
    if kind in (2, 3):
        return e4m3, e4m3
    return bf16, bf16


def _kdim(kind):
    return 64 if kind in (0, 1, 2) else 16


def run_sum(lib, torch, kind, a_codes, b_codes, a_scl, b_scl):
    """One MFMA; returns (worst err / largest |product|, worst err / fp32
    spacing at the exact value) over the 32 x 32 outputs."""
    got = _mfma_outputs(lib, torch, kind, a_codes, b_codes, a_scl, b_scl)
    fa, fb = _value_fns(kind)
    K = _kdim(kind)
    scaled = kind in (0, 1, 2)
    av = [[fa(a_codes[i][k]) * (Fraction(2) ** (a_scl[i][k // 32] - 127) if scaled else 1) for k in range(K)]
          for i in range(32)]
    bv = [[fb(b_codes[j][k]) * (Fraction(2) ** (b_scl[j][k // 32] - 127) if scaled else 1) for k in range(K)]
          for j in range(32)]
    worst_rel, worst_ulp = 0.0, 0.0
    for i in range(32):
        for j in range(32):
            prods = [av[i][k] * bv[j][k] for k in range(K)]
            exact = sum(prods)
            big = max(abs(p) for p in prods)
            err = abs(Fraction(float(got[i, j])) - exact)
            if big:
                worst_rel = max(worst_rel, float(err / big))
            if exact:
                ulp = Fraction(2) ** (math.floor(math.log2(abs(exact))) - 23)
                ulp = max(ulp, Fraction(2) ** -149)
                worst_ulp = max(worst_ulp, float(err / ulp))
            elif err:
                worst_ulp = max(worst_ulp, math.inf)
    return worst_rel, worst_ulp


def _random_codes(kind, rng, is_a):
    K = _kdim(kind)
    fa, fb = _value_fns(kind)
    f = fa if is_a else fb
    if f is e2m1:
        return rng.integers(0, 16, size=(32, K)).tolist()
    if f is e4m3:
        c = rng.integers(0, 256, size=(32, K))
        c[(c & 0x7F) == 0x7F] ^= 1           # no NaN codes
        return c.tolist()
    # bf16: exponents within 2**-20 .. 2**20, random mantissas and signs
    v = rng.choice([-1.0, 1.0], size=(32, K)) * rng.uniform(1, 2, size=(32, K)) * \
        np.exp2(rng.integers(-20, 21, size=(32, K)))
    return [[bf16_code(float(x)) for x in row] for row in v]


def _sweep_codes(kind):
    """Row i of A: the largest value at k = 0, then 2**-e_i (same sign) at
    every other k; row j of B likewise with 2**-f_j: output (i, j) sums one
    large product and K - 1 equal small ones, their ratio falling with i + j.
    E2M1 x E2M1 reaches small ratios through the second K-block's scale."""
    K = _kdim(kind)
    a, b = [[0] * K for _ in range(32)], [[0] * K for _ in range(32)]
    sa = [[127, 127] for _ in range(32)]
    sb = [[127, 127] for _ in range(32)]
    for r in range(32):
        if kind in (0, 2, 3):
            a[r] = [0x7E] + [e4m3_code(Fraction(2) ** -min(r % 10, 9))] * (K - 1)
        if kind == 0:
            b[r] = [0x7] + [0x2 if r < 16 else 0x1] * (K - 1)              # 1.0 or 0.5
        if kind in (2, 3):
            b[r] = [0x7E] + [e4m3_code(Fraction(2) ** -(r % 10))] * (K - 1)
        if kind == 1:
            a[r] = [0x7] + [0] * 31 + [0x2] * 32                            # 6, then 1.0 at K-block 1
            b[r] = [0x7] + [0] * 31 + [0x2] * 32
            sa[r][1] = 127 - r
            sb[r][1] = 127 - (r % 8)
        if kind == 4:
            a[r] = [bf16_code(256.0)] + [bf16_code(2.0 ** -r)] * (K - 1)
            b[r] = [bf16_code(256.0)] + [bf16_code(2.0 ** -(r % 8))] * (K - 1)
    return a, b, sa, sb


def _nearest_codes(x, table):
    """Codes of the table values nearest to x (ties to the lower magnitude;
    a probe input generator, not the method's rounding)."""
    mags = np.array([float(v) for v in table])
    order = np.argsort(mags)
    idx = np.clip(np.searchsorted(mags[order], np.abs(x)), 1, len(mags) - 1)
    lo, hi = mags[order][idx - 1], mags[order][idx]
    pick = np.where(np.abs(x) - lo <= hi - np.abs(x), order[idx - 1], order[idx])
    return pick


def w4a8_layer_errors(lib, torch, K=1152, seed=5):
    """A 32 x 32 output patch of a W4A8 layer of depth K on the scaled
    E4M3 x E2M1 MFMA: activations Student-t(3) with 0.5% of channels x50 and
    weights N(0, 0.02), each put on its grid with a power-of-two scale per
    32-block; K / 64 MFMAs per output, their fp32 results summed exactly on
    the host.  Returns the fraction of outputs whose MFMA error exceeds
    1e-5 * sum|a w| (the GEMM's error budget before output rounding) and the
    worst ratio of the error to that budget."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(32, K))
    x[:, rng.choice(K, max(1, K // 200), replace=False)] *= 50
    w = rng.normal(0, 0.02, size=(32, K))
    e4 = [e4m3(c) for c in range(0x7F)]                 # non-negative E4M3 values
    e2 = [_E2M1[c] for c in range(8)]

    def put(v, table, top):
        blocks = v.reshape(32, K // 32, 32)
        amax = np.abs(blocks).max(axis=2, keepdims=True)
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - math.floor(math.log2(top))
        mag = _nearest_codes(blocks / np.exp2(e), table)
        sign = (blocks < 0)
        return mag, sign, (e[..., 0] + 127).astype(int)

    am, asg, asc = put(x, e4, 448.0)
    wm, wsg, wsc = put(w, e2, 6.0)
    a_codes = (am | (asg << 7)).reshape(32, K)
    w_codes = (wm | (wsg << 3)).reshape(32, K)
    aval = np.array([[float(e4m3(int(c))) for c in row] for row in a_codes]) * np.repeat(np.exp2(asc - 127.0), 32, axis=1)
    wval = np.array([[float(e2m1(int(c))) for c in row] for row in w_codes]) * np.repeat(np.exp2(wsc - 127.0), 32, axis=1)
    got = np.zeros((32, 32))
    for k0 in range(0, K, 64):
        a = a_codes[:, k0:k0 + 64].tolist()
        b = w_codes[:, k0:k0 + 64].tolist()
        sa = asc[:, k0 // 32:k0 // 32 + 2].tolist()
        sb = wsc[:, k0 // 32:k0 // 32 + 2].tolist()
        got += _mfma_outputs(lib, torch, 0, a, b, sa, sb)
    prods = aval[:, None, :] * wval[None, :, :]
    exact = prods.sum(axis=2)
    budget = 1e-5 * np.abs(prods).sum(axis=2)
    err = np.abs(got - exact)
    return float(np.mean(err > budget)), float(np.max(err / budget))


def _mfma_outputs(lib, torch, kind, a_codes, b_codes, a_scl, b_scl):
    """D[i][j] (float64) of one MFMA."""
    dev = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    a_ops, b_ops = dev(_pack(kind, a_codes, True)), dev(_pack(kind, b_codes, False))
    sa = dev(np.array([a_scl[l % 32][l // 32] for l in range(64)], dtype=np.int32))
    sb = dev(np.array([b_scl[l % 32][l // 32] for l in range(64)], dtype=np.int32))
    d = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    st = lib.probe_mfma_sum(kind, *(C.c_void_p(t.data_ptr()) for t in (a_ops, b_ops, sa, sb, d)),
                            C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    raw = d.cpu().numpy().astype(np.float64)
    out = np.zeros((32, 32))
    for lane in range(64):
        for q in range(16):
            out[8 * (q // 4) + 4 * (lane // 32) + q % 4, lane % 32] = raw[lane, q]
    return out


def summation(lib, torch, seeds=12):
    out = []
    for kind, name in SUM_KINDS.items():
        rng = np.random.default_rng(1000 + kind)
        rel_r, ulp_r = 0.0, 0.0
        for _ in range(seeds):
            a, b = _random_codes(kind, rng, True), _random_codes(kind, rng, False)
            sa = rng.integers(119, 136, size=(32, 2)).tolist()
            sb = rng.integers(119, 136, size=(32, 2)).tolist()
            r, u = run_sum(lib, torch, kind, a, b, sa, sb)
            rel_r, ulp_r = max(rel_r, r), max(ulp_r, u)
        rel_s, ulp_s = run_sum(lib, torch, kind, *_sweep_codes(kind))
        for case, rel, ulp in (("random", rel_r, ulp_r), ("one large + small same-sign", rel_s, ulp_s)):
            out.append({"probe": "mfma_sum", "mfma": name, "case": case,
                        "mfmas": seeds if case == "random" else 1,
                        "worst_err_over_largest_product": rel,
                        "log2": (round(math.log2(rel), 2) if rel else None),
                        "worst_err_fp32_spacings_at_exact": ulp})
    frac, worst = w4a8_layer_errors(lib, torch)
    out.append({"probe": "mfma_sum", "mfma": SUM_KINDS[0],
                "case": "W4A8 layer patch: 32 x 32 outputs, K = 1152 (18 MFMAs each), Student-t(3) x 0.5% x50 "
                        "activations on E4M3, N(0, 0.02) weights on E2M1",
                "frac_outputs_err_over_1e-5_abs_sum": frac, "worst_err_over_1e-5_abs_sum": worst})
    return out


def rate(lib, torch, iters=4000):
    out = []
    stream = torch.cuda.current_stream()
    for kind, (name, flops, peak) in RATE_KINDS.items():
        for zero in (0, 1):
            for waves in (4, 8):
                blocks = 256                           # one workgroup per compute unit
                buf = torch.empty((blocks * waves * 64,), dtype=torch.float32, device="cuda")
                args = (kind, blocks, waves, iters, zero, C.c_void_p(buf.data_ptr()),
                        C.c_void_p(stream.cuda_stream))
                for _ in range(3):                      # clocks up
                    assert lib.probe_mfma_rate(*args) == 0
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    assert lib.probe_mfma_rate(*args) == 0
                e1.record()
                torch.cuda.synchronize()
                sec = e0.elapsed_time(e1) / 1e3 / 10
                tf = blocks * waves * iters * 8 * flops / sec / 1e12
                out.append({"probe": "mfma_rate", "mfma": name, "operands": "zero" if zero else "random",
                            "waves_per_cu": waves, "us_per_launch": round(sec * 1e6, 1),
                            "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / peak, 3)})
                print(json.dumps(out[-1]), flush=True)
    return out


def gemm_data(torch, shapes=((4096, 3072, 3072, 0), (4096, 3072, 3072, 32), (4096, 12288, 3072, 0)), rounds=3):
    """The library's MXFP4 GEMM on operands whose codes are random, all
    zero, or zero except 1 in 8 bytes: same instructions, same addresses,
    different switching activity (block scales random in every case).
    Median us per launch over HIP-graph replays across 8 buffer sets."""
    import statistics
    import fp8_quantized_linear_mxq_amd as mxq
    from fp8_quantized_linear_mxq_amd import _lib
    out = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)

    def operand(rows, cols, mode):
        q = _lib.empty_qtensor(mxq.MXFP4, rows, cols, "cuda")
        codes = torch.randint(0, 256, q.codes.shape, dtype=torch.uint8, device="cuda", generator=gen)
        if mode == "zero":
            codes.zero_()
        elif mode == "sparse":
            keep = torch.rand(q.codes.shape, device="cuda", generator=gen) < 0.125
            codes = torch.where(keep, codes, torch.zeros_like(codes))
        q.codes.copy_(codes)
        q.scales.copy_(torch.randint(118, 127, q.scales.shape, dtype=torch.uint8, device="cuda", generator=gen))
        return q

    for m, n, k, r in shapes:
        for mode in ("random", "sparse", "zero"):
            sets = []
            for _ in range(8):
                a, w = operand(m, k, mode), operand(n, k, mode)
                u = torch.randn((m, max(r, 1)), device="cuda", generator=gen) if r else None
                l2t = (torch.randn((n, r), device="cuda", generator=gen) * 0.02).to(torch.bfloat16) if r else None
                y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
                sets.append((a, w, u, l2t, y))
            stream = torch.cuda.Stream()

            def call(s):
                a, w, u, l2t, y = s
                mxq.gemm(a, w, u=u, l2t=l2t, out=y, workspace=False)
            with torch.cuda.stream(stream):
                for s in sets:
                    call(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for s in sets:
                    call(s)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                for _ in range(40):
                    g.replay()
            res = []
            for _ in range(rounds):
                with torch.cuda.stream(stream):
                    e0.record(stream)
                    for _ in range(30):
                        g.replay()
                    e1.record(stream)
                torch.cuda.synchronize()
                res.append(e0.elapsed_time(e1) * 1e3 / (30 * len(sets)))
            us = statistics.median(res)
            fl = 2.0 * m * n * k + 2.0 * m * n * r
            rec = {"probe": "gemm_data", "shape": [m, k, n], "rank": r, "codes": mode,
                   "us_per_launch": round(us, 2), "TFLOPs": round(fl / us / 1e6, 1)}
            out.append(rec)
            print(json.dumps(rec), flush=True)
    return out


def cvt_scale(lib, torch):
    """Each scaled E2M1 convert (to f16, bf16, f32) on all 16 codes times
    every positive finite E4M3 value, and times E4M3 values times a
    non-power-of-two fp32 g: the results against the exact products (which
    f16 and bf16 hold exactly for E4M3 scales: at most 6 significant bits,
    magnitudes 2**-10 .. 2688)."""
    vals = [float(e4m3(c)) for c in range(1, 0x7F)]
    scales = vals + [v * 1.1904761791229248 for v in vals[:40]]
    sd = torch.tensor(scales, dtype=torch.float32, device="cuda")
    out = []
    for kind, name in ((0, "pk_f16_fp4"), (1, "pk_bf16_fp4"), (2, "pk_f32_fp4")):
        res = torch.zeros((len(scales) * 16,), dtype=torch.int32, device="cuda")
        st = lib.probe_cvt_scale(kind, C.c_void_p(sd.data_ptr()), len(scales), C.c_void_p(res.data_ptr()),
                                 C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, st
        torch.cuda.synchronize()
        bits = res.cpu().numpy().astype(np.uint32)
        bad_e4m3, bad_g, worst = 0, 0, 0.0
        for i, s in enumerate(scales):
            s32 = float(np.float32(s))
            for c in range(16):
                want = float(e2m1(c)) * s32
                b = int(bits[16 * i + c])
                if kind == 0:
                    got = float(np.array([b], dtype=np.uint16).view(np.float16)[0])
                elif kind == 1:
                    got = float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
                else:
                    got = float(np.array([b], dtype=np.uint32).view(np.float32)[0])
                if got != want:
                    if i < len(vals):
                        bad_e4m3 += 1
                    else:
                        bad_g += 1
                    if want:
                        worst = max(worst, abs(got - want) / abs(want))
        rec = {"probe": "cvt_scale", "convert": name, "e4m3_scales": len(vals),
               "mismatches_e4m3_scales": bad_e4m3, "g_scaled_scales": len(scales) - len(vals),
               "mismatches_g_scaled": bad_g, "worst_rel_err": worst}
        out.append(rec)
        print(json.dumps(rec), flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rate-only", action="store_true")
    ap.add_argument("--sum-only", action="store_true")
    ap.add_argument("--layout", action="store_true")
    ap.add_argument("--gemm-data", action="store_true")
    ap.add_argument("--cvt", action="store_true")
    args = ap.parse_args()
    import torch
    assert torch.cuda.is_available(), "the probes need a GPU"
    lib = _lib()
    if args.cvt:
        cvt_scale(lib, torch)
        return
    if args.gemm_data:
        gemm_data(torch)
        return
    if args.layout:
        for kind in (0, 2, 1):
            res = layout(lib, torch, kind)
            # the map holds if every A slot meets exactly the B slot of the
            # same logical K, scaled by block K // 32's scales (2**(b + 2b))
            ok = True
            for (ha, t), hits in res.items():
                ka = _kmap(kind in (0, 2), ha, t)
                ok &= len(hits) == 1
                for hb, j, v in hits:
                    ok &= _kmap(kind == 2, hb, j) == ka and v == 2.0 ** (3 * (ka // 32))
            print(json.dumps({"probe": "layout", "mfma": SUM_KINDS[kind], "kmap_holds": bool(ok),
                              "pairs": {f"{ha}.{t}": h for (ha, t), h in res.items()}}), flush=True)
        return
    if not args.rate_only:
        for rec in summation(lib, torch):
            print(json.dumps(rec), flush=True)
    if not args.sum_only:
        rate(lib, torch)



def layout(lib, torch, kind):
    """Checks the lane layout _kmap states: which B operand slot each A slot
    of row 0 pairs with, and whose block scales apply.  A row 0 holds a
    single 1.0 at (half ha, slot t); B row j holds a single 1.0 at (half hb,
    slot j) (slots placed through _kmap, so a correct map pairs (ha, t) with
    the B slot of the same logical K).  D[0][j] is nonzero iff the two
    slots meet, and its value 2**(a + b) names the scale lanes used (A
    scales 2**0 / 2**1 on lanes 0 / 32, B 2**0 / 2**2 on lanes j / j + 32)."""
    one_a = 0x38 if kind in (0, 2) else 0x2
    one_b = 0x38 if kind == 2 else 0x2
    res = {}
    for ha in (0, 1):
        for t in range(32):
            hits = []
            for hb in (0, 1):
                a = [[0] * 64 for _ in range(32)]
                b = [[0] * 64 for _ in range(32)]
                a[0][_kmap(kind in (0, 2), ha, t)] = one_a
                for j in range(32):
                    b[j][_kmap(kind == 2, hb, j)] = one_b
                sa = [[127, 128] for _ in range(32)]
                sb = [[127, 129] for _ in range(32)]
                dev = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).cuda()
                a_ops, b_ops = dev(_pack(kind, a, True)), dev(_pack(kind, b, False))
                sad = dev(np.array([sa[l % 32][l // 32] for l in range(64)], dtype=np.int32))
                sbd = dev(np.array([sb[l % 32][l // 32] for l in range(64)], dtype=np.int32))
                d = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
                st = lib.probe_mfma_sum(kind, *(C.c_void_p(x.data_ptr()) for x in (a_ops, b_ops, sad, sbd, d)),
                                        C.c_void_p(torch.cuda.current_stream().cuda_stream))
                assert st == 0
                torch.cuda.synchronize()
                row0 = d.cpu().numpy()[0:32, 0]        # D[0][j] = lane j, register 0
                for j in np.nonzero(row0)[0]:
                    hits.append((hb, int(j), float(row0[j])))
            res[(ha, t)] = hits
    return res


if __name__ == "__main__":
    main()
