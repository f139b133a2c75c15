"""Exact-rational helpers for pinning the oracle (tests only).

Written from the format definitions independently of ``oracle/``: values are
Python ``Fraction`` objects and every rounding is decided by exact
comparison.
"""
from fractions import Fraction

F = Fraction


def e2m1_grid():
    # magnitudes of codes 0..7: subnormal m*1/2, then 2**(e-1) * (1 + m/2)
    vals = [F(0), F(1, 2)]
    for e in (1, 2, 3):
        for m in (0, 1):
            vals.append(F(2) ** (e - 1) * (1 + F(m, 2)))
    return vals


def e4m3_grid():
    vals = [F(m, 8) * F(1, 64) for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(F(2) ** (e - 7) * (1 + F(m, 8)))
    return vals


def round_to_grid(v, grid):
    """Index of the nearest grid magnitude to |v| (ties to even index, saturating)."""
    a = abs(v)
    if a >= grid[-1]:
        return len(grid) - 1
    for i in range(len(grid) - 1):
        lo, hi = grid[i], grid[i + 1]
        if a <= hi:
            mid = (lo + hi) / 2
            if a < mid:
                return i
            if a > mid:
                return i + 1
            return i if i % 2 == 0 else i + 1
    raise AssertionError


def rn_f32(q):
    """Round a non-negative Fraction to float32 (nearest even) as a Fraction."""
    if q == 0:
        return F(0)
    e = 0
    while F(2) ** e > q:
        e -= 1
    while F(2) ** (e + 1) <= q:
        e += 1
    quantum = F(2) ** (max(e, -126) - 23)
    n = q / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2):
        fl += 1
    return fl * quantum


def floor_log2(a):
    e = 0
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    return e


def signbit(x):
    import math
    return math.copysign(1.0, float(x)) < 0


def mx_block(xs, grid, emax, sign_bit):
    """Exact MX quantization of one block of floats -> (codes, scale_code)."""
    fr = [F(float(x)) for x in xs]
    amax = max(abs(v) for v in fr)
    e = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - emax))
    codes = []
    for x, v in zip(xs, fr):
        c = round_to_grid(v / F(2) ** e, grid)
        codes.append(c | (sign_bit if signbit(x) else 0))
    return codes, e + 127


def nvfp4_tensor(xs2d, g=None):
    """Exact NVFP4 of a list of rows (16-blocks) -> (codes, scale codes, g)."""
    e2 = e2m1_grid()
    e4 = e4m3_grid()
    fr = [[F(float(x)) for x in row] for row in xs2d]
    if g is None:
        amax = max(abs(v) for row in fr for v in row)
        g = rn_f32(amax / 2688)
    g = F(g)
    codes, scodes = [], []
    for row, xrow in zip(fr, xs2d):
        rc, rs = [], []
        for b in range(0, len(row), 16):
            blk = row[b:b + 16]
            ab = max(abs(v) for v in blk)
            s_code = 0 if g == 0 else round_to_grid(ab / (6 * g), e4)
            s = e4[s_code]
            rs.append(s_code)
            for j, v in enumerate(blk):
                x = xrow[b + j]
                c = 0 if s == 0 else round_to_grid(v / (s * g), e2)
                rc.append(c | (8 if signbit(x) else 0))
        codes.append(rc)
        scodes.append(rs)
    return codes, scodes, g


def int4_row(xs):
    """Exact INT4 of one row (32-blocks) -> (signed ints, scales as Fractions)."""
    fr = [F(float(x)) for x in xs]
    q, scales = [], []
    for b in range(0, len(fr), 32):
        blk = fr[b:b + 32]
        ab = max(abs(v) for v in blk)
        s = rn_f32(ab / 7)
        scales.append(s)
        for v in blk:
            if s == 0:
                q.append(0)
                continue
            t = v / s
            fl = t.numerator // t.denominator
            rem = t - fl
            r = fl + 1 if (rem > F(1, 2) or (rem == F(1, 2) and fl % 2)) else fl
            q.append(max(-7, min(7, r)))
    return q, scales
