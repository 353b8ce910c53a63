"""Exact-rational pins of the oracle's asymmetric branches (ARITH 2025 report on
MX training, main results 3 and conclusions 3: asymmetric min/max scaling
helps INT4 far more than E2M1).

Every step is re-derived here from its definition with Python fractions, one
IEEE rounding at a time, independently of the oracle:

  E2M1 with a mid-range offset
    o  = bf16_RNE( fl32( fl32(max/2) + fl32(min/2) ) )   (each end halved first)
    y  = fl32(x - o);  e = E8M0 rule on max|y| (Qmax 6)
    q  = RTNE onto the signed E2M1 grid of fl32(y * 2^-e), saturating
    x^ = fl32(fl32(q * 2^e) + o)      (q * 2^e is exact in fp32 unless it overflows)

  INT4 with a min/max range
    m  = the largest bf16 <= min;  R = fl32(max - m)
    e  = E8M0 rule on R (Qmax 15; FLOOR: floor(log2 R) - 3)
    q  = clamp(RTNE(fl32(x - m) * 2^-e), 0, 15)
    x^ = fl32(m + fl32(q * 2^e))      (Inf when q * 2^e overflows, e.g. e = 127)

An E8M0 exponent is clamped to [-127, 127]; a range that overflowed fp32 takes
e = 127.  The probe blocks hold bf16 ties of the offset and their fp32
neighbours, E2M1 and integer ties after scaling, sums that overflow fp32,
subnormals and random shifted blocks.  Each test also shows that the probes
tell the stated reading apart from plausible slips (offset rounded down,
exponent from max|x|, no bf16 rounding, the sum formed before halving, ...):
each slip disagrees with the oracle on some probe.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

FLT_MAX = Fr(2) ** 127 * (2 - Fr(1, 2 ** 23))
E2M1_GRID = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]
B = 8                                   # block width of the probes (one block per row)
INF = math.inf


def flog2(a):
    """exact floor(log2 a) for a rational a > 0"""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    return e


def rne(v, p):
    """v rounded to nearest-even in a binary format with p significant bits
    and fp32's exponent range (p = 24: fp32, p = 8: bf16); +-inf on overflow"""
    if v == INF or v == -INF:
        return v
    if v == 0:
        return Fr(0)
    a = abs(v)
    q = Fr(2) ** (max(flog2(a), -126) - (p - 1))
    n = a / q
    r = math.floor(n)
    frac = n - r
    if frac > Fr(1, 2) or (frac == Fr(1, 2) and r % 2 == 1):
        r += 1
    res = r * q
    top = Fr(2) ** 127 * (2 - Fr(2) ** (1 - p))           # the format's largest value
    if res > top:
        return INF if v > 0 else -INF
    return res if v > 0 else -res


def fl(v):
    return rne(v, 24)


def bf16_nearest(v):
    return rne(v, 8)


def bf16_down(v):
    """the largest bf16 value <= v (v finite)"""
    if v == 0:
        return Fr(0)
    q = Fr(2) ** (max(flog2(abs(v)), -126) - 7)
    return math.floor(v / q) * q


def sub(a, b):
    """fl32(a - b) with infinite operands allowed"""
    if a in (INF, -INF) or b in (INF, -INF):
        return float(a) - float(b)
    return fl(a - b)


def e8m0(rule, tau, qmax, emax, a):
    if not a > 0:
        return -127
    if a == INF:
        return 127
    if rule == 0:
        e = flog2(a) - emax
    else:
        q = Fr(qmax) if rule == 1 else Fr(tau)
        e = flog2(a) - flog2(q)
        while q * Fr(2) ** e < a:
            e += 1
        while q * Fr(2) ** (e - 1) >= a:
            e -= 1
    return max(-127, min(127, e))


def e2m1_code(v, neg):
    """RTNE onto the E2M1 grid (ties to the even code), saturating; v >= 0 is
    the magnitude (possibly inf), neg its sign"""
    if v == INF or v >= 6:
        idx = 7
    else:
        idx = min(range(8), key=lambda i: (abs(E2M1_GRID[i] - v), i % 2))
    return (8 if neg else 0) | idx


def uint4_code(v):
    """RTNE onto 0..15 (ties to the even integer), saturating; v >= 0 or inf"""
    if v == INF or v >= 15:
        return 15
    r = math.floor(v)
    f = v - r
    if f > Fr(1, 2) or (f == Fr(1, 2) and r % 2 == 1):
        r += 1
    return min(int(r), 15)


def times2(v, e):
    return v if v in (INF, -INF) else fl(v * Fr(2) ** e)


def derive_e2m1(xs, rule, tau, slip=None):
    """(scale code, offset bits as a rational, codes, dequant) of one block"""
    X = [Fr(float(x)) for x in xs]
    mx, mn = max(X), min(X)
    if slip == "sum_first":
        s = fl(mx + mn)
        mid = INF if s in (INF, -INF) or abs(s) > FLT_MAX else fl(s / 2)
    else:
        mid = fl(fl(mx / 2) + fl(mn / 2))
    if mid == INF:
        o = INF
    elif slip == "offset_down":
        o = bf16_down(mid)
    elif slip == "offset_unrounded":
        o = mid
    else:
        o = bf16_nearest(mid)
    if o in (INF, -INF):
        return None          # the offset itself overflowed: the reading rules this out
    ys = [sub(x, o) for x in X]
    ymax = max(abs(Fr(y)) if y not in (INF, -INF) else INF for y in ys)
    if slip == "exp_from_x":
        ymax = max(abs(x) for x in X)
    e = e8m0(rule, tau, 6, 2, ymax)
    codes, dq = [], []
    for y in ys:
        neg = (y < 0) if y not in (INF, -INF) else y < 0
        v = times2(y, -e)
        c = e2m1_code(abs(v) if v not in (INF, -INF) else INF, neg)
        q = E2M1_GRID[c & 7] * (-1 if c & 8 else 1)
        codes.append(c)
        t = times2(q, e)
        dq.append(sub(t, -o) if t in (INF, -INF) else fl(t + o))
    return e + 127, o, codes, dq


def derive_uint4(xs, rule, tau, slip=None):
    X = [Fr(float(x)) for x in xs]
    mx, mn = max(X), min(X)
    m = bf16_nearest(mn) if slip == "min_nearest" else bf16_down(mn)
    R = sub(mx, mn if slip == "range_from_min" else m)
    emax = 2 if slip == "emax_2" else 3
    e = e8m0(rule, tau, 15, emax, abs(R) if R not in (INF, -INF) else INF) if R != 0 else -127
    codes, dq = [], []
    for x in X:
        d = sub(x, m)
        if d in (INF, -INF):
            v = d
        else:
            v = times2(d, -e)
        c = 0 if (v not in (INF,) and v < 0) else uint4_code(v)
        codes.append(c)
        t = times2(Fr(c), e)
        dq.append(sub(t, -m) if t in (INF, -INF) else fl(m + t))
    return e + 127, m, codes, dq


def bf16_value(bits):
    u = int(bits) << 16
    return Fr(float(np.array([u], np.uint32).view(np.float32)[0]))


def nib(codes_row, i):
    return (int(codes_row[i // 2]) >> (4 * (i % 2))) & 0xF


def as_frac(v):
    return INF if v == np.inf else (-INF if v == -np.inf else Fr(float(v)))


def f32(v):
    return np.float32(v)


def e2m1_probe_blocks():
    rng = np.random.default_rng(2025)
    blocks = []
    # a symmetric block whose elements land on every E2M1 tie after scaling
    blocks.append([4, -4, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5])
    blocks.append([4, -4, -0.25, -0.75, -1.25, -2.5, -3.5, 5])
    # bf16 ties of the mid-range, and their fp32 neighbours: mid = 1 + 2^-8 is
    # half-way between the bf16 values 1 and 1 + 2^-7
    for base in (1.0, 3.0, -1.5, 1e-3, 200.0):
        ulp = 2.0 ** (math.floor(math.log2(abs(base))) - 7)
        mid = f32(base + ulp / 2)
        for d in (0.5, 0.125, 2.0 ** -6):
            dd = f32(abs(base) * d)
            for nudge in (0, 1, -1):
                hi = f32(mid + dd)
                if nudge:
                    hi = np.nextafter(hi, f32(np.inf) if nudge > 0 else f32(-np.inf))
                lo = f32(mid - dd)
                inner = rng.uniform(float(lo), float(hi), B - 2).astype(np.float32)
                blocks.append([hi, lo, *inner])
    # a midpoint that is not a bf16 value and lies above the half-way point:
    # nearest rounds up, round-down does not
    for base in (1.0, 5.0, -7.0):
        ulp = 2.0 ** (math.floor(math.log2(abs(base))) - 7)
        mid = base + 0.75 * ulp
        blocks.append([f32(mid + 0.1), f32(mid - 0.1), *[f32(mid + 0.05 * k) for k in range(-3, 3)]])
    # both ends near FLT_MAX: their sum overflows fp32 (halving first does not)
    blocks.append([f32(3.0e38), f32(2.9e38), f32(3.1e38), f32(2.95e38), f32(3.2e38), f32(3.0e38),
                   f32(2.99e38), f32(3.05e38)])
    blocks.append([f32(-3.3e38), f32(-3.0e38), f32(-3.2e38), f32(-3.1e38), f32(-3.25e38), f32(-3.3e38),
                   f32(-3.0e38), f32(-3.15e38)])
    blocks.append([f32(3.4e38), f32(-3.4e38), f32(1e38), f32(-2e38), f32(0.5), 0, f32(3e38), f32(-1)])
    # subnormals and the smallest normals
    blocks.append([f32(1e-40), f32(3e-39), f32(2e-39), f32(1.17549435e-38), f32(-1e-41), f32(4e-40),
                   f32(2.5e-39), f32(1e-39)])
    blocks.append([f32(2.0 ** -149 * k) for k in (1, 2, 3, 5, 8, 13, 21, 34)])
    # shifted random blocks: offset much larger than, comparable to, and
    # smaller than the spread
    for shift, spread in ((10, 1), (1, 1), (0.1, 1), (1e-3, 1e-4), (-50, 3), (1e5, 7), (0, 1)):
        for _ in range(25):
            blocks.append(list((shift + spread * rng.standard_normal(B)).astype(np.float32)))
    return np.array(blocks, np.float32)


def uint4_probe_blocks():
    rng = np.random.default_rng(17)
    blocks = []
    # integer ties after scaling: min 0 (a bf16 value), range 15 -> e = 0 (CEIL)
    blocks.append([0, 15, 0.5, 1.5, 2.5, 3.5, 14.5, 7.5])
    blocks.append([0, 14, 0.5, 13.5, 6.5, 9.49999, 9.5, 10.5])
    # a minimum that is not a bf16 value: round-down and nearest differ
    for mn in (1.0 + 2.0 ** -9, 1.0 + 2.0 ** -8 + 2.0 ** -10, -3.0 - 2.0 ** -7 - 2.0 ** -9, 1e-3 * (1 + 2.0 ** -10)):
        mn = f32(mn)
        blocks.append([mn, *[f32(mn + k * 0.37 * abs(mn) / 7) for k in range(1, B)]])
    # a range that overflows fp32 (both ends near FLT_MAX, opposite signs)
    blocks.append([f32(3.0e38), f32(-3.0e38), 0, f32(1e38), f32(-1e38), f32(2e38), f32(-2e38), 1])
    # subnormals
    blocks.append([f32(1e-40), f32(3e-39), f32(2e-39), f32(1.17549435e-38), f32(-1e-41), f32(4e-40),
                   f32(2.5e-39), f32(1e-39)])
    # constant blocks (range zero when the value is a bf16 number)
    blocks.append([f32(1.5)] * B)
    blocks.append([f32(1.0 + 2.0 ** -12)] * B)
    for shift, spread in ((10, 1), (1, 1), (0, 1), (1e-3, 1e-4), (-50, 3), (1e5, 7), (0.25, 0.01)):
        for _ in range(25):
            blocks.append(list((shift + spread * rng.standard_normal(B)).astype(np.float32)))
    return np.array(blocks, np.float32)


def oracle_blocks(ref, x, kw):
    q = ref.quantize(x, ref.Format(block_cols=B, asymmetric=1, **kw))
    return q["scales"][:, 0], q["offsets"][:, 0], q["codes"], q["dequant"]


def check_blocks(ref, x, kw, derive, rule, tau, slip=None):
    """number of blocks where derive(..., slip) disagrees with the oracle"""
    sc, off, codes, dq = oracle_blocks(ref, x, kw)
    bad = 0
    for i in range(x.shape[0]):
        d = derive(x[i], rule, tau, slip)
        if d is None:
            bad += 1
            continue
        s, o, cs, ds = d
        got = (int(sc[i]), bf16_value(off[i]), [nib(codes[i], j) for j in range(B)],
               [as_frac(v) for v in dq[i]])
        if got != (s, o, cs, ds):
            bad += 1
    return bad


RULES = [(0, 0.0), (1, 0.0), (2, 7.5), (2, 6.5)]


@pytest.mark.parametrize("rule,tau", RULES)
def test_asymmetric_e2m1_exact(ref, rule, tau):
    x = e2m1_probe_blocks()
    kw = dict(rule=rule, oas_tau=tau)
    assert check_blocks(ref, x, kw, derive_e2m1, rule, tau) == 0


@pytest.mark.parametrize("slip", ["offset_down", "offset_unrounded", "exp_from_x", "sum_first"])
def test_asymmetric_e2m1_probes_catch_slips(ref, slip):
    x = e2m1_probe_blocks()
    assert check_blocks(ref, x, dict(rule=0), derive_e2m1, 0, 0.0, slip) > 0


INT4_RULES = [(0, 0.0), (1, 0.0), (2, 20.0), (2, 29.5)]


@pytest.mark.parametrize("rule,tau", INT4_RULES)
def test_asymmetric_int4_exact(ref, rule, tau):
    x = uint4_probe_blocks()
    kw = dict(elem=ref.INT4, rule=rule, oas_tau=tau)
    assert check_blocks(ref, x, kw, derive_uint4, rule, tau) == 0


@pytest.mark.parametrize("slip", ["min_nearest", "range_from_min", "emax_2"])
def test_asymmetric_int4_probes_catch_slips(ref, slip):
    x = uint4_probe_blocks()
    assert check_blocks(ref, x, dict(elem=ref.INT4, rule=0), derive_uint4, 0, 0.0, slip) > 0


def test_asymmetric_e2m1_near_flt_max_is_finite(ref):
    """Both ends near FLT_MAX: the offset and every dequantized value stay
    finite (a sum formed before halving would overflow to Inf)."""
    x = np.full((1, 32), np.float32(3.0e38), np.float32)
    x[0, ::2] = np.float32(3.3e38)
    q = ref.quantize(x, ref.Format(asymmetric=1))
    assert np.isfinite(float(bf16_value(q["offsets"][0, 0])))
    assert np.all(np.isfinite(q["dequant"]))
    rel = np.abs(q["dequant"].astype(np.float64) - x) / x
    assert rel.max() < 0.1
