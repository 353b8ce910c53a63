"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: values the
pages state (tests/golden/format_facts.json), a hand-worked block re-derived
here with exact rationals, published known-answer vectors (Philox), exact
brute force over every grid point, tie and neighbour, closed forms, and
structural invariants (transposition, scale equivariance, idempotence).
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def minifloat(ebits, mbits, bias, exp0_is_zero=False):
    """Non-negative values of a sign-magnitude minifloat, decoded from its bit
    fields (independent of the oracle's tables)."""
    out = []
    for code in range(1 << (ebits + mbits)):
        e, m = code >> mbits, code & ((1 << mbits) - 1)
        if e == 0:
            v = Fr(0) if exp0_is_zero else Fr(m, 1 << mbits) * Fr(2) ** (1 - bias)
        else:
            v = (1 + Fr(m, 1 << mbits)) * Fr(2) ** (e - bias)
        out.append(v)
    return out


def grid_of(ref, elem, asym=0):
    if elem == ref.E2M1:
        return minifloat(2, 1, 1)
    if elem == ref.E3M0:
        return minifloat(3, 0, 3, exp0_is_zero=True)
    if elem == ref.FP6_E2M3:
        return minifloat(2, 3, 1)
    if elem == ref.FP6_E3M2:
        return minifloat(3, 2, 3)
    if elem == ref.INT4:
        return [Fr(i) for i in range(16 if asym else 8)]
    if elem == ref.FP8_E4M3:       # magnitude code 0x7F is NaN
        return minifloat(4, 3, 7)[:0x7F]
    if elem == ref.FP8_E5M2:       # 0x7C is Inf, 0x7D-0x7F NaN
        return minifloat(5, 2, 15)[:0x7C]
    raise ValueError(elem)


def f32(v):
    return float(np.float32(v))


def nextafter32(v, d):
    return float(np.nextafter(np.float32(v), np.float32(d)))


def sign_code(ref, elem, asym, neg, idx):
    if elem == ref.INT4:
        return idx if asym else ((-idx if neg else idx) & 0xF)
    bits = ref.elem_bits(elem)
    return (int(neg) << (bits - 1)) | idx


ELEMS = [("E2M1", 0, 0), ("INT4", 1, 0), ("UINT4", 1, 1), ("E2M3", 2, 0), ("E3M2", 3, 0), ("E3M0", 4, 0),
         ("E4M3", 5, 0), ("E5M2", 6, 0)]


# ---------------------------------------------------------------- formats --
def test_format_facts_from_pages(ref):
    facts = golden("format_facts.json")
    vals = sorted({abs(ref.code_value(ref.E2M1, 0, c)) for c in range(16)})
    nz = [v for v in vals if v > 0]
    assert max(vals) == facts["e2m1_max"]
    assert min(nz) == facts["e2m1_min_nonzero"]
    assert max(vals) / min(nz) == facts["e2m1_dynamic_range"]
    # UE4M3 / UE5M3 smallest non-zero scale
    assert ref.fp8_scale_value(ref.SC_UE4M3, 1) == 2.0 ** facts["ue4m3_min_scale_log2"]
    assert ref.fp8_scale_value(ref.SC_UE5M3, 1) == 2.0 ** facts["ue5m3_min_scale_log2"]
    # an element of 5 (between 4 and 6) comes back as 4 under RTNE: a 20% error
    q = ref.round_code(ref.E2M1, 0, ref.RTNE, 5.0)
    assert abs(5.0 - ref.code_value(ref.E2M1, 0, q)) / 5.0 == facts["gap_4_6_relative_error"]


@pytest.mark.parametrize("name,elem,asym", ELEMS)
def test_grid_values_decode_from_bit_fields(ref, name, elem, asym):
    g = grid_of(ref, elem, asym)
    nbits = 4 if elem in (0, 1, 4) else (8 if elem in (5, 6) else 6)
    for code in range(1 << nbits):
        if nbits == 8 and (code & 0x7F) >= len(g):
            assert math.isnan(ref.code_value(elem, asym, code))     # Inf / NaN codes
            continue
        v = Fr(ref.code_value(elem, asym, code))
        if elem == ref.INT4:
            want = Fr(code) if asym else Fr(code - 16 if code & 8 else code)
        else:
            s = code >> (nbits - 1)
            want = (-1 if s else 1) * g[code & ((1 << (nbits - 1)) - 1)]
        assert v == want, (name, code)


def test_fp8_scale_grids(ref):
    ue4 = [Fr(ref.fp8_scale_value(ref.SC_UE4M3, c)) for c in range(0x7F)]
    assert ue4 == minifloat(4, 3, 7)[:0x7F]
    assert max(ue4) == 448 and ue4[8] == Fr(1, 64)          # max, smallest normal 2^-6
    assert math.isnan(ref.fp8_scale_value(ref.SC_UE4M3, 0x7F))
    ue5 = [Fr(ref.fp8_scale_value(ref.SC_UE5M3, c)) for c in range(0xFF)]
    assert ue5 == minifloat(5, 3, 15)[:0xFF]
    assert ue5[8] == Fr(1, 2 ** 14) and max(ue5) == Fr(7, 4) * 2 ** 16
    assert math.isnan(ref.fp8_scale_value(ref.SC_UE5M3, 0xFF))


def nearest_even(grid, t):
    """index of the nearest grid value to t >= 0, ties to the even index,
    saturating at the top (exact rationals, grid ascending)."""
    if t >= grid[-1]:
        return len(grid) - 1
    best = min(range(len(grid)), key=lambda i: (abs(grid[i] - t), i % 2))
    return best


@pytest.mark.parametrize("kind,bits,bias,ncodes", [(1, 4, 7, 0x7F), (3, 5, 15, 0xFF)])
def test_fp8_scale_rne_brute_force(ref, kind, bits, bias, ncodes):
    grid = minifloat(bits, 3, bias)[:ncodes]
    probes = []
    for i in range(ncodes - 1):
        a, b = grid[i], grid[i + 1]
        mid = (a + b) / 2
        for v in (a, b, mid):
            fv = f32(float(v))
            probes += [fv, nextafter32(fv, 0), nextafter32(fv, np.inf)]
    probes += [f32(float(grid[-1]) * 1.01), float("inf"), 0.0, 1e-45]
    for t in probes:
        if t < 0:
            continue
        want = nearest_even(grid, Fr(t)) if math.isfinite(t) else ncodes - 1
        assert ref.fp8_scale_code(kind, t) == want, (kind, t)


# ----------------------------------------------------- element rounding --
def probe_values(grid):
    vals = []
    for i in range(len(grid) - 1):
        a, b = grid[i], grid[i + 1]
        for v in (a, b, (a + b) / 2, a + (b - a) / 4, a + 3 * (b - a) / 4):
            fv = f32(float(v))
            vals += [fv, nextafter32(fv, 0), nextafter32(fv, np.inf)]
    top = float(grid[-1])
    vals += [top * 1.1, top * 2, 1e30, 1e-45, 0.0]
    return sorted(set(v for v in vals if v >= 0))


@pytest.mark.parametrize("name,elem,asym", ELEMS)
def test_rtne_brute_force(ref, name, elem, asym):
    grid = grid_of(ref, elem, asym)
    for m in probe_values(grid):
        for neg in ((False,) if asym else (False, True)):
            v = -m if neg else m
            idx = nearest_even(grid, Fr(m))
            want = sign_code(ref, elem, asym, neg, idx)
            assert ref.round_code(elem, asym, ref.RTNE, v) == want, (name, v)


def test_e2m1_ties_and_saturation(ref):
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 1, 1, 2, 2, 4, 4]
    got = [ref.code_value(ref.E2M1, 0, ref.round_code(ref.E2M1, 0, ref.RTNE, t)) for t in ties]
    assert got == want
    for big in (6.0, 6.9, 7.0, 8.0, 1e20):
        assert ref.round_code(ref.E2M1, 0, ref.RTNE, big) == 0x7
        assert ref.round_code(ref.E2M1, 0, ref.RTNE, -big) == 0xF
    assert ref.round_code(ref.E2M1, 0, ref.RTNE, -0.1) == 0x8      # negative flush keeps the sign


@pytest.mark.parametrize("name,elem,asym", ELEMS)
def test_ceil_brute_force(ref, name, elem, asym):
    grid = grid_of(ref, elem, asym)
    for m in probe_values(grid):
        for neg in ((False,) if asym else (False, True)):
            v = -m if neg else m
            if Fr(m) >= grid[-1]:
                idx = len(grid) - 1
            elif neg:       # smallest grid value >= v: magnitude rounds down
                idx = max(i for i in range(len(grid)) if grid[i] <= Fr(m))
            else:
                idx = min(i for i in range(len(grid)) if grid[i] >= Fr(m))
            want = sign_code(ref, elem, asym, neg, idx)
            assert ref.round_code(elem, asym, ref.CEIL, v) == want, (name, v)


@pytest.mark.parametrize("name,elem,asym", [e for e in ELEMS if e[0] in ("E2M1", "INT4", "E3M2", "E4M3", "E5M2")])
def test_sr_exact_expectation(ref, name, elem, asym):
    """Enumerate every 16-bit draw: the mean lies in [v, v + step * 2^-16)."""
    grid = grid_of(ref, elem, asym)
    rng = np.random.default_rng(7)
    for _ in range(6):
        i = int(rng.integers(0, len(grid) - 1))
        a, b = grid[i], grid[i + 1]
        v = f32(float(a + (b - a) * Fr(float(rng.random()))))
        if v >= float(b):
            continue
        total = Fr(0)
        ups = 0
        for r in range(65536):
            code = ref.round_code(elem, asym, ref.SR, v, r)
            q = Fr(ref.code_value(elem, asym, code))
            assert q in (a, b)
            ups += q == b
            total += q
        mean = total / 65536
        assert Fr(v) <= mean < Fr(v) + (b - a) / 65536, (name, v)
        assert ups == math.ceil((Fr(v) - a) / (b - a) * 65536)


def test_sr_saturates_and_keeps_sign(ref):
    for r in (0, 1, 65535):
        assert ref.round_code(ref.E2M1, 0, ref.SR, 7.0, r) == 0x7
        assert ref.round_code(ref.E2M1, 0, ref.SR, -7.0, r) == 0xF
    # an exact grid value never moves
    for r in (0, 12345, 65535):
        assert ref.round_code(ref.E2M1, 0, ref.SR, 3.0, r) == 0x5


# ---------------------------------------------------------------- scales --
def exact_floor_log2(a):
    a = Fr(a)
    e = 0
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    return e


def exact_e_ceil(a, q):
    a, q = Fr(a), Fr(q)
    e = 0
    while q * Fr(2) ** e < a:
        e += 1
    while q * Fr(2) ** (e - 1) >= a:
        e -= 1
    return e


def amax_probes():
    rng = np.random.default_rng(3)
    vals = [1e-45, 1e-40, 1.17549435e-38, 0.02, 0.05, 1.0, 3.0, 4.0, 6.0, 7.5, 8.0, 1e30, 3.4e38]
    vals += [f32(2.0 ** k * 6) for k in range(-20, 20, 3)]
    vals += [f32(2.0 ** k * 3) for k in range(-20, 20, 3)]
    vals += [f32(x) for x in rng.lognormal(0, 8, 40)]
    out = []
    for v in vals:
        v = f32(v)
        out += [v, nextafter32(v, 0), nextafter32(v, np.inf)]
    return [v for v in out if v > 0 and math.isfinite(v)]


def clamp127(e):
    return max(-127, min(127, e))


@pytest.mark.parametrize("name,elem,asym", ELEMS)
def test_e8m0_rules_exact(ref, name, elem, asym):
    grid = grid_of(ref, elem, asym)
    qmax = grid[-1]
    emax = exact_floor_log2(qmax)
    tau = f32(float(qmax) * 1.25)
    for a in amax_probes():
        assert ref.e8m0_exponent(ref.RULE_FLOOR, 0, elem, asym, a) == clamp127(exact_floor_log2(a) - emax)
        assert ref.e8m0_exponent(ref.RULE_CEIL, 0, elem, asym, a) == clamp127(exact_e_ceil(a, qmax))
        assert ref.e8m0_exponent(ref.RULE_OAS, tau, elem, asym, a) == clamp127(exact_e_ceil(a, tau))


# ----------------------------------------------------------------- Philox --
def test_philox_known_answers(ref):
    with open(os.path.join(GOLD, "philox4x32_10_kat.txt")) as fh:
        rows = [ln.split() for ln in fh if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(t, 16) for t in r]
        assert ref.philox4x32_10(v[0:4], v[4:6]) == v[6:10]


def test_r16_counter_mapping(ref):
    seed, off = synth.SR_SEED, 0x1122334455667788
    for j in (0, 1, 7, (1 << 32) + 5):
        words = ref.philox4x32_10([j & 0xFFFFFFFF, j >> 32, off & 0xFFFFFFFF, off >> 32],
                                  [seed & 0xFFFFFFFF, seed >> 32])
        for t in range(8):
            w = words[t // 2]
            want = (w >> 16) if t % 2 else (w & 0xFFFF)
            assert ref.r16(seed, off, 8 * j + t) == want


# --------------------------------------------------------------- Hadamard --
@pytest.mark.parametrize("h", [16, 32, 128])
def test_hadamard_is_sylvester_and_orthogonal(ref, h):
    c = ref.hadamard_const(h)
    eye = np.eye(h, dtype=np.float32)
    cols = ref.hadamard_rows(eye, h)          # row i = c * H e_i
    H = np.rint(cols / np.float32(c)).astype(np.int64)
    assert np.all(np.abs(H) == 1)
    assert np.array_equal(H @ H.T, h * np.eye(h, dtype=np.int64))
    # Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]]
    n = h // 2
    assert np.array_equal(H[:n, :n], H[:n, n:]) and np.array_equal(H[n:, :n], H[:n, :n])
    assert np.array_equal(H[n:, n:], -H[:n, :n])
    # small integers: butterflies are exact, then one rounding by c
    x = np.random.default_rng(h).integers(-50, 50, (4, h)).astype(np.float32)
    got = ref.hadamard_rows(x, h)
    exact = (x.astype(np.int64) @ H.T).astype(np.float32) * np.float32(c)
    assert np.array_equal(got.view(np.uint32), exact.view(np.uint32))


def test_hadamard_constants_are_nearest_fp32(ref):
    for h, bits in ((16, 0x3E800000), (32, 0x3E3504F3), (64, 0x3E000000), (128, 0x3DB504F3)):
        c = np.float32(ref.hadamard_const(h))
        assert int(c.view(np.uint32)) == bits
        lo = Fr(float(np.nextafter(c, np.float32(0))))
        hi = Fr(float(np.nextafter(c, np.float32(1))))
        cf = Fr(float(c))
        # c is nearest to 1/sqrt(h): both midpoints bracket 1/sqrt(h)
        assert ((lo + cf) / 2) ** 2 * h <= 1 <= ((cf + hi) / 2) ** 2 * h


# ------------------------------------------------------ the worked block --
def exact_qsnr(x, y):
    s = sum(Fr(float(np.float32(a))) ** 2 for a in x)
    e = sum((Fr(float(np.float32(a))) - Fr(float(b))) ** 2 for a, b in zip(x, y))
    return 10 * math.log10(s / e)


@pytest.mark.parametrize("rule,key", [(0, "floor"), (1, "ceil")])
def test_worked_block(ref, rule, key):
    g = golden("worked_block_e2m1_e8m0.json")
    want = g[key]
    x = np.array([g["x"]], np.float32)
    q = ref.quantize(x, ref.Format(block_cols=4, rule=rule))
    assert int(q["scales"][0, 0]) == want["scale_code"] == want["exponent"] + 127
    assert list(q["codes"][0]) == want["bytes"]
    codes = [(b >> (4 * k)) & 0xF for b in want["bytes"] for k in (0, 1)]
    assert codes == want["codes"]
    assert list(q["dequant"][0]) == want["dequant"]
    assert q["stats"]["flushed"] == want["flushed"]
    assert abs(ref.qsnr_db(q["stats"]) - want["qsnr_db"]) < 1e-4
    # independent exact re-derivation
    amax = max(abs(Fr(float(v))) for v in x[0])
    e = exact_floor_log2(amax) - 2 if rule == 0 else exact_e_ceil(amax, 6)
    assert e == want["exponent"]
    grid = minifloat(2, 1, 1)
    deq = []
    for v in x[0]:
        m = abs(Fr(float(v))) / Fr(2) ** e
        deq.append(float((-1 if v < 0 else 1) * grid[nearest_even(grid, m)] * Fr(2) ** e))
    assert deq == want["dequant"]
    assert abs(exact_qsnr(x[0], deq) - want["qsnr_db"]) < 1e-4


# ------------------------------------------------ tensor-level invariants --
ALL_FORMATS = [
    dict(),
    dict(rule=1), dict(rule=2, oas_tau=7.5), dict(block_cols=16), dict(block_cols=8),
    dict(elem=1), dict(elem=2), dict(elem=3), dict(elem=4), dict(elem=4, round=2),
    dict(round=1, seed=5, rng_offset=9), dict(round=2),
    dict(scale=1, block_cols=16), dict(scale=2, block_cols=16), dict(scale=3, block_cols=16),
    dict(scale=4, rule=1), dict(elem=1, asymmetric=1, rule=1), dict(asymmetric=1),
    dict(block_rows=32, block_cols=1), dict(block_rows=32, block_cols=32),
    dict(block_rows=8, block_cols=8, round=1, seed=3),
    dict(hadamard=32), dict(hadamard=128), dict(macro_cols=128, block_cols=16),
    dict(macro_cols=128, block_cols=16, rule=2, oas_tau=7.5),
]


def fmt_id(d):
    return ",".join(f"{k}={v}" for k, v in d.items()) or "mxfp4"


@pytest.mark.parametrize("kw", ALL_FORMATS, ids=fmt_id)
def test_dequantize_matches_quantize_output(ref, kw):
    x = synth.w4(shape=(64, 256), seed=11)
    f = ref.Format(**kw)
    q = ref.quantize(x, f)
    y = ref.dequantize(f, q, 64, 256)
    assert np.array_equal(y.view(np.uint32), q["dequant"].view(np.uint32))


@pytest.mark.parametrize("kw", [dict(), dict(rule=1), dict(rule=2, oas_tau=7.0),
                                dict(round=1, seed=1), dict(elem=1), dict(elem=3),
                                dict(block_rows=16, block_cols=16)], ids=fmt_id)
def test_scale_equivariance_e8m0(ref, kw):
    """x * 2^k leaves element codes unchanged and shifts E8M0 codes by k."""
    x = synth.bf16_bits_to_f32(synth.w3(shape=(64, 128), seed=5))
    f = ref.Format(**kw)
    q0 = ref.quantize(x, f)
    for k in (-9, 5):
        q1 = ref.quantize((x * np.float32(2.0 ** k)).astype(np.float32), f)
        assert np.array_equal(q0["codes"], q1["codes"])
        nz = q0["scales"] > 0
        assert np.array_equal(q1["scales"][nz].astype(int), q0["scales"][nz].astype(int) + k)


def test_nvfp4_equivariant_and_top_block(ref):
    x = synth.bf16_bits_to_f32(synth.w2(0.02, shape=(32, 256), seed=4))
    f = ref.Format(scale=ref.SC_NVFP4, block_cols=16)
    q0 = ref.quantize(x, f)
    q1 = ref.quantize((x * np.float32(2.0 ** -20)).astype(np.float32), f)
    assert np.array_equal(q0["codes"], q1["codes"]) and np.array_equal(q0["scales"], q1["scales"])
    assert q1["tensor_scale"][0] == np.float32(q0["tensor_scale"][0] * np.float32(2.0 ** -20))
    # the block holding the tensor maximum gets the largest E4M3 scale, 448
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q0["scales"][r, c // 16] == 0x7E
    assert q0["tensor_scale"][0] == np.float32(np.float32(np.abs(x).max()) / np.float32(2688))


def test_ue4m3_vs_ue5m3_flush_boundary(ref):
    """Without a tensor scale, UE4M3 flushes a block whose t = amax/6 rounds
    below 2^-9 to zero; UE5M3 reaches down to 2^-17 (the page-2 zero-rounding
    error term and its UE5M3 remedy)."""
    for amax, ue4_zero, ue5_zero in ((6 * 2.0 ** -10, True, False),
                                     (6 * 2.0 ** -10 * 1.01, False, False),
                                     (6 * 2.0 ** -18, True, True),
                                     (6 * 2.0 ** -18 * 1.01, True, False)):
        x = np.full((1, 16), np.float32(amax) / 3, np.float32)
        x[0, 0] = np.float32(amax)
        for kind, want in ((ref.SC_UE4M3, ue4_zero), (ref.SC_UE5M3, ue5_zero)):
            q = ref.quantize(x, ref.Format(scale=kind, block_cols=16))
            assert (q["stats"]["zero_blocks"] == 1) == want, (amax, kind)


def test_zero_block_probability_matches_normal_model(ref):
    """P(block flushes) = erf(a / (sigma sqrt 2))^b with a = 6 * 2^-10 for
    UE4M3 scales without a tensor scale (N(0, sigma^2) data)."""
    sigma, b = 2.5e-3, 16
    x = synth.normal((4096, 256), sigma, 77, dtype="f32")
    q = ref.quantize(x, ref.Format(scale=ref.SC_UE4M3, block_cols=b))
    nblk = x.size // b
    frac = q["stats"]["zero_blocks"] / nblk
    p = math.erf(6 * 2.0 ** -10 / (sigma * math.sqrt(2))) ** b
    assert abs(frac - p) < 4 * math.sqrt(p * (1 - p) / nblk) + 1e-4


def test_floor_rule_idempotent(ref):
    x = synth.bf16_bits_to_f32(synth.w4(shape=(32, 256), seed=2))
    for kw in (dict(), dict(elem=2), dict(elem=1), dict(block_rows=8, block_cols=8)):
        f = ref.Format(**kw)
        q = ref.quantize(x, f)
        q2 = ref.quantize(q["dequant"], f)
        assert np.array_equal(q["codes"], q2["codes"]) and np.array_equal(q["scales"], q2["scales"])
        assert np.array_equal(q["dequant"], q2["dequant"])


@pytest.mark.parametrize("b", [16, 32])
def test_bits_per_element(ref, b):
    facts = golden("format_facts.json")
    x = synth.w1(shape=(64, 256))
    q = ref.quantize(x, ref.Format(block_cols=b))
    bits = 8 * (q["codes"].nbytes + q["scales"].nbytes) / x.size
    assert bits == facts["bits_per_element"][str(b)]


def test_qsnr_closed_forms(ref):
    a = np.random.default_rng(0).integers(-1000, 1000, 4096).astype(np.float32)
    a[a == 0] = 1
    eps = 2.0 ** -8
    b = (a * np.float32(1 - eps)).astype(np.float32)
    assert np.array_equal(b, a - a * np.float32(eps))          # exact
    _, d = ref.qsnr(a, b)
    assert abs(d - (-20 * math.log10(eps))) < 1e-9
    _, d0 = ref.qsnr(a, np.zeros_like(a))
    assert d0 == 0.0
    st, dinf = ref.qsnr(a, a.copy())
    assert dinf == float("inf") and st["flushed"] == 0


def test_transposition_column_blocks(ref):
    """b x 1 blocks of x are 1 x b blocks of x^T (RTNE, any scale rule)."""
    x = synth.bf16_bits_to_f32(synth.w3(shape=(64, 96), seed=8))
    for kw in (dict(), dict(rule=1), dict(elem=1, asymmetric=1, rule=1), dict(scale=4, rule=1)):
        qc = ref.quantize(x, ref.Format(block_rows=32, block_cols=1, **kw))
        qr = ref.quantize(np.ascontiguousarray(x.T), ref.Format(block_rows=1, block_cols=32, **kw))
        assert np.array_equal(qc["dequant"], qr["dequant"].T)
        assert np.array_equal(qc["scales"], qr["scales"].T)


def test_2d_block_scale_is_max_of_row_scales(ref):
    x = synth.bf16_bits_to_f32(synth.w3(shape=(64, 128), seed=9))
    for rule in (0, 1):
        q2 = ref.quantize(x, ref.Format(block_rows=32, block_cols=32, rule=rule))
        q1 = ref.quantize(x, ref.Format(block_rows=1, block_cols=32, rule=rule))
        want = q1["scales"].reshape(2, 32, 4).max(axis=1)
        assert np.array_equal(q2["scales"], want)


def test_hadamard_fused_equals_prerotated(ref):
    x = synth.bf16_bits_to_f32(synth.w4(shape=(32, 256), seed=12))
    for h in (32, 128):
        q = ref.quantize(x, ref.Format(hadamard=h))
        xr = ref.hadamard_rows(x, h)
        q2 = ref.quantize(xr, ref.Format())
        assert np.array_equal(q["codes"], q2["codes"]) and np.array_equal(q["dequant"], q2["dequant"])
        # the rotation is orthonormal and its own inverse: QSNR in both domains agree
        back = ref.hadamard_rows(q["dequant"], h)
        _, d_orig = ref.qsnr(x, back)
        assert abs(d_orig - ref.qsnr_db(q["stats"])) < 1e-3


def test_rotation_helps_laplace_mxfp4(ref):
    """Soft check: a block Hadamard rotation raises MXFP4 QSNR on heavy-tailed
    (Laplace) data ('Bridging the Gap', Sec. 2.1)."""
    x = synth.bf16_bits_to_f32(synth.w4(shape=(256, 1024), seed=13, channels=0))
    base = ref.qsnr_db(ref.quantize(x, ref.Format())["stats"])
    rot = ref.qsnr_db(ref.quantize(x, ref.Format(hadamard=32))["stats"])
    assert rot > base


def test_oas_limits_and_gain(ref):
    x = synth.bf16_bits_to_f32(synth.w4(shape=(128, 512), seed=14))
    ceil = ref.quantize(x, ref.Format(rule=1))
    floor = ref.quantize(x, ref.Format(rule=0))
    t6 = ref.quantize(x, ref.Format(rule=2, oas_tau=6.0))
    t8 = ref.quantize(x, ref.Format(rule=2, oas_tau=nextafter32(8.0, 0)))
    for a, b in ((ceil, t6), (floor, t8)):
        assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    # soft check on outlier-free Laplace data: tolerating overflow beats the
    # conventional rule by about half a dB ('Unveiling', Sec. 4 OAS)
    x = synth.bf16_bits_to_f32(synth.w4(shape=(256, 1024), seed=14, channels=0))
    ceil = ref.quantize(x, ref.Format(rule=1))
    oas = ref.quantize(x, ref.Format(rule=2, oas_tau=7.5))
    assert ref.qsnr_db(oas["stats"]) > ref.qsnr_db(ceil["stats"]) + 0.3
    assert oas["stats"]["flushed"] < ceil["stats"]["flushed"]


def test_mbs_invariants(ref):
    x = synth.bf16_bits_to_f32(synth.w4(shape=(64, 512), seed=15))
    f = ref.Format(macro_cols=128, block_cols=16, rule=1)
    q = ref.quantize(x, f)
    sm = np.array([ref.fp8_scale_value(ref.SC_UE4M3, int(c)) for c in q["macro_scales"].ravel()])
    assert set(np.unique(sm)) <= {1 + k / 8 for k in range(9)}
    # dequant = element * 2^e * s_M exactly
    codes = np.zeros(x.shape, np.int64)
    codes[:, 0::2] = q["codes"] & 0xF
    codes[:, 1::2] = q["codes"] >> 4
    for r in range(0, 64, 7):
        for c in range(0, 512, 5):
            val = Fr(ref.code_value(ref.E2M1, 0, int(codes[r, c])))
            e = int(q["scales"][r, c // 16]) - 127
            s = Fr(ref.fp8_scale_value(ref.SC_UE4M3, int(q["macro_scales"][r, c // 128])))
            assert Fr(float(q["dequant"][r, c])) == val * Fr(2) ** e * s
    # the macro maximum comes back within the element grid's and s_M's rounding
    for r in range(64):
        for m in range(4):
            blk = x[r, m * 128:(m + 1) * 128]
            i = np.argmax(np.abs(blk))
            assert abs(q["dequant"][r, m * 128 + i] - blk[i]) <= abs(blk[i]) * (1 / 16 + 1 / 6)
    # soft check: MBS beats plain 1x16 E8M0 with the same rule
    plain = ref.quantize(x, ref.Format(block_cols=16, rule=1))
    assert ref.qsnr_db(q["stats"]) > ref.qsnr_db(plain["stats"])


def test_e3m0_scale_invariants(ref):
    x = synth.bf16_bits_to_f32(synth.w3(shape=(64, 256), seed=16))
    x[0, :32] = 0
    f = ref.Format(scale=ref.SC_E3M0, rule=1)
    q = ref.quantize(x, f)
    at = Fr(float(np.abs(x).max()))
    eref = int(q["ref_exp"][0])
    assert 6 * Fr(2) ** (eref - 1) < at <= 6 * Fr(2) ** eref
    assert q["scales"][0, 0] == 7 and q["scales"].max() <= 7
    blocks = np.abs(x).reshape(64, 8, 32).max(axis=2)
    for (i, j), c in np.ndenumerate(q["scales"]):
        a = Fr(float(blocks[i, j]))
        if a == 0 or c in (0, 7):
            continue
        assert 6 * Fr(2) ** (eref - int(c) - 1) < a <= 6 * Fr(2) ** (eref - int(c))


def test_asymmetric_int4_invariants(ref):
    x = synth.bf16_bits_to_f32(synth.w3(shape=(32, 256), seed=17)) + np.float32(3e-4)
    f = ref.Format(elem=ref.INT4, asymmetric=1, rule=1)
    q = ref.quantize(x, f)
    blocks = x.reshape(32, 8, 32)
    off = synth.bf16_bits_to_f32(q["offsets"])
    ob = q["offsets"].astype(np.int64)
    neg = (ob & 0x8000) != 0
    up = np.where(neg, ob - 1, ob + 1)               # next bf16 toward +inf
    up = np.where(ob == 0x8000, 0x0001, up)
    nxt = synth.bf16_bits_to_f32(up.astype(np.uint16))
    assert np.all(off <= blocks.min(axis=2))
    assert np.all(nxt > blocks.min(axis=2))          # the largest bf16 <= the block minimum
    X = 2.0 ** (q["scales"].astype(np.float64) - 127)
    err = np.abs(q["dequant"].reshape(32, 8, 32).astype(np.float64) - blocks)
    assert np.all(err <= X[..., None] / 2 + 1e-12)
    R = blocks.max(axis=2) - off
    assert np.all((R <= 15 * X) & (R > 7.5 * X))
    # soft check: asymmetric scaling helps INT4 on shifted data (ARITH report, findings 3)
    sym = ref.quantize(x, ref.Format(elem=ref.INT4, rule=1))
    assert ref.qsnr_db(q["stats"]) > ref.qsnr_db(sym["stats"])


def test_nonfinite_block(ref):
    x = synth.w1(shape=(2, 64))
    x[0, 5] = np.nan
    x[1, 40] = np.inf
    q = ref.quantize(x, ref.Format())
    assert q["scales"][0, 0] == 0xFF and q["scales"][1, 1] == 0xFF
    assert np.all(q["codes"][0, :16] == 0) and np.all(np.isnan(q["dequant"][0, :32]))
    assert np.all(np.isfinite(q["dequant"][0, 32:]))
    y = ref.dequantize(ref.Format(), q, 2, 64)
    assert np.all(np.isnan(y[1, 32:]))


def test_sr_unbiased_on_tensor(ref):
    v = np.float32(0.3)
    x = np.full((256, 256), v, np.float32)
    x[:, ::32] = np.float32(6.0)      # pins every block's scale at 2^0 (FLOOR)
    q = ref.quantize(x, ref.Format(round=ref.SR, seed=synth.SR_SEED))
    d = q["dequant"].astype(np.float64)
    mask = np.ones_like(x, bool)
    mask[:, ::32] = False
    vals = d[mask]
    assert set(np.unique(vals)) == {0.0, 0.5}
    p = 0.3 / 0.5
    n = vals.size
    assert abs(vals.mean() - 0.3) < 4 * 0.5 * math.sqrt(p * (1 - p) / n)
    q2 = ref.quantize(x, ref.Format(round=ref.SR, seed=synth.SR_SEED))
    assert np.array_equal(q["codes"], q2["codes"])
    q3 = ref.quantize(x, ref.Format(round=ref.SR, seed=synth.SR_SEED, rng_offset=1))
    assert not np.array_equal(q["codes"], q3["codes"])


def test_flush_below_smallest_grid_value(ref):
    """Under E8M0 FLOOR every |x| < 2^(e-2) (a quarter of the scale) flushes:
    the 12x range of E2M1 leaves nothing below half its smallest value."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 4.0
    x[0, 1:] = np.linspace(0.01, 0.25, 31, dtype=np.float32)
    q = ref.quantize(x, ref.Format())
    assert int(q["scales"][0, 0]) == 127
    assert np.all(q["dequant"][0, 1:] == 0)
    assert q["stats"]["flushed"] == 31


def test_gemm_oracle_exact_case(ref):
    """All scales 2^0: every product is a multiple of 1/4, so the float64
    product equals an exact integer product / 16."""
    rng = np.random.default_rng(1)
    m, n, k = 24, 40, 96
    qa = rng.integers(0, 16, (m, k))
    qb = rng.integers(0, 16, (n, k))
    va = np.array([ref.code_value(0, 0, int(c)) for c in range(16)])
    A, B = va[qa], va[qb]
    C = ref.gemm_f64(A, B)
    Ci = (np.rint(A * 2).astype(np.int64) @ np.rint(B * 2).astype(np.int64).T)
    assert np.array_equal(C * 4, Ci.astype(np.float64))
    mi = rng.integers(0, m, 50)
    ni = rng.integers(0, n, 50)
    assert np.array_equal(ref.gemm_f64_sampled(A, B, mi, ni), C[mi, ni])


def test_bad_arguments_rejected(ref):
    x = synth.w1(shape=(4, 64))
    for kw in (dict(block_cols=24), dict(elem=9), dict(rule=2, oas_tau=5.0),
               dict(hadamard=24), dict(macro_cols=64), dict(asymmetric=1, scale=1)):
        with pytest.raises(ValueError):
            ref.quantize(x, ref.Format(**kw))


def test_fp8_element_grid_facts(ref):
    """The OCP 8-bit MX element types: E4M3 max 448 = 1.75 * 2^8, smallest
    subnormal 2^-9, 126 positive values; E5M2 max 57344 = 1.75 * 2^15, smallest
    subnormal 2^-16; both saturate (no Inf/NaN is produced) and the FLOOR
    rule uses emax 8 and 15."""
    for elem, top, tiny, emax in ((ref.FP8_E4M3, 448.0, 2.0 ** -9, 8), (ref.FP8_E5M2, 57344.0, 2.0 ** -16, 15)):
        vals = sorted({abs(v) for v in (ref.code_value(elem, 0, c) for c in range(256)) if not math.isnan(v)})
        assert vals[-1] == top and vals[1] == tiny
        assert ref.code_value(elem, 0, ref.round_code(elem, 0, ref.RTNE, 1e30)) == top
        assert ref.code_value(elem, 0, ref.round_code(elem, 0, ref.RTNE, -1e30)) == -top
        assert ref.e8m0_exponent(ref.RULE_FLOOR, 0, elem, 0, 1.0) == -emax
