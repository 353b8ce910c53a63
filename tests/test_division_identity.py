"""The row quantizer divides each element by its block's fp8 scale, or by its
macro block's UE4M3 scale, through one correctly rounded reciprocal r = RN(1/b)
and Markstein's correction step per element:

    q = RN(a r);  e = RN(a - q b)  (exact: one FMA);  q' = RN(q + e r),  sign of a

This test emulates that sequence exactly in binary32 (numpy float32 products,
float64 for the exact intermediate sums, fractions wherever a float64 value
lands on a binary32 tie) and holds it to the correctly rounded quotient
RN(a / b), which is what the oracle's divide gives:

  - every finite bf16 input a with |a| >= 2^-96 against every finite UE4M3 and
    UE5M3 block-scale value: equal bit for bit wherever 2^-96 <= |a / b| <=
    2^120 (a block's quotients never exceed max(8, amax / 448)), and below
    2^-96 of a's sign and under 2^-80 (far under every E2M1 rounding point,
    so the code is the same);
  - every such input against every macro scale 1, 1.125, ..., 2, over the
    whole range;
  - random NVFP4-like divisors (a UE4M3 value times an fp32 tensor scale).

Inputs below 2^-96 (or non-finite) send the kernel's wave to the exact divide,
so they are outside this identity.  Host-only arithmetic: no GPU, no oracle."""
from fractions import Fraction

import numpy as np

LOW = 2.0 ** -96


def _rn32(fr):
    """binary32 nearest-even of a Fraction in the normal range"""
    if fr == 0:
        return np.float32(0)
    s = -1 if fr < 0 else 1
    fr = abs(fr)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    q = fr / Fraction(2) ** (e - 23)
    n, rem = divmod(q.numerator, q.denominator)
    rem = Fraction(rem, q.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2):
        n += 1
    return np.float32(s * float(Fraction(n) * Fraction(2) ** (e - 23)))


def _to32(x64, exact):
    """binary32 rounding of float64 values; where a value sits exactly on a
    binary32 midpoint (a double-rounding hazard) the exact value decides"""
    f = x64.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    f64 = f.astype(np.float64)
    tie = (x64 == (f64 + up) / 2) | (x64 == (f64 + dn) / 2)
    for i in np.nonzero(tie & np.isfinite(x64))[0]:
        f[i] = exact(i)
    return f


def _check(a, b, hi=2.0 ** 120):
    a = a.astype(np.float32)
    b = np.float32(b)
    r = np.float32(1) / b
    q = (a * r).astype(np.float32)
    e = (a.astype(np.float64) - q.astype(np.float64) * np.float64(b)).astype(np.float32)
    q2 = _to32(q.astype(np.float64) + e.astype(np.float64) * np.float64(r),
               lambda i: _rn32(Fraction(float(q[i])) + Fraction(float(e[i])) * Fraction(float(r))))
    q2 = np.copysign(q2, a)
    want = _to32(a.astype(np.float64) / np.float64(b), lambda i: _rn32(Fraction(float(a[i])) / Fraction(float(b))))
    ex = np.abs(a.astype(np.float64) / np.float64(b))
    big = (ex >= LOW) & (ex <= hi)
    assert np.array_equal(q2[big].view(np.uint32), want[big].view(np.uint32)), f"b = {b}"
    small = ex < LOW
    assert np.all(np.signbit(q2[small]) == np.signbit(a[small])) and np.all(np.abs(q2[small]) < 2.0 ** -80)


def _bf16_inputs():
    a = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    a = a[np.isfinite(a)]
    return a[np.abs(a) >= LOW]


def _fp8_values(bias, nan_codes):
    vals = []
    for c in range(128):
        if c in nan_codes:
            continue
        e, m = c >> 3, c & 7
        v = (m / 8) * 2.0 ** (1 - bias) if e == 0 else (1 + m / 8) * 2.0 ** (e - bias)
        if v > 0:
            vals.append(np.float32(v))
    return vals


def test_every_bf16_input_against_every_ue4m3_scale():
    a = _bf16_inputs()
    with np.errstate(over="ignore", invalid="ignore"):
        for b in _fp8_values(7, {0x7f}):
            _check(a, b)


def test_every_bf16_input_against_every_ue5m3_scale():
    a = _bf16_inputs()
    with np.errstate(over="ignore", invalid="ignore"):
        for b in _fp8_values(15, {0x7f}):
            _check(a, b)


def test_every_bf16_input_against_every_macro_scale():
    a = _bf16_inputs()
    for m in range(9):
        _check(a, np.float32(1 + m / 8), hi=np.inf)


def test_random_nvfp4_divisors():
    rng = np.random.default_rng(5)
    a_all = _bf16_inputs()
    ue4m3 = _fp8_values(7, {0x7f})
    with np.errstate(over="ignore", invalid="ignore"):
        for _ in range(40):
            g = np.float32(np.exp2(rng.uniform(-100, 60)))
            b = np.float32(ue4m3[rng.integers(0, len(ue4m3))] * g)
            _check(a_all[rng.integers(0, len(a_all), 50000)], b)


def _fp32_sample(rng, n, lo_exp, hi_exp):
    """random binary32 values with exponents uniform in [lo_exp, hi_exp) and random significands and signs"""
    e = rng.integers(lo_exp + 127, hi_exp + 127, n).astype(np.uint32)
    m = rng.integers(0, 1 << 23, n).astype(np.uint32)
    s = rng.integers(0, 2, n).astype(np.uint32)
    return ((s << 31) | (e << 23) | m).view(np.float32)


def test_block_maxima_over_six():
    """The NVFP4 / UE4M3 / UE5M3 block scale starts from amax / 6: the kernel
    takes the same correction step with r = RN(1/6) for maxima in [2^-90,
    2^120] (quotients in [2^-93, 2^118]); others divide exactly."""
    rng = np.random.default_rng(11)
    a = _bf16_inputs()
    a = a[(np.abs(a) >= 2.0 ** -90) & (np.abs(a) <= 2.0 ** 120)]
    _check(a, np.float32(6))
    _check(np.abs(_fp32_sample(rng, 400000, -90, 120)), np.float32(6))


def test_block_maxima_over_tensor_scales():
    """NVFP4's amax / 6 is divided by the fp32 tensor scale g through r =
    RN(1/g): the kernel takes that path when the dividend lies in [2^-90,
    2^119] and RN(a r) in [2^-94, 2^118], which keeps the exact quotient
    inside [2^-96, 2^120]; random g over 2^-126 .. 2^100."""
    rng = np.random.default_rng(12)
    for _ in range(60):
        g = np.float32(np.exp2(rng.uniform(-126, 100)))
        a = np.abs(_fp32_sample(rng, 20000, -90, 119))
        with np.errstate(over="ignore", under="ignore"):
            q0 = (a * (np.float32(1) / g)).astype(np.float32)
        a = a[(q0 >= 2.0 ** -94) & (q0 <= 2.0 ** 118)]
        if len(a):
            _check(a, g)
