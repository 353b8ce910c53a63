"""The row and tile quantizers decide E2M1 stochastic rounding from the fp32
bits of v (an element already divided by its block's power-of-two scale)
instead of searching the grid.  Between neighbours lo <= |v| < hi the oracle
goes up iff r16 < f 2^16 with f = (|v| - lo) / (hi - lo).  On the E2M1 grid the
step hi - lo is 2^(E-1) for |v| = 2^E (1 + m 2^-23) in [1, 6) and 0.5 below 1,
so f 2^16 is exact and

  - |v| in [1, 6):    lo = (bits >> 22) - 252, up iff (r16 << 6) < (bits & 0x3fffff)
  - |v| in [0.5, 1):  lo = 1,                  up iff (r16 << 7) < (bits & 0x7fffff)
  - |v| below 0.5:    lo = 0,                  up iff r16 < |v| 2^17 (an exact product)
  - |v| >= 6 and Inf: the largest code; the sign bit goes to bit 3.

(A NaN element is not decided here: a block holding one gets the NaN scale and
zero codes as a whole, in the kernels and in the oracle.)

This test emulates that formula on the host and holds it to the oracle's
ref_round_code on every bf16 magnitude in [0, 8) and on random binary32 values,
each with draws on both sides of its threshold and at the extremes.  Host
only: no GPU."""
import numpy as np

import oracle


def _formula(bits, r16):
    u = bits & 0x7fffffff
    neg = bits >> 31
    if u >= 0x40c00000:
        idx = 7
    elif u >= 0x3f800000:
        idx = ((u >> 22) - 252) + (1 if (r16 << 6) < (u & 0x3fffff) else 0)
    elif u >= 0x3f000000:
        idx = 1 + (1 if (r16 << 7) < (u & 0x7fffff) else 0)
    else:
        m = float(np.uint32(u).view(np.float32))
        idx = 1 if float(r16) < float(np.float32(m) * np.float32(131072.0)) else 0
    return (neg << 3) | idx


def _draws(bits):
    """r16 values around the threshold t = f 2^16 of v, plus the extremes"""
    u = bits & 0x7fffffff
    m = float(np.uint32(u).view(np.float32))
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = {0, 1, 0x7fff, 0xfffe, 0xffff}
    if m < 6.0:
        lo = max(i for i, g in enumerate(grid) if g <= m)
        t = (m - grid[lo]) / (grid[lo + 1] - grid[lo]) * 65536.0
        for d in (-2, -1, 0, 1, 2):
            r = int(np.floor(t)) + d
            if 0 <= r <= 0xffff:
                out.add(r)
    return sorted(out)


def _check(bits_list):
    bad = []
    for bits in bits_list:
        v = float(np.uint32(bits).view(np.float32))
        for r in _draws(bits):
            want = oracle.round_code(oracle.E2M1, 0, oracle.SR, v, r)
            got = _formula(int(bits), r)
            if want != got:
                bad.append((hex(int(bits)), r, want, got))
    assert not bad, bad[:10]


def test_every_bf16_magnitude_below_eight():
    u = np.arange(0, 0x4100, dtype=np.uint32) << 16          # +0 .. 8 in bf16 steps
    _check(list(u) + list(u | 0x80000000))


def test_random_binary32_values():
    rng = np.random.default_rng(21)
    e = rng.integers(100, 130, 4000).astype(np.uint32)        # 2^-27 .. 2^2
    m = rng.integers(0, 1 << 23, 4000).astype(np.uint32)
    s = rng.integers(0, 2, 4000).astype(np.uint32)
    _check(list((s << 31) | (e << 23) | m))


def test_saturation_and_specials():
    specials = [0x40c00000, 0x40bfffff, 0x40e00000, 0x7f800000, 0x00000001, 0x00800000, 0x3effffff,
                0x3f7fffff, 0x3fffffff, 0x407fffff]
    _check(specials + [b | 0x80000000 for b in specials])
