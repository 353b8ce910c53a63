"""Host-side analysis tools for microscaling formats (numpy / scipy, no GPU).

Two data-only tools that sit beside the GPU quantizer:

* ``mse_model`` -- the expected per-element MSE of block quantization of
  i.i.d. N(0, sigma^2) data, split into the three contributions named in
  "Is Finer Better? The Limits of Microscaling Formats in LLMs" (theoretical
  framework): the error of the non-maximum elements, the error of the block
  maximum itself (non-zero once the scale is quantized), and the zero-rounding
  error of blocks whose maximum falls below the smallest scale the format can
  hold, which then round to zero entirely.  ``inversions`` uses it to find the
  block sizes at which halving the block raises the error (the perplexity
  inversion of narrow distributions with UE4M3 scales).

* ``mse_scale_search`` -- the MSE-optimised scales of "Bridging the Gap
  Between Promise and Performance for Microscaling FP4 Quantization" (Sec.
  2.2, MSE-optimised grids): alternate between the group scales (each the
  candidate with the smallest block error) and one global scale (the candidate
  with the smallest tensor error), starting from round-to-nearest scales.

Element grid and rounding follow the library: E2M1 magnitudes {0, .5, 1, 1.5,
2, 3, 4, 6}, round to nearest with ties to the even code, saturation at 6;
UE4M3 scales (bias 7, subnormal step 2^-9, max 448), UE5M3 (bias 15, subnormal
step 2^-17) and E8M0 powers of two.
"""
import math

import numpy as np
from scipy.special import ndtr

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
# rounding boundaries between consecutive grid magnitudes (midpoints); a value
# on a boundary goes to the even code: down at .25, 1.25, 2.5, 5, up at .75,
# 1.75, 3.5
_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_TIE_UP = np.array([False, True, False, True, False, True, False])


def e2m1_round(v):
    """Magnitude-preserving RTNE onto E2M1 with saturation (sign kept)."""
    v = np.asarray(v, np.float64)
    m = np.abs(v)
    idx = np.searchsorted(_MIDS, m, side="left")          # m <= mid -> below
    on = (idx < len(_MIDS)) & (m == _MIDS[np.minimum(idx, len(_MIDS) - 1)])
    idx = np.where(on & _TIE_UP[np.minimum(idx, len(_MIDS) - 1)], idx + 1, idx)
    return np.copysign(E2M1_GRID[idx], v)


def _fp8_round(t, bias, max_value):
    """RNE of positive t onto an unsigned minifloat with 3 mantissa bits."""
    t = np.asarray(t, np.float64)
    out = np.zeros_like(t)
    pos = t > 0
    tp = t[pos]
    e = np.floor(np.log2(tp))
    e = np.maximum(e, 1 - bias)                           # subnormals share the lowest step
    q = np.exp2(e - 3)
    out[pos] = np.minimum(np.round(tp / q) * q, max_value)
    return out


def scale_round(t, scale):
    """Scale value for the ideal scale t = amax / 6 under a scale format."""
    if scale == "ue4m3":
        return _fp8_round(t, 7, 448.0)
    if scale == "ue5m3":
        return _fp8_round(t, 15, 1.75 * 2.0 ** 16)
    raise ValueError(scale)


def _scale_of_amax(a, scale, rule, tensor_scale):
    a = np.asarray(a, np.float64)
    if scale == "e8m0":
        out = np.zeros_like(a)
        pos = a > 0
        if rule == "floor":
            out[pos] = np.exp2(np.floor(np.log2(a[pos])) - 2)
        else:                                             # ceil: smallest 2^e with 6 * 2^e >= a
            out[pos] = np.exp2(np.ceil(np.log2(a[pos] / 6.0)))
        return out
    g = 1.0 if tensor_scale is None else float(tensor_scale)
    return scale_round(a / 6.0 / g, scale) * g


def _normal_moments(l, u, sigma):
    """Partial moments of |X|, X ~ N(0, sigma^2), over [l, u]: the integrals of
    f, x f and x^2 f with f the density of |X|."""
    zl, zu = l / sigma, u / sigma
    pl, pu = np.exp(-0.5 * zl * zl) / math.sqrt(2 * math.pi), np.exp(-0.5 * zu * zu) / math.sqrt(2 * math.pi)
    m0 = 2.0 * (ndtr(zu) - ndtr(zl))
    m1 = 2.0 * sigma * (pl - pu)
    m2 = 2.0 * sigma * sigma * ((ndtr(zu) - ndtr(zl)) - (zu * pu - zl * pl))
    return m0, m1, m2


def _err_below(a, s, sigma):
    """Integral over 0 <= x < a of (x - Q(x))^2 f(x), Q the E2M1 quantizer with
    scale s (elementwise over arrays a, s; s == 0 flushes: Q = 0)."""
    a = np.asarray(a, np.float64)
    s = np.asarray(s, np.float64)
    lo_t = np.concatenate([[0.0], _MIDS])                 # cell k: [lo_t[k], hi_t[k]) * s -> grid[k]
    hi_t = np.concatenate([_MIDS, [np.inf]])
    tot = np.zeros(np.broadcast(a, s).shape)
    flush = s == 0
    for k in range(len(E2M1_GRID)):
        l = np.minimum(lo_t[k] * s, a)
        u = a if np.isinf(hi_t[k]) else np.minimum(hi_t[k] * s, a)
        c = E2M1_GRID[k] * s
        m0, m1, m2 = _normal_moments(l, u, sigma)
        tot += np.where(flush, 0.0, m2 - 2 * c * m1 + c * c * m0)
    m0, m1, m2 = _normal_moments(np.zeros_like(a), a, sigma)
    return np.where(flush, m2, tot)


def mse_model(sigma, block, scale="ue4m3", rule="floor", tensor_scale=None, npts=40000):
    """Expected MSE per element of quantizing N(0, sigma^2) in blocks of
    `block` with E2M1 elements and the given scale format ("e8m0" with the
    "floor" or "ceil" rule, "ue4m3", "ue5m3"; `tensor_scale` multiplies the
    fp8 scales as NVFP4's per-tensor scale does).

    Conditioning on the block maximum A (density b f(a) F(a)^(b-1), f and F of
    |X|), the scale s(A) is fixed; the maximum contributes (A - Q(A))^2 and
    each of the other b - 1 elements, distributed as |X| below A, its expected
    squared error.  Blocks whose scale rounds to zero contribute their whole
    energy.  Returns the total and the three parts, per element."""
    sigma = float(sigma)
    b = int(block)
    # the block maximum lives within a few sigma of sqrt(2 log b) sigma; the
    # grid is dense in the body and in the zero-rounding corner
    hi = sigma * (math.sqrt(2 * math.log(max(b, 2))) + 9.0)
    a = np.unique(np.concatenate([np.linspace(0.0, hi, npts), np.geomspace(sigma * 1e-4, hi, npts)]))
    F = 2.0 * ndtr(a / sigma) - 1.0
    f = 2.0 * np.exp(-0.5 * (a / sigma) ** 2) / (sigma * math.sqrt(2 * math.pi))
    dens = b * f * np.power(np.maximum(F, 0.0), b - 1)
    s = _scale_of_amax(a, scale, rule, tensor_scale)
    flush = s == 0
    qa = np.where(flush, 0.0, s * np.abs(e2m1_round(np.divide(a, s, out=np.zeros_like(a), where=~flush))))
    err_max = (a - qa) ** 2
    inner = np.divide(_err_below(a, s, sigma), F, out=np.zeros_like(a), where=F > 0)
    nonmax = np.where(flush, 0.0, (b - 1) * inner)
    zero = np.where(flush, a * a + (b - 1) * inner, 0.0)
    maxp = np.where(flush, 0.0, err_max)
    integ = lambda y: float(np.trapezoid(y * dens, a)) / b
    parts = {"nonmax": integ(nonmax), "max": integ(maxp), "zero": integ(zero)}
    parts["total"] = parts["nonmax"] + parts["max"] + parts["zero"]
    return parts


def inversions(sigma, blocks=(8, 16, 32, 64, 128, 256), scale="ue4m3", rule="floor", tensor_scale=None):
    """For consecutive block sizes b < b', whether the smaller block has the
    larger modelled MSE (an inversion)."""
    blocks = sorted(blocks)
    mse = {b: mse_model(sigma, b, scale, rule, tensor_scale)["total"] for b in blocks}
    return [{"small": b0, "large": b1, "mse_small": mse[b0], "mse_large": mse[b1], "inverted": mse[b0] > mse[b1]}
            for b0, b1 in zip(blocks, blocks[1:])]


# ---- MSE-optimised scales ------------------------------------------------------

def _e4m3_grid(lo=2.0 ** -9, hi=448.0):
    vals = []
    for e in range(0, 16):
        for m in range(8):
            v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            if lo <= v <= hi:
                vals.append(v)
    return np.array(sorted(set(vals)))


def _block_sse(x, s, chunk=16384):
    """Sum of squared errors of blocks x (nblk, b) under scales s (nblk, ncand)."""
    out = np.empty(s.shape)
    for i in range(0, x.shape[0], chunk):
        xc, sc = x[i:i + chunk, None, :], s[i:i + chunk, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.nan_to_num(xc / sc)
        q = np.where(sc > 0, e2m1_round(v) * sc, 0.0)
        out[i:i + chunk] = ((xc - q) ** 2).sum(axis=2)
    return out


def mse_scale_search(w, fmt="mxfp4", iters=4, ncand=5, nglobal=33):
    """MSE-optimised scales for a weight matrix w (rows x cols, cols a multiple
    of the block: 32 for "mxfp4" with E8M0 group scales, 16 for "nvfp4" with
    UE4M3 group scales).  Alternates between (1) every group scale: the best
    of `ncand` candidates around the current one (E8M0: neighbouring powers of
    two; UE4M3: neighbouring codes), and (2) the global fp32 scale: the best of
    `nglobal` candidates spaced geometrically over one octave around the
    current one (0: the global scale stays).  Starts from round-to-nearest scales (FLOOR rule for E8M0,
    RNE(amax / 6 / g) with g = amax_t / 2688 for NVFP4, the smallest non-zero
    code where that rounds to zero), and no step raises the error.

    Returns dict(global_scale, group_scales (rows, cols / block), dequant,
    mse_history): dequant = global * group * E2M1(w / (global * group))."""
    w = np.asarray(w, np.float64)
    rows, cols = w.shape
    bsz = 32 if fmt == "mxfp4" else 16
    x = w.reshape(-1, bsz)
    amax = np.abs(x).max(axis=1)
    if fmt == "mxfp4":
        g = 1.0
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0.0)
        grid = None
    else:
        at = float(np.abs(w).max())
        g = at / 2688.0 if at > 0 else 1.0
        grid = _e4m3_grid()
        idx = np.searchsorted(grid, scale_round(amax / 6.0 / g, "ue4m3"))
        idx = np.clip(idx, 0, len(grid) - 1)

    def group_values():
        return np.exp2(e) if fmt == "mxfp4" else grid[idx]

    def total_sse(gv):
        return float(_block_sse(x, (gv * g)[:, None])[:, 0].sum())

    hist = [total_sse(group_values()) / w.size]
    half = ncand // 2
    for _ in range(iters):
        # (1) group scales, global fixed
        offs = np.arange(-half, half + 1)
        if fmt == "mxfp4":
            cand_e = e[:, None] + offs[None, :]
            cand = np.exp2(cand_e) * g
        else:
            cand_i = np.clip(idx[:, None] + offs[None, :], 0, len(grid) - 1)
            cand = grid[cand_i] * g
        best = np.argmin(_block_sse(x, cand), axis=1)
        if fmt == "mxfp4":
            e = cand_e[np.arange(len(best)), best]
        else:
            idx = cand_i[np.arange(len(best)), best]
        # (2) global scale, group scales fixed; kept unless a candidate is better
        if nglobal > 0:
            gv = group_values()
            gs = g * np.exp2(np.linspace(-0.5, 0.5, nglobal))
            sse = [float(_block_sse(x, (gv * gg)[:, None])[:, 0].sum()) for gg in gs]
            k = int(np.argmin(sse))
            if sse[k] < total_sse(gv):
                g = float(gs[k])
        hist.append(total_sse(group_values()) / w.size)
    gv = group_values()
    s = (gv * g)[:, None]
    deq = (e2m1_round(x / s) * s).reshape(rows, cols)
    return {"global_scale": g, "group_scales": gv.reshape(rows, cols // bsz), "dequant": deq, "mse_history": hist}
