"""GPU parity of the block-scaled GEMM (MXFP4, MXFP6 and mixed operands) and of
the QSNR reduction.

The oracle is the plain definition: the dequantized operands (exact in fp32)
multiplied with float64 accumulation.  When every scale is 2^0 each product is
a multiple of 1/4 and every partial sum is exact in fp32, so the fp32 output
must match bit for bit and the bf16 output must be the nearest-even rounding
of the exact value.  Otherwise the relative Frobenius error of the bf16 output
against the bf16-rounded oracle must stay within 1e-3 (fp32 output: 1e-5).
"""
import math

import numpy as np
import pytest
import torch

import microscaling_block_quantization_amd as mx
import oracle
import synth
from parity import to_dev

pytestmark = pytest.mark.gpu


def make_q(codes, scales, rows, cols):
    return mx.QTensor(rows, cols, torch.from_numpy(codes.reshape(-1).copy()).cuda(),
                      torch.from_numpy(scales.reshape(-1).copy()).cuda())


def ref_deq(codes, scales, rows, cols):
    return oracle.dequantize(oracle.Format(), {"codes": codes, "scales": scales}, rows, cols)


def rel_frob(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def bf16_of(x64):
    return oracle.f32_to_bf16_bits(np.asarray(x64, np.float32))


@pytest.mark.parametrize("M,N,K", [(200, 136, 512), (128, 128, 128), (1, 1, 256), (257, 300, 384),
                                   (70, 90, 32), (130, 40, 96), (33, 300, 160), (256, 256, 224),
                                   (257, 300, 1024), (200, 520, 2048), (300, 257, 3072), (512, 256, 1024),
                                   (2304, 8200, 1024), (2304, 8204, 1024)])
def test_exact_case_bit_exact(M, N, K):
    rng = np.random.default_rng(M * 7 + N)
    ca = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    cb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    exact = oracle.gemm_f64(ref_deq(ca, sa, M, K), ref_deq(cb, sb, N, K))
    qa, qb = make_q(ca, sa, M, K), make_q(cb, sb, N, K)
    c32 = mx.mx_gemm(mx.MXFP4, qa, mx.MXFP4, qb, out_dtype=torch.float32)
    c16 = mx.mx_gemm(mx.MXFP4, qa, mx.MXFP4, qb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(c32.cpu().numpy(), exact.astype(np.float32))
    got16 = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, bf16_of(exact))


@pytest.mark.parametrize("M,N,K", [(320, 192, 1024), (96, 520, 256), (200, 136, 96), (64, 64, 352),
                                   (130, 700, 3072), (513, 260, 2048)])
def test_random_scales(M, N, K):
    rng = np.random.default_rng(K)
    ca = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    cb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = rng.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(118, 137, (N, K // 32), dtype=np.uint8)
    ref = oracle.gemm_f64(ref_deq(ca, sa, M, K), ref_deq(cb, sb, N, K))
    qa, qb = make_q(ca, sa, M, K), make_q(cb, sb, N, K)
    c32 = mx.mx_gemm(mx.MXFP4, qa, mx.MXFP4, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(mx.MXFP4, qa, mx.MXFP4, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    assert rel_frob(c32, ref) <= 1e-5
    assert rel_frob(oracle.bf16_bits_to_f32(c16), oracle.bf16_bits_to_f32(bf16_of(ref))) <= 1e-3


# ---- MXFP6 and mixed 4-/6-bit operands -----------------------------------------
# (element, largest magnitude, smallest non-zero magnitude): E2M1 6 and 1/2;
# FP6 E2M3 7.5 and 1/8; FP6 E3M2 28 and 1/16
ELEMS = {"e2m1": (oracle.E2M1, 6.0, 0.5), "e2m3": (oracle.FP6_E2M3, 7.5, 0.125),
         "e3m2": (oracle.FP6_E3M2, 28.0, 0.0625)}
PAIRS = [(a, b) for a in ELEMS for b in ELEMS]


def fmt_pair(ea, eb):
    return (mx.Format(elem=ELEMS[ea][0]), mx.Format(elem=ELEMS[eb][0]),
            oracle.Format(elem=ELEMS[ea][0]), oracle.Format(elem=ELEMS[eb][0]))


def rand_codes(rng, elem, rows, cols):
    return rng.integers(0, 256, (rows, oracle.code_row_bytes(elem, cols)), dtype=np.uint8)


def exact_k(ea, eb, cap):
    """Largest K (multiple of 32, at most cap) for which, with unit scales,
    every partial sum of every output is an integer multiple of the product of
    the two smallest magnitudes below 2^24 of them: then fp32 accumulation in
    any order is exact."""
    _, ma, qa = ELEMS[ea]
    _, mb, qb = ELEMS[eb]
    per = ma * mb / (qa * qb)
    return min(cap, int((2 ** 24 - 1) // per) // 32 * 32)


# Precision of the block-scaled matrix instruction, measured on gfx950
# (test_fp6_instruction_window_measured below): the products of each 32-wide
# scale block are added in fixed point, keeping 14 bits below the leading bit
# of the block's largest product (bits below are dropped toward zero); the two
# block sums and the instruction results accumulate in fp32.  E2M1, E2M3 and
# every pair other than E3M2 x E3M2 have no product bits that far down (their
# smallest product step is at least 2^-14 of their largest product), so those
# are exact.  E3M2 x E3M2 products span 2^-8 .. 784 (18 binades) and lose the
# low bits of small products summed with large ones: each of an instruction's
# 64 products, and each of its partial sums, loses less than one unit of
# 2^(E - 14), E = floor(log2) of the instruction's largest product magnitude
# (a bound that also covers the per-block window).
MFMA_WINDOW = 14
TRUNCATING = {("e3m2", "e3m2")}


def window_bound(deq_a, deq_b):
    """Per output element: the sum over 64-wide K steps (one instruction each)
    of (64 + 8) units of 2^(E - 14), a bound on what the fixed-point window
    can drop."""
    A = np.asarray(deq_a, np.float64)
    B = np.asarray(deq_b, np.float64)
    M, K = A.shape
    N = B.shape[0]
    out = np.zeros((M, N))
    for m0 in range(0, M, 16):
        P = np.abs(A[m0:m0 + 16, None, :] * B[None, :, :])
        P = np.pad(P, ((0, 0), (0, 0), (0, -K % 64))).reshape(P.shape[0], N, -1, 64)
        top = P.max(axis=3)
        unit = np.where(top > 0, np.exp2(np.floor(np.log2(np.where(top > 0, top, 1.0))) - MFMA_WINDOW), 0.0)
        out[m0:m0 + 16] = 72.0 * unit.sum(axis=2)
    return out


def test_fp6_instruction_window_measured():
    """The fixed-point window behind MFMA_WINDOW, measured through mx_gemm with
    one 64-wide K step (one matrix instruction per output), FP6 E3M2 operands
    under unit scales (the oracle's quantization of the values below, exact):
    every output is 28 x 28 = 784 (leading bit 2^9) plus one product p of the
    same 32-wide block, p = +-2^e x (1 or 2^-4), so |p| runs from 2^-8 to 2^3.
    A product of at least 2^(9 - 14) is kept exactly.  A positive smaller one
    is dropped (the sum stays 784); a negative one changes the sum by at most
    one unit of 2^(9 - 14).  (A small product in another block of the same
    instruction is kept: each block's products are summed on their own and
    the block sums are added in fp32.)"""
    M, N, K = 16, 8, 64
    es = np.arange(-4, 4)
    a = np.zeros((M, K), np.float32)
    b = np.zeros((N, K), np.float32)
    a[:, 0] = 28.0
    b[:, 0] = 28.0
    a[:8, 1] = np.exp2(es)
    a[8:, 1] = -np.exp2(es)
    b[:4, 1] = 1.0
    b[4:, 1] = 0.0625
    a[:, 33] = 2.0 ** -4            # the same small product in the second block: always kept
    b[:, 33] = 2.0 ** -4
    fo = oracle.Format(elem=oracle.FP6_E3M2)
    ra, rb = oracle.quantize(a, fo), oracle.quantize(b, fo)
    assert np.array_equal(ra["dequant"], a) and np.array_equal(rb["dequant"], b)
    fm = mx.Format(elem=oracle.FP6_E3M2)
    qa = make_q(ra["codes"], ra["scales"], M, K)
    qb = make_q(rb["codes"], rb["scales"], N, K)
    c = mx.mx_gemm(fm, qa, fm, qb, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    other = 2.0 ** -8                 # the second block's product
    low = 9 - MFMA_WINDOW
    unit = 2.0 ** low
    for i in range(M):
        for j in range(N):
            p = float(a[i, 1]) * float(b[j, 1])
            got = c[i, j] - 784.0 - other
            if abs(p) >= unit:
                assert got == p, (i, j, p, got)
            elif p > 0:
                assert got == 0.0, (i, j, p, got)
            else:
                assert -unit <= got <= 0.0, (i, j, p, got)
    print("kept from 2^%d on; e.g. p = 2^-6 ->" % low, c[0, 4] - 784.0 - other)


@pytest.mark.parametrize("ea,eb", PAIRS)
@pytest.mark.parametrize("M,N,cap", [(130, 200, 1024), (33, 65, 96)])
def test_fp6_mixed_exact_case(ea, eb, M, N, cap):
    K = exact_k(ea, eb, cap)
    fa, fb, ra, rb = fmt_pair(ea, eb)
    rng = np.random.default_rng(M + N + K)
    ca, cb = rand_codes(rng, ra.elem, M, K), rand_codes(rng, rb.elem, N, K)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    da = oracle.dequantize(ra, {"codes": ca, "scales": sa}, M, K)
    db = oracle.dequantize(rb, {"codes": cb, "scales": sb}, N, K)
    exact = oracle.gemm_f64(da, db)
    qa, qb = make_q(ca, sa, M, K), make_q(cb, sb, N, K)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got16 = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    if (ea, eb) in TRUNCATING:
        assert np.all(np.abs(c32.astype(np.float64) - exact) <= window_bound(da, db))
        # the bf16 output is the nearest-even rounding of the same fp32 sums
        assert np.array_equal(got16, bf16_of(c32))
    else:
        assert np.array_equal(c32, exact.astype(np.float32))
        assert np.array_equal(got16, bf16_of(exact))


@pytest.mark.parametrize("ea,eb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(257, 130, 1024), (64, 96, 352)])
def test_fp6_mixed_random_scales(ea, eb, M, N, K):
    fa, fb, ra, rb = fmt_pair(ea, eb)
    rng = np.random.default_rng(K + 3)
    ca, cb = rand_codes(rng, ra.elem, M, K), rand_codes(rng, rb.elem, N, K)
    sa = rng.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(118, 137, (N, K // 32), dtype=np.uint8)
    da = oracle.dequantize(ra, {"codes": ca, "scales": sa}, M, K)
    db = oracle.dequantize(rb, {"codes": cb, "scales": sb}, N, K)
    ref = oracle.gemm_f64(da, db)
    qa, qb = make_q(ca, sa, M, K), make_q(cb, sb, N, K)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    # fp32 accumulation bound, widened by what the window may drop
    slack = np.linalg.norm(window_bound(da, db)) if (ea, eb) in TRUNCATING else 0.0
    assert np.linalg.norm(c32 - ref) <= 1e-5 * np.linalg.norm(ref) + slack
    assert rel_frob(oracle.bf16_bits_to_f32(c16), oracle.bf16_bits_to_f32(bf16_of(ref))) <= 1e-3


@pytest.mark.parametrize("ea,eb", [("e2m3", "e2m3"), ("e2m3", "e2m1"), ("e3m2", "e2m1"), ("e3m2", "e3m2")])
def test_fp6_quantized_operands(ea, eb):
    """MX6 weights and activations, and 6-bit x 4-bit products ('MX6 W-A, MX4 G'
    of the ARITH 2025 MX-training report, main results): operands quantized on
    the GPU, product against the oracle's dequantized product."""
    a, b = synth.w5(m=192, n=320, k=1024)
    fa, fb, ra, rb = fmt_pair(ea, eb)
    qa, _, _ = mx.mx_quantize(fa, to_dev(a))
    qb, _, _ = mx.mx_quantize(fb, to_dev(b))
    da, db = oracle.quantize(a, ra)["dequant"], oracle.quantize(b, rb)["dequant"]
    ref = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    slack = np.linalg.norm(window_bound(da, db)) if (ea, eb) in TRUNCATING else 0.0
    assert np.linalg.norm(c32 - ref) <= 1e-5 * np.linalg.norm(ref) + slack


# ---- MXFP8 operands and 8-bit x 6-/4-bit pairs -------------------------------
# The MX family's 8-bit elements ("Unveiling ... MXFP4", current state: MX
# formats of 8, 6 and 4 bits; the proposed methods also apply to MXFP8) on the
# same scaled matrix instruction, type fields 0 (E4M3) and 1 (E5M2).
FP8 = {"e4m3": oracle.FP8_E4M3, "e5m2": oracle.FP8_E5M2}
ALL8 = {**{k: v[0] for k, v in ELEMS.items()}, **FP8}
FP8_PAIRS = [(a, b) for a in ALL8 for b in ALL8 if a in FP8 or b in FP8]


def fp8_codes(rng, elem, rows, cols, lo_exp=None):
    """random FP8 codes without the Inf / NaN encodings; with lo_exp, only
    magnitudes in [1, 4) (exponent fields lo_exp and lo_exp + 1)"""
    mb = 3 if elem == oracle.FP8_E4M3 else 2
    if lo_exp is None:
        top = 0x7F if elem == oracle.FP8_E4M3 else 0x7C
        mag = rng.integers(0, top, (rows, cols))
    else:
        mag = rng.integers(lo_exp << mb, (lo_exp + 2) << mb, (rows, cols))
    return (mag | (rng.integers(0, 2, (rows, cols)) << 7)).astype(np.uint8)


def codes8(rng, name, rows, cols, narrow):
    e = ALL8[name]
    if name in FP8:
        return fp8_codes(rng, e, rows, cols, (7 if name == "e4m3" else 15) if narrow else None)
    return rand_codes(rng, e, rows, cols)


def fmt8(name):
    return mx.Format(elem=ALL8[name]), oracle.Format(elem=ALL8[name])


@pytest.mark.parametrize("ea,eb", FP8_PAIRS)
@pytest.mark.parametrize("M,N,K", [(130, 260, 1024), (33, 65, 96)])
def test_fp8_exact_case(ea, eb, M, N, K):
    """Unit scales and FP8 magnitudes in [1, 4): every product lies within the
    instruction's 14-bit summation window of the largest (at most 28 * 4 =
    112 against a smallest step of 2^-7) and every partial sum is an exact
    fp32 value (below 2^24 of the smallest step), so fp32 output is bit-exact
    and bf16 output is the nearest-even rounding of the exact sum.  K = 1024
    takes the LDS-staged kernel, K = 96 the register-only one."""
    fa, ra = fmt8(ea)
    fb, rb = fmt8(eb)
    rng = np.random.default_rng(M * 3 + N + K)
    ca, cb = codes8(rng, ea, M, K, True), codes8(rng, eb, N, K, True)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    da = oracle.dequantize(ra, {"codes": ca, "scales": sa}, M, K)
    db = oracle.dequantize(rb, {"codes": cb, "scales": sb}, N, K)
    exact = oracle.gemm_f64(da, db)
    qa, qb = make_q(ca, sa, M, K), make_q(cb, sb, N, K)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(c32, exact.astype(np.float32))
    assert np.array_equal(c16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_of(exact))


@pytest.mark.parametrize("ea,eb", FP8_PAIRS)
@pytest.mark.parametrize("M,N,K", [(257, 130, 1024), (64, 96, 352)])
def test_fp8_random_scales(ea, eb, M, N, K):
    """Every finite code and random scales: fp32 output within the fp32
    accumulation bound widened by what the 14-bit summation window may drop
    (FP8 products span up to 36 binades), bf16 output within 1e-3."""
    fa, ra = fmt8(ea)
    fb, rb = fmt8(eb)
    rng = np.random.default_rng(K + 5)
    ca, cb = codes8(rng, ea, M, K, False), codes8(rng, eb, N, K, False)
    sa = rng.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(118, 137, (N, K // 32), dtype=np.uint8)
    da = oracle.dequantize(ra, {"codes": ca, "scales": sa}, M, K)
    db = oracle.dequantize(rb, {"codes": cb, "scales": sb}, N, K)
    ref = oracle.gemm_f64(da, db)
    qa, qb = make_q(ca, sa, M, K), make_q(cb, sb, N, K)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    slack = np.linalg.norm(window_bound(da, db))
    assert np.linalg.norm(c32 - ref) <= 1e-5 * np.linalg.norm(ref) + slack
    assert rel_frob(oracle.bf16_bits_to_f32(c16), oracle.bf16_bits_to_f32(bf16_of(ref))) <= 1e-3


@pytest.mark.parametrize("ea,eb", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e2m1"), ("e2m1", "e4m3"),
                                   ("e4m3", "e2m3"), ("e2m3", "e5m2")])
def test_fp8_quantized_operands(ea, eb):
    """MXFP8 operands quantized on the GPU, alone and against 6- and 4-bit
    ones; the product against the oracle's dequantized product, and (soft
    check) an error against the exact bf16 product well below MXFP4's."""
    a, b = synth.w5(m=192, n=320, k=1024)
    fa, ra = fmt8(ea)
    fb, rb = fmt8(eb)
    qa, _, _ = mx.mx_quantize(fa, to_dev(a))
    qb, _, _ = mx.mx_quantize(fb, to_dev(b))
    da, db = oracle.quantize(a, ra)["dequant"], oracle.quantize(b, rb)["dequant"]
    ref = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    slack = np.linalg.norm(window_bound(da, db))
    assert np.linalg.norm(c32 - ref) <= 1e-5 * np.linalg.norm(ref) + slack
    if ea in FP8 and eb in FP8:
        exact = synth.bf16_bits_to_f32(a).astype(np.float64) @ synth.bf16_bits_to_f32(b).astype(np.float64).T
        q4 = oracle.gemm_f64(oracle.quantize(a, oracle.Format())["dequant"], oracle.quantize(b, oracle.Format())["dequant"])
        err8, err4 = np.linalg.norm(c32 - exact), np.linalg.norm(q4 - exact)
        assert err8 < err4 / 1.5         # E4M3 about 3.9x lower, E5M2 about 2x


# ---- macro-block scaled MXFP4 ("Unveiling ... MXFP4", Sec. 4, MBS, Fig. 5) -----
MBS_ORACLE = oracle.Format(macro_cols=128)
MBS_DEV = mx.Format(macro_cols=128)


def mbs_case(rng, rows, K, macro_codes):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(118, 137, (rows, K // 32), dtype=np.uint8)
    mac = rng.choice(np.asarray(macro_codes, np.uint8), (rows, K // 128))
    deq = oracle.dequantize(MBS_ORACLE, {"codes": codes, "scales": scales, "macro_scales": mac}, rows, K)
    q = make_q(codes, scales, rows, K)
    q.macro_scales = torch.from_numpy(mac.reshape(-1).copy()).cuda()
    return q, deq


@pytest.mark.parametrize("side", ["both", "a", "b"])
@pytest.mark.parametrize("M,N,K", [(130, 200, 1024), (64, 97, 384), (257, 33, 128)])
def test_mbs_random(side, M, N, K):
    rng = np.random.default_rng(M * 3 + K)
    # UE4M3 codes of the macro scales the quantizer writes: 1, 1.125, ..., 2
    macro = list(range(0x38, 0x41))
    if side in ("both", "a"):
        qa, da = mbs_case(rng, M, K, macro)
        fa = MBS_DEV
    else:
        ca, sa = rng.integers(0, 256, (M, K // 2), dtype=np.uint8), rng.integers(118, 137, (M, K // 32), dtype=np.uint8)
        qa, da, fa = make_q(ca, sa, M, K), ref_deq(ca, sa, M, K), mx.MXFP4
    if side in ("both", "b"):
        qb, db = mbs_case(rng, N, K, macro)
        fb = MBS_DEV
    else:
        cb, sb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8), rng.integers(118, 137, (N, K // 32), dtype=np.uint8)
        qb, db, fb = make_q(cb, sb, N, K), ref_deq(cb, sb, N, K), mx.MXFP4
    ref = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    assert rel_frob(c32, ref) <= 1e-5
    assert rel_frob(oracle.bf16_bits_to_f32(c16), oracle.bf16_bits_to_f32(bf16_of(ref))) <= 1e-3


@pytest.mark.parametrize("M,N,K", [(130, 200, 1024), (33, 65, 256)])
def test_mbs_exact_case(M, N, K):
    """Unit E8M0 scales and macro scales of 1 and 2: every partial sum is a
    multiple of 1/4 below 2^24 in magnitude, so the fp32 result is exact."""
    rng = np.random.default_rng(K + 11)
    qa, da = mbs_case(rng, M, K, [0x38, 0x40])
    qb, db = mbs_case(rng, N, K, [0x38, 0x40])
    for q, rows in ((qa, M), (qb, N)):
        q.scales.fill_(127)
    da = oracle.dequantize(MBS_ORACLE, {"codes": qa.codes.cpu().numpy().reshape(M, K // 2),
                                        "scales": qa.scales.cpu().numpy().reshape(M, K // 32),
                                        "macro_scales": qa.macro_scales.cpu().numpy().reshape(M, K // 128)}, M, K)
    db = oracle.dequantize(MBS_ORACLE, {"codes": qb.codes.cpu().numpy().reshape(N, K // 2),
                                        "scales": qb.scales.cpu().numpy().reshape(N, K // 32),
                                        "macro_scales": qb.macro_scales.cpu().numpy().reshape(N, K // 128)}, N, K)
    exact = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(MBS_DEV, qa, MBS_DEV, qb, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(c32, exact.astype(np.float32))


def test_mbs_quantized_operands():
    """Operands quantized on the GPU with 1 x 128 macro scales over 1 x 32 E8M0
    sub-blocks; the product against the oracle's dequantized product, and the
    product's fidelity (eq. (2)) not below plain MXFP4's."""
    a, b = synth.w5(m=256, n=384, k=1024)
    qa, _, _ = mx.mx_quantize(MBS_DEV, to_dev(a))
    qb, _, _ = mx.mx_quantize(MBS_DEV, to_dev(b))
    ra, rb = oracle.quantize(a, MBS_ORACLE), oracle.quantize(b, MBS_ORACLE)
    ref = oracle.gemm_f64(ra["dequant"], rb["dequant"])
    c32 = mx.mx_gemm(MBS_DEV, qa, MBS_DEV, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(c32.cpu().numpy(), ref) <= 1e-5
    R = oracle.gemm_f64(synth.bf16_bits_to_f32(a), synth.bf16_bits_to_f32(b)).astype(np.float32)
    _, db_mbs = oracle.qsnr(R, c32.cpu().numpy())
    q4a, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(a))
    q4b, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(b))
    _, db_4 = oracle.qsnr(R, mx.mx_gemm(mx.MXFP4, q4a, mx.MXFP4, q4b, out_dtype=torch.float32).cpu().numpy())
    assert db_mbs > db_4


# ---- MBS over E8M0 sub-blocks of other widths (c4's 1 x 128 macro over 1 x 16) ----
# The scaled instruction takes one power-of-two scale per 32 K-values, so these
# products go through the decode kernels: each block's scale is 2^e times its
# macro block's UE4M3 scale, exact in fp32, and the decode applies it.
def mbs_operand(rng, rows, K, bc, macro_codes):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(118, 137, (rows, K // bc), dtype=np.uint8)
    mac = rng.choice(np.asarray(macro_codes, np.uint8), (rows, K // 128))
    fo = oracle.Format(block_cols=bc, macro_cols=128)
    deq = oracle.dequantize(fo, {"codes": codes, "scales": scales, "macro_scales": mac}, rows, K)
    q = make_q(codes, scales, rows, K)
    q.macro_scales = torch.from_numpy(mac.reshape(-1).copy()).cuda()
    return q, deq, mx.Format(block_cols=bc, macro_cols=128)


@pytest.mark.parametrize("sides", ["both", "a", "b"])
@pytest.mark.parametrize("bc,M,N,K", [(16, 130, 200, 1024), (16, 257, 33, 128), (16, 64, 300, 384),
                                      (32, 200, 70, 256), (64, 96, 130, 512), (8, 40, 50, 256)])
def test_mbs_sub_blocks_random(sides, bc, M, N, K):
    """Random codes, E8M0 block scales over 1 x bc sub-blocks and UE4M3 macro
    scales of 1 .. 2 (the quantizer's range) on one or both operands; the other
    operand plain E8M0 1 x bc (LDS-staged decode kernel for bc 16 and 32 when
    the plain side is 1 x 16 / 1 x 32, register-only otherwise).  fp32 output
    within 1e-5 relative Frobenius of the fp64 oracle product, bf16 output
    within 1e-3."""
    rng = np.random.default_rng(bc * 1000 + M + K)
    macro = list(range(0x38, 0x41))
    if sides in ("both", "a"):
        qa, da, fa = mbs_operand(rng, M, K, bc, macro)
    else:
        ca, sa = rng.integers(0, 256, (M, K // 2), dtype=np.uint8), rng.integers(118, 137, (M, K // bc), dtype=np.uint8)
        qa, fa = make_q(ca, sa, M, K), mx.Format(block_cols=bc)
        da = oracle.dequantize(oracle.Format(block_cols=bc), {"codes": ca, "scales": sa}, M, K)
    if sides in ("both", "b"):
        qb, db, fb = mbs_operand(rng, N, K, bc, macro)
    else:
        cb, sb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8), rng.integers(118, 137, (N, K // bc), dtype=np.uint8)
        qb, fb = make_q(cb, sb, N, K), mx.Format(block_cols=bc)
        db = oracle.dequantize(oracle.Format(block_cols=bc), {"codes": cb, "scales": sb}, N, K)
    ref = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    assert rel_frob(c32, ref) <= 1e-5
    assert rel_frob(oracle.bf16_bits_to_f32(c16), oracle.bf16_bits_to_f32(bf16_of(ref))) <= 1e-3


@pytest.mark.parametrize("M,N,K", [(130, 200, 512), (33, 65, 256)])
def test_mbs_sub_blocks_exact_case(M, N, K):
    """Unit block scales and macro scales of 1 and 2 over 1 x 16 sub-blocks:
    every partial sum is a multiple of 1/4 below 2^24 in magnitude, so the fp32
    result equals the oracle's exact product bit for bit."""
    rng = np.random.default_rng(K + 17)
    qa, _, fa = mbs_operand(rng, M, K, 16, [0x38, 0x40])
    qb, _, fb = mbs_operand(rng, N, K, 16, [0x38, 0x40])
    for q in (qa, qb):
        q.scales.fill_(127)
    fo = oracle.Format(block_cols=16, macro_cols=128)
    da = oracle.dequantize(fo, {"codes": qa.codes.cpu().numpy().reshape(M, K // 2),
                                "scales": qa.scales.cpu().numpy().reshape(M, K // 16),
                                "macro_scales": qa.macro_scales.cpu().numpy().reshape(M, K // 128)}, M, K)
    db = oracle.dequantize(fo, {"codes": qb.codes.cpu().numpy().reshape(N, K // 2),
                                "scales": qb.scales.cpu().numpy().reshape(N, K // 16),
                                "macro_scales": qb.macro_scales.cpu().numpy().reshape(N, K // 128)}, N, K)
    exact = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(c32, exact.astype(np.float32))


def test_mbs_sub_blocks_quantized_operands():
    """c4's MBS format (1 x 128 UE4M3 macro over 1 x 16 E8M0 blocks) quantized
    on the GPU from activation-like and weight-like tensors, then multiplied:
    the product against the oracle's dequantized product, and its fidelity
    (eq. (2)) above plain 1 x 16 E8M0 blocks without the macro scales."""
    a, b = synth.w5(m=256, n=384, k=1024)
    f16m = mx.Format(block_cols=16, macro_cols=128)
    qa, _, _ = mx.mx_quantize(f16m, to_dev(a))
    qb, _, _ = mx.mx_quantize(f16m, to_dev(b))
    fo = oracle.Format(block_cols=16, macro_cols=128)
    ra, rb = oracle.quantize(a, fo), oracle.quantize(b, fo)
    ref = oracle.gemm_f64(ra["dequant"], rb["dequant"])
    c32 = mx.mx_gemm(f16m, qa, f16m, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(c32.cpu().numpy(), ref) <= 1e-5
    R = oracle.gemm_f64(synth.bf16_bits_to_f32(a), synth.bf16_bits_to_f32(b)).astype(np.float32)
    _, db_mbs = oracle.qsnr(R, c32.cpu().numpy())
    f16 = mx.Format(block_cols=16)
    pa, _, _ = mx.mx_quantize(f16, to_dev(a))
    pb, _, _ = mx.mx_quantize(f16, to_dev(b))
    _, db_16 = oracle.qsnr(R, mx.mx_gemm(f16, pa, f16, pb, out_dtype=torch.float32).cpu().numpy())
    assert db_mbs > db_16


# ---- FP4 under UE4M3 / NVFP4 / UE5M3 / non-32 E8M0 blocks: bf16 decode path ----
# (scale kind, block, unit scale code, codes drawn for random scales)
UPC = {"nvfp4": (oracle.SC_NVFP4, 16, 0x38, (0x28, 0x48)), "ue4m3": (oracle.SC_UE4M3, 16, 0x38, (0x28, 0x48)),
       "ue5m3": (oracle.SC_UE5M3, 16, 0x78, (0x68, 0x88)), "ue5m3_32": (oracle.SC_UE5M3, 32, 0x78, (0x68, 0x88)),
       "e8m0_16": (oracle.SC_E8M0, 16, 127, (118, 137)), "e8m0_64": (oracle.SC_E8M0, 64, 127, (118, 137)),
       "mxfp4": (oracle.SC_E8M0, 32, 127, (118, 137))}


def upc_operand(rng, kind, rows, K, unit=False, g=None):
    sc, bc, one, (lo, hi) = UPC[kind]
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = (np.full((rows, K // bc), one, np.uint8) if unit
              else rng.integers(lo, hi, (rows, K // bc), dtype=np.uint8))
    q = {"codes": codes, "scales": scales}
    dq = make_q(codes, scales, rows, K)
    if sc == oracle.SC_NVFP4:
        gv = np.array([1.0 if unit else g], np.float32)
        q["tensor_scale"] = gv
        dq.tensor_scale = torch.from_numpy(gv).cuda()
    fo = oracle.Format(scale=sc, block_cols=bc)
    return dq, mx.Format(scale=sc, block_cols=bc), oracle.dequantize(fo, q, rows, K)


UPC_PAIRS = [("nvfp4", "nvfp4"), ("ue4m3", "ue4m3"), ("ue5m3", "ue5m3"), ("ue5m3_32", "e8m0_16"),
             ("e8m0_64", "e8m0_16"), ("nvfp4", "mxfp4"), ("mxfp4", "ue5m3")]


@pytest.mark.parametrize("ka,kb", UPC_PAIRS)
@pytest.mark.parametrize("M,N,K", [(130, 200, 1024), (33, 65, 96), (40, 72, 192)])
def test_upcvt_exact_case(ka, kb, M, N, K):
    """Unit block scales (and tensor scales): every product of two E2M1 values
    is a multiple of 1/4 and every partial sum is exact in fp32."""
    if K % UPC[ka][1] or K % UPC[kb][1]:
        pytest.skip("K is not a whole number of blocks")
    rng = np.random.default_rng(M + K)
    qa, fa, da = upc_operand(rng, ka, M, K, unit=True)
    qb, fb, db = upc_operand(rng, kb, N, K, unit=True)
    exact = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(c32, exact.astype(np.float32))
    assert np.array_equal(c16, bf16_of(exact))


@pytest.mark.parametrize("ka,kb", UPC_PAIRS)
@pytest.mark.parametrize("M,N,K", [(257, 130, 1024), (64, 96, 352), (520, 1030, 512), (512, 1024, 384)])
def test_upcvt_random_scales(ka, kb, M, N, K):
    """Random block scales: within fp32 accumulation error of the oracle's
    fp64 product.  The shapes take both kernels: K a multiple of 128 with
    1 x 16 or 1 x 32 blocks the LDS-staged one (several ragged tiles; an odd
    stage count; a tile count that is a multiple of 8), else the register one."""
    if K % UPC[ka][1] or K % UPC[kb][1]:
        pytest.skip("K is not a whole number of blocks")
    rng = np.random.default_rng(K + 7)
    qa, fa, da = upc_operand(rng, ka, M, K, g=3.0e-3)
    qb, fb, db = upc_operand(rng, kb, N, K, g=0.37)
    ref = oracle.gemm_f64(da, db)
    c32 = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    c16 = mx.mx_gemm(fa, qa, fb, qb).view(torch.int16).cpu().numpy().view(np.uint16)
    assert rel_frob(c32, ref) <= 1e-5
    assert rel_frob(oracle.bf16_bits_to_f32(c16), oracle.bf16_bits_to_f32(bf16_of(ref))) <= 1e-3


def test_nvfp4_quantized_operands():
    """NVFP4 operands quantized on the GPU (E2M1, UE4M3 per 16, fp32 tensor
    scale): the product against the oracle's dequantized product; its QSNR
    (eq. (2)) above MXFP4's on the same data ('Unveiling ... MXFP4', Sec. 3)."""
    a, b = synth.w5(m=256, n=384, k=1024)
    fmt, fo = mx.Format(scale=mx.SCALE_NVFP4, block_cols=16), oracle.Format(scale=oracle.SC_NVFP4, block_cols=16)
    qa, _, _ = mx.mx_quantize(fmt, to_dev(a))
    qb, _, _ = mx.mx_quantize(fmt, to_dev(b))
    ref = oracle.gemm_f64(oracle.quantize(a, fo)["dequant"], oracle.quantize(b, fo)["dequant"])
    c32 = mx.mx_gemm(fmt, qa, fmt, qb, out_dtype=torch.float32).cpu().numpy()
    assert rel_frob(c32, ref) <= 1e-5
    R = oracle.gemm_f64(synth.bf16_bits_to_f32(a), synth.bf16_bits_to_f32(b)).astype(np.float32)
    q4a, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(a))
    q4b, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(b))
    _, db_nv = oracle.qsnr(R, c32)
    _, db_4 = oracle.qsnr(R, mx.mx_gemm(mx.MXFP4, q4a, mx.MXFP4, q4b, out_dtype=torch.float32).cpu().numpy())
    assert db_nv > db_4


def test_quantized_operands_and_qsnr_eq2():
    """W4A4 product of operands quantized on the GPU, and QSNR(AB) of eq. (2)
    ('Unveiling ... MXFP4', Sec. 3) against the bf16 product."""
    a, b = synth.w5(m=256, n=384, k=1024)
    fa = oracle.Format()
    ra = oracle.quantize(a, fa)
    rb = oracle.quantize(b, fa)
    ref = oracle.gemm_f64(ra["dequant"], rb["dequant"])
    qa, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(a))
    qb, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(b))
    c32 = mx.mx_gemm(mx.MXFP4, qa, mx.MXFP4, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(c32.cpu().numpy(), ref) <= 1e-5
    # eq. (2): reference product of the unquantized bf16 operands
    R = oracle.gemm_f64(synth.bf16_bits_to_f32(a), synth.bf16_bits_to_f32(b)).astype(np.float32)
    st_ref, db_ref = oracle.qsnr(R, c32.cpu().numpy())
    st, db = mx.mx_qsnr(torch.from_numpy(R).cuda(), c32)
    assert abs(db - db_ref) <= 1e-4
    assert st["nonzero"] == st_ref["nonzero"] and st["flushed"] == st_ref["flushed"]
    assert 10 < db < 30           # 4-bit operands: a QSNR in the teens of dB


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_qsnr_kernel(dtype):
    x = synth.w1(shape=(333, 1000))
    y = (x + np.float32(1e-3) * synth.w1(shape=(333, 1000), seed=9)).astype(np.float32)
    if dtype == "bf16":
        x, y = synth.to_bf16_bits(x), synth.to_bf16_bits(y)
    st_ref, db_ref = oracle.qsnr(x, y)
    st, db = mx.mx_qsnr(to_dev(x), to_dev(y))
    assert abs(db - db_ref) <= 1e-4
    for k in ("n", "nonzero", "flushed"):
        assert st[k] == st_ref[k]


@pytest.mark.slow
def test_full_size_whole_product():
    """The benchmark's product at its full shape, A 8192x4096 ~ N(0, 1) and
    B 14336x4096 ~ N(0, 0.02^2) quantized to MXFP4 on the GPU, checked on
    every output against the oracle's float64 product of its own dequantized
    operands ("Unveiling ... MXFP4", Sec. 3, eq. (2)).

    The quantized operands first equal the oracle's bit for bit.  Then, for an
    output whose products are all multiples of q = 2^(eA_min - 1) * 2^(eB_min - 1)
    (the finest E2M1 step of its A row times that of its B row) and whose
    |a|.|b| bound (here Cauchy-Schwarz, ||a|| ||b||) stays below 2^24 q, every
    partial sum in any order is exact in fp32; there the bf16 output must be
    the nearest-even rounding of the exact sum, bit for bit.  Over the whole
    matrix the relative Frobenius error against the bf16-rounded oracle must
    stay within 1e-3."""
    from parity import compare_codes
    a, b = synth.w5()
    ra = oracle.quantize(a, oracle.Format())
    rb = oracle.quantize(b, oracle.Format())
    qa, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(a))
    qb, _, _ = mx.mx_quantize(mx.MXFP4, to_dev(b))
    c = mx.mx_gemm(mx.MXFP4, qa, mx.MXFP4, qb)
    torch.cuda.synchronize()
    compare_codes(ra, qa, "w5 A")
    compare_codes(rb, qb, "w5 B")
    got = c.view(torch.int16).cpu().numpy().view(np.uint16)
    del c
    exact = oracle.gemm_f64(ra["dequant"], rb["dequant"])
    want = bf16_of(exact)
    # the finest E2M1 step per row: half the smallest block scale of the row
    step_a = np.exp2(ra["scales"].min(axis=1).astype(np.float64) - 127 - 1)
    step_b = np.exp2(rb["scales"].min(axis=1).astype(np.float64) - 127 - 1)
    na = np.linalg.norm(ra["dequant"].astype(np.float64), axis=1)
    nb = np.linalg.norm(rb["dequant"].astype(np.float64), axis=1)
    exact_in_fp32 = np.outer(na / step_a, nb / step_b) < 2.0 ** 24
    frac_exact = exact_in_fp32.mean()
    assert frac_exact > 0.99, f"only {frac_exact:.4f} of the outputs are exact in fp32"
    bad = np.argwhere(exact_in_fp32 & (got != want))
    assert bad.size == 0, f"{len(bad)} exactly summable outputs differ, first at {bad[:3].tolist()}"
    assert np.array_equal(np.isnan(exact), np.zeros_like(exact, bool))
    got32 = oracle.bf16_bits_to_f32(got)
    del got
    assert rel_frob(got32, oracle.bf16_bits_to_f32(want)) <= 1e-3


# ---- non-finite inputs: the quantizer's NaN block scale through every path ----
NAN_CASES = [("mxfp4", "mxfp4", 1024), ("mxfp4", "mxfp4", 384), ("mxfp4", "mxfp4", 96), ("e2m3", "mxfp4", 384),
             ("nvfp4", "nvfp4", 1024), ("nvfp4", "nvfp4", 96), ("ue5m3", "ue5m3", 1024), ("nvfp4", "mxfp4", 1024)]


def nan_formats(kind):
    return {"mxfp4": (mx.MXFP4, oracle.Format()),
            "e2m3": (mx.Format(elem=mx.ELEM_FP6_E2M3), oracle.Format(elem=oracle.FP6_E2M3)),
            "nvfp4": (mx.Format(scale=mx.SCALE_NVFP4, block_cols=16),
                      oracle.Format(scale=oracle.SC_NVFP4, block_cols=16)),
            "ue5m3": (mx.Format(scale=mx.SCALE_UE5M3, block_cols=16),
                      oracle.Format(scale=oracle.SC_UE5M3, block_cols=16))}[kind]


@pytest.mark.parametrize("ka,kb,K", NAN_CASES)
def test_nonfinite_block_propagates(ka, kb, K):
    """A block holding NaN or Inf gets the NaN scale code (E8M0 0xFF; UE4M3
    0x7F; UE5M3 0xFF) and zero codes, so its dequantized values are NaN; in
    the product that makes the block's row of A (column of B) all NaN, on the
    native scaled instruction (the hardware's E8M0 NaN), the LDS-staged and
    register-only kernels and both decode routes alike.  The rest of C
    matches the oracle's product."""
    rng = np.random.default_rng(K + len(ka))
    M, N = 40, 48
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    a[3, 5] = np.nan
    b[7, K - 1] = np.inf
    (fa, ra), (fb, rb) = nan_formats(ka), nan_formats(kb)
    qa, _, _ = mx.mx_quantize(fa, to_dev(a))
    qb, _, _ = mx.mx_quantize(fb, to_dev(b))
    da, db = oracle.quantize(a, ra)["dequant"], oracle.quantize(b, rb)["dequant"]
    with np.errstate(invalid="ignore"):
        ref = oracle.gemm_f64(da, db)
    c = mx.mx_gemm(fa, qa, fb, qb, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(np.isnan(c), np.isnan(ref))
    assert np.isnan(c[3]).all() and np.isnan(c[:, 7]).all()
    fin = ~np.isnan(ref)
    assert rel_frob(c[fin], ref[fin]) <= 1e-5


# ---- C as a strided view: every kernel's store path ---------------------------
@pytest.mark.parametrize("kind,K", [("mxfp4", 1024), ("mxfp4", 384), ("mxfp4", 96), ("e2m3", 384), ("nvfp4", 1024),
                                    ("nvfp4", 96)])
@pytest.mark.parametrize("pad", [8, 3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_strided_output(kind, K, pad, dtype):
    """C written into the first N columns of a wider buffer (row stride
    N + pad elements; pad 8 keeps bf16 rows 16-byte aligned for the tiled
    kernel's vector stores, pad 3 does not): the same values as a dense C and
    the padding columns untouched."""
    rng = np.random.default_rng(K + pad)
    M, N = 300, 264
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    (fa, _), (fb, _) = nan_formats(kind), nan_formats("mxfp4" if kind == "e2m3" else kind)
    qa, _, _ = mx.mx_quantize(fa, to_dev(a))
    qb, _, _ = mx.mx_quantize(fb, to_dev(b))
    dense = mx.mx_gemm(fa, qa, fb, qb, out_dtype=dtype)
    big = torch.full((M, N + pad), 7.0, dtype=dtype, device=dense.device)
    view = big[:, :N]
    mx.mx_gemm(fa, qa, fb, qb, c=view)
    torch.cuda.synchronize()
    assert torch.equal(view, dense)
    assert bool((big[:, N:] == 7.0).all())
