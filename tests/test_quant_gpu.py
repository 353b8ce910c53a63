"""GPU parity of the quantizer: the HIP library against the CPU oracle, element
by element, on seeded synthetic inputs shaped like the pages' workloads
(reduced sizes that still span many workgroups and a ragged tail), plus the
edge cases.  Codes, scales, offsets, macro scales, tensor scales and
dequantized values must match bit for bit; counts exactly; QSNR within 1e-4 dB.
"""
import numpy as np
import pytest
import torch

import synth
from parity import check_dequantize, check_quantize

pytestmark = pytest.mark.gpu

E2M1, INT4, E2M3, E3M2, E3M0, E4M3, E5M2 = 0, 1, 2, 3, 4, 5, 6
E8M0, UE4M3, NVFP4, UE5M3, SE3M0 = 0, 1, 2, 3, 4
FLOOR, CEIL, OAS = 0, 1, 2
RTNE, SR, CEILR = 0, 1, 2


def kid(kw):
    return ",".join(f"{k}={v}" for k, v in kw.items()) or "mxfp4"


# ---- fp32 1024x1024 N(0, 0.02^2), MXFP4 1x32, FLOOR, RTNE: the full-size small case
def test_w1_mxfp4_full_size():
    x = synth.w1()
    ref, q = check_quantize(x, {}, "w1")
    check_dequantize(ref, q, {}, 1024, 1024)


def test_w1_bf16_dequant_output():
    x = synth.w1(shape=(256, 1024))
    check_quantize(x, {}, "w1-bf16dq", dq_dtype=torch.bfloat16)


# ---- NVFP4 vs MXFP4 vs UE5M3 (+ UE4M3 without tensor scale) block-size sweep, N(0, sigma^2) bf16
W2_CASES = [dict(scale=s, block_cols=b) for s in (E8M0, NVFP4, UE5M3, UE4M3) for b in (8, 16, 32, 64, 128, 256)]


@pytest.mark.parametrize("sigma", [1e-3, 2e-2])
@pytest.mark.parametrize("kw", W2_CASES, ids=kid)
def test_w2_sweep(sigma, kw):
    x = synth.w2(sigma, shape=(200, 1024), seed=102)
    check_quantize(x, kw, f"w2 sigma={sigma} {kid(kw)}")


# ---- gradient-like Laplace(0, 1e-4) with 0.1% x50 entries, bf16
W3_FORMATS = [dict(round=SR, seed=synth.SR_SEED),
              dict(scale=SE3M0, rule=CEIL),
              dict(elem=INT4, asymmetric=1, rule=CEIL)]
W3_SHAPES = [dict(block_rows=1, block_cols=32), dict(block_rows=32, block_cols=1),
             dict(block_rows=32, block_cols=32)]


@pytest.mark.parametrize("shape", W3_SHAPES, ids=kid)
@pytest.mark.parametrize("kw", W3_FORMATS, ids=kid)
def test_w3_gradients(kw, shape):
    x = synth.w3(shape=(96, 1792), seed=103)
    kw = {**kw, **shape}
    ref, q = check_quantize(x, kw, f"w3 {kid(kw)}")
    check_dequantize(ref, q, kw, 96, 1792)


# ---- activation-like Laplace(0, 1) with 8 outlier channels x100, bf16
W4_FORMATS = [dict(), dict(hadamard=32), dict(hadamard=128), dict(block_cols=16),
              dict(rule=OAS, oas_tau=6.0), dict(rule=OAS, oas_tau=7.0), dict(rule=OAS, oas_tau=7.5),
              dict(rule=OAS, oas_tau=7.5, block_cols=16), dict(rule=CEIL, block_cols=16),
              dict(macro_cols=128, block_cols=16, rule=CEIL),
              dict(macro_cols=128, block_cols=16, rule=OAS, oas_tau=7.5),
              dict(macro_cols=128, block_cols=32, rule=FLOOR),
              dict(scale=NVFP4, block_cols=16), dict(scale=NVFP4, block_cols=16, hadamard=16),
              dict(scale=NVFP4, block_cols=16, hadamard=32), dict(hadamard=64, rule=OAS, oas_tau=7.5),
              dict(hadamard=32, round=SR, seed=17), dict(macro_cols=128, block_cols=16, rule=CEIL, round=SR, seed=19),
              dict(elem=INT4, hadamard=32)]


@pytest.mark.parametrize("kw", W4_FORMATS, ids=kid)
def test_w4_activations(kw):
    x = synth.w4(shape=(128, 1024), seed=104)
    ref, q = check_quantize(x, kw, f"w4 {kid(kw)}")
    check_dequantize(ref, q, kw, 128, 1024)


# ---- every element type and rounding mode, both input dtypes
ELEM_FORMATS = [dict(elem=INT4), dict(elem=INT4, rule=CEIL), dict(elem=E2M3), dict(elem=E3M2, rule=CEIL),
                dict(elem=E3M0), dict(elem=E3M0, round=CEILR), dict(round=CEILR),
                dict(elem=INT4, round=SR, seed=7), dict(elem=E2M3, round=SR, seed=9, rng_offset=3),
                dict(asymmetric=1), dict(asymmetric=1, rule=CEIL, round=SR, seed=1),
                dict(elem=INT4, asymmetric=1, rule=OAS, oas_tau=20.0),
                dict(scale=UE5M3, elem=E3M2, block_cols=16), dict(scale=NVFP4, elem=INT4, block_cols=16),
                dict(scale=SE3M0, rule=CEIL, elem=E2M3),
                dict(elem=E4M3), dict(elem=E5M2, rule=CEIL), dict(elem=E4M3, round=SR, seed=13),
                dict(elem=E5M2, round=CEILR), dict(elem=E4M3, rule=OAS, oas_tau=500.0),
                dict(elem=E5M2, scale=UE5M3, block_cols=16)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kw", ELEM_FORMATS, ids=kid)
def test_element_types(dtype, kw):
    x = synth.w4(shape=(72, 512), seed=21)
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x) * np.float32(1.0 + 2.0 ** -12)
    ref, q = check_quantize(x, kw, f"{dtype} {kid(kw)}")
    check_dequantize(ref, q, kw, 72, 512)
    check_dequantize(ref, q, kw, 72, 512, out_dtype=torch.bfloat16)


# ---- the MXFP4 fast kernel (with and without a dequantized output), every instantiation:
# bf16 and fp32 input, every block width it takes, the FLOOR rule and the
# exact-comparison rules (CEIL, OAS); 201 x 1280 leaves a ragged last wave tile
FAST_RULES = [dict(), dict(rule=CEIL), dict(rule=OAS, oas_tau=6.0), dict(rule=OAS, oas_tau=7.0),
              dict(rule=OAS, oas_tau=7.5), dict(rule=OAS, oas_tau=11.9)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b", [8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("rule", FAST_RULES, ids=kid)
def test_fast_kernel_instantiations(dtype, b, rule):
    x = synth.w4(shape=(201, 1280), seed=51)
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x) * np.float32(1.0 + 2.0 ** -12)
    check_quantize(x, {**rule, "block_cols": b}, f"fast {dtype} b={b} {kid(rule)}")


# ---- bf16 dequantized output of the wave-tile row kernel's formats, both
# input dtypes (fp32 input stores half as many bytes per chunk)
HW_DQ_FORMATS = [dict(scale=NVFP4, block_cols=16), dict(scale=UE5M3), dict(scale=SE3M0, rule=CEIL),
                 dict(round=SR, seed=5), dict(elem=INT4, asymmetric=1, rule=CEIL), dict(hadamard=32),
                 dict(macro_cols=128, block_cols=16, rule=CEIL)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kw", HW_DQ_FORMATS, ids=kid)
def test_bf16_dequant_output_wave_tile_formats(dtype, kw):
    x = synth.w4(shape=(201, 1280), seed=61)
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x) * np.float32(1.0 + 2.0 ** -12)
    check_quantize(x, kw, f"bf16 dq {dtype} {kid(kw)}", dq_dtype=torch.bfloat16)


# ---- column and 2D blocks of every size, both dtypes
TILE_FORMATS = [dict(), dict(round=SR, seed=3), dict(scale=NVFP4), dict(elem=INT4, asymmetric=1, rule=CEIL),
                dict(asymmetric=1), dict(elem=E3M2), dict(scale=UE5M3, rule=CEIL), dict(scale=SE3M0, rule=CEIL),
                dict(elem=E4M3), dict(elem=E5M2, round=SR, seed=4)]


@pytest.mark.parametrize("b", [8, 16, 32])
@pytest.mark.parametrize("two_d", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kw", TILE_FORMATS, ids=kid)
def test_column_and_2d_blocks(b, two_d, dtype, kw):
    x = synth.w3(shape=(96, 512), seed=31)
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x)
    kw = {**kw, "block_rows": b, "block_cols": b if two_d else 1}
    ref, q = check_quantize(x, kw, f"tiles {dtype} {kid(kw)}")
    check_dequantize(ref, q, kw, 96, 512)


# ---- edge cases
def test_eight_column_chunks():
    """cols = 8 mod 16 takes the 8-element-per-thread path"""
    x = synth.w2(0.02, shape=(33, 1032), seed=5)
    for kw in (dict(block_cols=8), dict(block_cols=8, scale=NVFP4), dict(block_cols=8, elem=E2M3, round=SR, seed=2)):
        check_quantize(x, kw, f"ch8 {kid(kw)}")


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 64), (1, 8), (257, 96)])
def test_ragged_and_tiny(rows, cols):
    x = synth.w2(0.02, shape=(rows, cols), seed=6)
    kws = [dict(), dict(scale=NVFP4, block_cols=16)] if cols % 16 == 0 else [dict(block_cols=8)]
    for kw in kws:
        if cols % kw.get("block_cols", 32):
            continue
        check_quantize(x, kw, f"ragged {rows}x{cols} {kid(kw)}")


def test_empty_tensor():
    import microscaling_block_quantization_amd as mx
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, dq, st = mx.mx_quantize(mx.Format(), x, dequant=torch.float32, stats=True)
    torch.cuda.synchronize()
    s = mx.stats_to_dict(st)
    assert s["n"] == 0 and s["sig2"] == 0 and s["zero_blocks"] == 0
    q, _, _ = mx.mx_quantize(mx.Format(scale=NVFP4, block_cols=16), x)
    torch.cuda.synchronize()
    assert float(q.tensor_scale.cpu()[0]) == 1.0


def test_special_values():
    x = synth.w1(shape=(8, 256))
    x[0, 3] = np.nan
    x[1, 40] = np.inf
    x[2, 70] = -np.inf
    x[3, :32] = 0.0
    x[3, 32:64] = -0.0
    x[4, :32] = np.float32(1e-40)              # denormals
    x[4, 32:64] = np.float32(-3e-39)
    x[5, :32] = np.float32(2.0 ** -130) * np.arange(32, dtype=np.float32)
    x[6, :32] = np.float32(3.0e38)
    x[6, 32:64] = np.float32(-3.3e38) * np.linspace(0.01, 1, 32, dtype=np.float32)
    x[7, :32] = np.float32(6.0) * np.float32(2.0 ** -126)
    for kw in (dict(), dict(rule=CEIL), dict(rule=OAS, oas_tau=7.5), dict(scale=NVFP4, block_cols=16),
               dict(scale=UE5M3, block_cols=16), dict(scale=UE4M3, block_cols=16), dict(round=SR, seed=11),
               dict(elem=INT4, asymmetric=1, rule=CEIL), dict(asymmetric=1), dict(scale=SE3M0, rule=CEIL),
               dict(elem=E3M2), dict(round=CEILR), dict(block_rows=8, block_cols=8), dict(elem=E4M3),
               dict(elem=E5M2, block_rows=8, block_cols=1), dict(asymmetric=1, block_rows=8, block_cols=8)):
        check_quantize(x, kw, f"special {kid(kw)}")


SPECIAL_FORMATS = [dict(), dict(rule=CEIL), dict(rule=OAS, oas_tau=7.5), dict(block_cols=8),
                   dict(block_cols=64, rule=CEIL), dict(block_cols=256),
                   dict(elem=E4M3), dict(elem=E5M2, rule=CEIL), dict(elem=E4M3, rule=OAS, oas_tau=500.0),
                   dict(elem=E2M3), dict(elem=E3M2, rule=CEIL), dict(elem=E2M3, rule=OAS, oas_tau=9.0)]


def special_tensor_bf16():
    """the special rows above in bf16: NaN, +-Inf, +-0 blocks, subnormal blocks
    (bf16 keeps fp32's exponent range), a block of 2^-130 * k, blocks near the
    largest finite value, and a block at 6 * 2^-126"""
    x = synth.w1(shape=(8, 256))
    x[0, 3] = np.nan
    x[1, 40] = np.inf
    x[2, 70] = -np.inf
    x[3, :32] = 0.0
    x[3, 32:64] = -0.0
    x[4, :32] = np.float32(1e-40)
    x[4, 32:64] = np.float32(-3e-39)
    x[4, 64:96] = np.float32(2.0 ** -133) * np.arange(32, dtype=np.float32)
    x[5, :32] = np.float32(2.0 ** -130) * np.arange(32, dtype=np.float32)
    x[5, 32:64] = -np.float32(2.0 ** -127) * np.arange(32, dtype=np.float32)
    x[6, :32] = np.float32(3.0e38)
    x[6, 32:64] = np.float32(-3.3e38) * np.linspace(0.01, 1, 32, dtype=np.float32)
    x[7, :32] = np.float32(6.0) * np.float32(2.0 ** -126)
    return synth.to_bf16_bits(x)


@pytest.mark.parametrize("kw", SPECIAL_FORMATS, ids=kid)
def test_special_values_bf16(kw):
    """bf16 input through every route, the fast kernel included: there the
    convert sees x * 2^127 for subnormal blocks and keeps the sign of zero"""
    check_quantize(special_tensor_bf16(), kw, f"special bf16 {kid(kw)}")


def test_repeat_runs_are_bit_identical():
    import microscaling_block_quantization_amd as mx
    x = torch.from_numpy(synth.w2(0.02, shape=(512, 2048), seed=8).view(np.int16)).cuda().view(torch.bfloat16)
    outs = []
    for _ in range(2):
        q, dq, st = mx.mx_quantize(mx.Format(round=SR, seed=5), x, dequant=torch.float32, stats=True)
        torch.cuda.synchronize()
        outs.append((q.codes.cpu(), q.scales.cpu(), dq.cpu(), st.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ---- the pages' full workload shapes (same launch configuration as the benchmark)
@pytest.mark.slow
@pytest.mark.parametrize("kw", [dict(), dict(scale=NVFP4, block_cols=16), dict(scale=UE5M3, block_cols=8)], ids=kid)
def test_w2_full_size(kw):
    x = synth.w2(2e-2)
    check_quantize(x, kw, f"w2 full {kid(kw)}")


@pytest.mark.slow
def test_w3_full_size_sr():
    x = synth.w3()
    check_quantize(x, dict(round=SR, seed=synth.SR_SEED, block_rows=32, block_cols=32), "w3 full SR 2D")


# the gradient cells whose rows take the wave-tile kernel, and column blocks of the others
@pytest.mark.slow
@pytest.mark.parametrize("kw", [dict(round=SR, seed=synth.SR_SEED), dict(scale=SE3M0, rule=CEIL),
                                dict(elem=INT4, asymmetric=1, rule=CEIL),
                                dict(scale=SE3M0, rule=CEIL, block_rows=32, block_cols=1),
                                dict(elem=INT4, asymmetric=1, rule=CEIL, block_rows=32, block_cols=1)], ids=kid)
def test_w3_full_size_cells(kw):
    x = synth.w3()
    check_quantize(x, kw, f"w3 full {kid(kw)}")


@pytest.mark.slow
def test_w4_full_size_h128():
    x = synth.w4()
    check_quantize(x, dict(hadamard=128), "w4 full H128")


@pytest.mark.slow
def test_w5_operands_full_size():
    a, b = synth.w5()
    check_quantize(a, {}, "w5 A")
    check_quantize(b, {}, "w5 B")


@pytest.mark.slow
def test_w5_as_the_benchmark_calls():
    """The benchmark's own call sequence at its full shapes: preallocated codes,
    scales, workspace and statistics, no dequantized output (the fast kernel
    with fused statistics), A then B on one stream.  Codes and scales bit for
    bit, counts exactly and QSNR within 1e-4 dB of the oracle."""
    import microscaling_block_quantization_amd as mx
    from parity import compare_codes, compare_stats, to_dev
    import oracle
    a, b = synth.w5()
    fmt = mx.MXFP4
    outs = []
    for x in (a, b):
        xd = to_dev(x)
        rows, cols = x.shape
        q = mx.alloc_qtensor(fmt, rows, cols, xd.device)
        ws = mx.alloc_workspace(fmt, rows, cols, xd.device)
        st = torch.empty(64, dtype=torch.uint8, device=xd.device)
        mx.mx_quantize(fmt, xd, out=q, stats=st, workspace=ws)
        outs.append((q, st))
    torch.cuda.synchronize()
    for (q, st), x, name in zip(outs, (a, b), "AB"):
        ref = oracle.quantize(x, oracle.Format())
        compare_codes(ref, q, f"w5 {name} bench call")
        compare_stats(ref["stats"], mx.stats_to_dict(st), f"w5 {name} bench call")


@pytest.mark.parametrize("kw", [dict(), dict(rule=CEIL, block_cols=16), dict(rule=OAS, oas_tau=7.5),
                                dict(block_cols=8)], ids=kid)
def test_strided_input_takes_the_general_kernel(kw):
    """A row stride larger than the row (a column slice of a wider tensor)
    goes through the general row kernel; its codes, scales and counts equal
    those of the dense call without a dequantized output (the MXFP4 fast
    kernel), and the oracle's on the dense copy."""
    import microscaling_block_quantization_amd as mx
    from parity import to_dev
    x = synth.w4(shape=(96, 1024), seed=41)
    wide = to_dev(np.concatenate([x, x[:, :256]], axis=1))
    xs = wide[:, :1024]
    assert xs.stride(0) == 1280
    q1, dq1, st1 = mx.mx_quantize(mx.Format(**kw), xs, dequant=torch.float32, stats=True)
    q2, _, st2 = mx.mx_quantize(mx.Format(**kw), to_dev(x), stats=True)     # dense: the fast kernel
    torch.cuda.synchronize()
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    s1, s2 = mx.stats_to_dict(st1), mx.stats_to_dict(st2)
    for k in ("nonzero", "flushed", "zero_blocks", "n"):
        assert s1[k] == s2[k]
    check_quantize(x, kw, f"dense {kid(kw)}")


def test_one_workspace_serves_every_call():
    """One workspace, large enough for all of them and filled with a stale
    pattern, serves a run of statistics calls of different formats, shapes
    and kernel routes (fast rows, hardware-convert rows, general rows, 2D
    tiles, an empty tensor), each matching the oracle."""
    import microscaling_block_quantization_amd as mx
    from parity import compare_stats, to_dev
    import oracle
    cases = [(synth.w2(1.0, shape=(256, 1024), seed=11), dict()),
             (synth.w2(0.02, shape=(128, 2048), seed=12), dict(scale=NVFP4, block_cols=16)),
             (synth.w2(1.0, shape=(64, 512), seed=13), dict(elem=E2M3, rule=CEIL)),
             (synth.w2(1.0, shape=(96, 256), seed=14), dict(block_rows=32, block_cols=32)),
             (synth.w2(1.0, shape=(256, 1024), seed=11), dict()),
             (np.zeros((0, 64), dtype=np.float32), dict())]
    need = max(mx.mx_query_sizes(mx.Format(**kw), *x.shape)["workspace"] for x, kw in cases)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    for i, (x, kw) in enumerate(cases):
        fmt = mx.Format(**kw)
        xd = to_dev(x) if x.size else torch.empty(x.shape, dtype=torch.float32, device="cuda")
        q = mx.alloc_qtensor(fmt, *x.shape, xd.device)
        st = torch.full((64,), 0xA5, dtype=torch.uint8, device=xd.device)
        mx.mx_quantize(fmt, xd, out=q, stats=st, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.quantize(x, oracle.Format(**kw))
        got = mx.stats_to_dict(st)
        if x.size == 0:
            assert got["n"] == 0 and got["sig2"] == 0 and got["nonzero"] == 0
        else:
            compare_stats(ref["stats"], got, f"shared workspace call {i} {kid(kw)}")
