"""Helpers for the GPU parity tests: run the HIP library and the CPU oracle on
the same seeded input and compare codes, scales, side outputs and dequantized
values bit for bit, and the statistics within tolerance."""
import math

import numpy as np
import torch

import microscaling_block_quantization_amd as mx
import oracle

QSNR_TOL_DB = 1e-4        # the QSNR tolerance of the parity contract


def to_dev(x):
    """numpy float32 / uint16 (bf16 bits) -> torch device tensor"""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32).copy()).cuda()


def host_u8(t, n):
    return t.detach().cpu().numpy().reshape(-1)[:n]


def run_gpu(x, kw, dq_dtype=torch.float32, stats=True):
    """One mx_quantize call (dq_dtype None: no dequantized output).  MXFP4
    (E2M1, E8M0 scales, RTNE, dense rows) takes the fast kernel with every
    output set; the benchmark times it with statistics and no dequantized
    output.  Other formats take their own kernels."""
    xd = to_dev(x)
    q, dq, st = mx.mx_quantize(mx.Format(**kw), xd, dequant=dq_dtype, stats=True if stats else None)
    torch.cuda.synchronize()
    return q, dq, (mx.stats_to_dict(st) if stats else None)


def bits_equal_f32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def qsnr_of(st):
    if st["err2"] == 0:
        return math.inf
    return 10 * math.log10(st["sig2"] / st["err2"])


def compare_codes(ref, q, label):
    """codes, scales and the format's side outputs, bit for bit"""
    codes = host_u8(q.codes, ref["codes"].size).reshape(ref["codes"].shape)
    bad = np.argwhere(codes != ref["codes"])
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first at {bad[:3].tolist()}: " \
        f"gpu {codes[tuple(bad[0])]:#04x} ref {ref['codes'][tuple(bad[0])]:#04x}"
    scales = host_u8(q.scales, ref["scales"].size).reshape(ref["scales"].shape)
    bad = np.argwhere(scales != ref["scales"])
    assert bad.size == 0, f"{label}: {len(bad)} scales differ, first at {bad[:3].tolist()}: " \
        f"gpu {scales[tuple(bad[0])]} ref {ref['scales'][tuple(bad[0])]}"
    if ref["offsets"] is not None:
        off = q.offsets.cpu().numpy().view(np.uint16)[:ref["offsets"].size].reshape(ref["offsets"].shape)
        assert np.array_equal(off, ref["offsets"]), f"{label}: offsets differ"
    if ref["macro_scales"] is not None:
        m = host_u8(q.macro_scales, ref["macro_scales"].size).reshape(ref["macro_scales"].shape)
        assert np.array_equal(m, ref["macro_scales"]), f"{label}: macro scales differ"
    if ref["tensor_scale"] is not None:
        assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == ref["tensor_scale"].view(np.uint32)[0], label
    if ref["ref_exp"] is not None:
        assert int(q.ref_exp.cpu()[0]) == int(ref["ref_exp"][0]), label


def compare_stats(rs, st, label):
    """counts exactly, QSNR within the contract's tolerance"""
    for k in ("n", "nonzero", "flushed", "zero_blocks"):
        assert st[k] == rs[k], f"{label}: stats {k} {st[k]} != {rs[k]}"
    if math.isfinite(rs["sig2"]) and rs["sig2"] > 0:
        a, b = qsnr_of(st), qsnr_of(rs)
        if math.isfinite(b):
            assert abs(a - b) <= QSNR_TOL_DB, f"{label}: QSNR {a} vs {b}"
        else:
            assert a == b, f"{label}: QSNR {a} vs {b}"


def check_quantize(x, kw, label="", dq_dtype=torch.float32):
    """Full element-by-element parity of one quantization, through every
    output set a caller can ask for: with a dequantized output and statistics,
    with statistics only, and codes only (dense rows take the same kernel in
    all three: the fast one for MXFP4, the wave-tile one for the formats it
    covers).  Each route is held to the oracle:
    codes, scales and side outputs bit for bit, dequantized values bit for
    bit, counts exactly, QSNR within 1e-4 dB."""
    ref = oracle.quantize(x, oracle.Format(**kw),
                          dq_dtype=oracle.BF16 if dq_dtype == torch.bfloat16 else oracle.F32)
    q, dq, st = run_gpu(x, kw, dq_dtype)
    compare_codes(ref, q, f"{label} [dequant+stats]")
    if dq_dtype == torch.bfloat16:
        got = dq.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref["dequant"]), f"{label}: bf16 dequant differs"
    else:
        got = dq.cpu().numpy()
        assert bits_equal_f32(got, ref["dequant"]), f"{label}: dequant differs at " \
            f"{np.argwhere(got.view(np.uint32) != ref['dequant'].view(np.uint32))[:3].tolist()}"
    compare_stats(ref["stats"], st, f"{label} [dequant+stats]")
    q2, _, st2 = run_gpu(x, kw, None, stats=True)
    compare_codes(ref, q2, f"{label} [stats]")
    compare_stats(ref["stats"], st2, f"{label} [stats]")
    q3, _, _ = run_gpu(x, kw, None, stats=False)
    compare_codes(ref, q3, f"{label} [codes]")
    return ref, q


def check_dequantize(ref, q, kw, rows, cols, out_dtype=torch.float32, label=""):
    y = mx.mx_dequantize(mx.Format(**kw), q, out_dtype=out_dtype)
    torch.cuda.synchronize()
    want = oracle.dequantize(oracle.Format(**kw), ref, rows, cols,
                             out_dtype=oracle.BF16 if out_dtype == torch.bfloat16 else oracle.F32)
    if out_dtype == torch.bfloat16:
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), want), label
    else:
        assert bits_equal_f32(y.cpu().numpy(), want), label
