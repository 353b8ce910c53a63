"""CPU oracle for microscaling block quantization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library:
the C source ``mx_ref.c`` carries its own format tables and rules, written from
the pages that define the method (the MXFP4/NVFP4 component lists and QSNR
eq. (1)-(2) of "Unveiling the Potential of Quantization with MXFP4", the UE5M3
scale of "Is Finer Better?", the block Hadamard rotation of "Bridging the Gap
... Microscaling FP4 Quantization", and the element types, rounding modes and
block organisations of the ARITH 2025 MX-training report).

Arrays are numpy: fp32 tensors as ``float32``, bf16 tensors as their raw
``uint16`` bits.  The block-scaled GEMM oracle is the plain definition: the
dequantized operands (exact in fp32) multiplied with float64 accumulation.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxref.so")

# element types, scale types, exponent rules, rounding modes, dtypes
E2M1, INT4, FP6_E2M3, FP6_E3M2, E3M0, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4, 5, 6
SC_E8M0, SC_UE4M3, SC_NVFP4, SC_UE5M3, SC_E3M0 = 0, 1, 2, 3, 4
RULE_FLOOR, RULE_CEIL, RULE_OAS = 0, 1, 2
RTNE, SR, CEIL = 0, 1, 2
F32, BF16 = 0, 1


class _Fmt(ctypes.Structure):
    _fields_ = [("elem", ctypes.c_int32), ("scale", ctypes.c_int32),
                ("rule", ctypes.c_int32), ("round", ctypes.c_int32),
                ("block_rows", ctypes.c_int32), ("block_cols", ctypes.c_int32),
                ("asymmetric", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("macro_cols", ctypes.c_int32), ("oas_tau", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("rng_offset", ctypes.c_uint64)]


class _QT(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("macro_scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("ref_exp", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _Stats(ctypes.Structure):
    _fields_ = [("sig2", ctypes.c_double), ("err2", ctypes.c_double),
                ("n", ctypes.c_int64), ("nonzero", ctypes.c_int64),
                ("flushed", ctypes.c_int64), ("zero_blocks", ctypes.c_int64)]


@dataclass
class Format:
    elem: int = E2M1
    scale: int = SC_E8M0
    rule: int = RULE_FLOOR
    round: int = RTNE
    block_rows: int = 1
    block_cols: int = 32
    asymmetric: int = 0
    hadamard: int = 0
    macro_cols: int = 0
    oas_tau: float = 0.0
    seed: int = 0
    rng_offset: int = 0

    def _c(self):
        return _Fmt(self.elem, self.scale, self.rule, self.round, self.block_rows,
                    self.block_cols, self.asymmetric, self.hadamard, self.macro_cols,
                    self.oas_tau, self.seed, self.rng_offset)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, u64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_uint32, ctypes.c_uint64)
        L.ref_quantize.argtypes = [ctypes.POINTER(_Fmt), i32, vp, i64, i64, i64,
                                   ctypes.POINTER(_QT), vp, i32, ctypes.POINTER(_Stats)]
        L.ref_dequantize.argtypes = [ctypes.POINTER(_Fmt), ctypes.POINTER(_QT), i32, vp, i64]
        L.ref_qsnr.argtypes = [i32, vp, vp, i64, ctypes.POINTER(_Stats),
                               ctypes.POINTER(ctypes.c_double)]
        L.ref_philox4x32_10.argtypes = [vp, vp, vp]
        L.ref_philox4x32_10.restype = None
        L.ref_r16.argtypes = [u64, u64, u64]
        L.ref_r16.restype = u32
        L.ref_round_code.argtypes = [i32, i32, i32, ctypes.c_float, u32]
        L.ref_code_value.argtypes = [i32, i32, i32]
        L.ref_code_value.restype = ctypes.c_double
        L.ref_fp8_scale_code.argtypes = [i32, ctypes.c_float]
        L.ref_fp8_scale_value.argtypes = [i32, i32]
        L.ref_fp8_scale_value.restype = ctypes.c_double
        L.ref_e8m0_exponent.argtypes = [i32, ctypes.c_float, i32, i32, ctypes.c_float]
        L.ref_hadamard_const.argtypes = [i32]
        L.ref_hadamard_const.restype = ctypes.c_float
        L.ref_hadamard_row.argtypes = [i32, vp]
        L.ref_hadamard_row.restype = None
        L.ref_set_threads.argtypes = [i32]
        L.ref_set_threads.restype = None
        L.ref_get_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def elem_bits(elem):
    if elem in (FP8_E4M3, FP8_E5M2):
        return 8
    return 6 if elem in (FP6_E2M3, FP6_E3M2) else 4


def code_row_bytes(elem, cols):
    return {8: cols, 6: cols * 3 // 4}.get(elem_bits(elem), cols // 2)


def set_threads(n):
    lib().ref_set_threads(int(n))


def get_threads():
    return lib().ref_get_threads()


def quantize(x, fmt: Format, in_dtype=None, dq_dtype=F32):
    """Quantize a 2-D host array.  ``x`` is float32 (fp32) or uint16 (bf16 bits).

    Returns a dict with codes, scales (+ offsets, macro_scales, tensor_scale,
    ref_exp where the format has them), the dequantized tensor and the stats."""
    x = np.ascontiguousarray(x)
    if in_dtype is None:
        in_dtype = BF16 if x.dtype == np.uint16 else F32
    rows, cols = x.shape
    br, bc = fmt.block_rows, fmt.block_cols
    nsc = (rows // br) * (cols // bc) if br and bc else 0
    out = {
        "codes": np.zeros((rows, code_row_bytes(fmt.elem, cols)), np.uint8),
        "scales": np.zeros((rows // br, cols // bc), np.uint8),
        "offsets": np.zeros((rows // br, cols // bc), np.uint16) if fmt.asymmetric else None,
        "macro_scales": np.zeros((rows, cols // 128), np.uint8) if fmt.macro_cols else None,
        "tensor_scale": np.zeros(1, np.float32) if fmt.scale == SC_NVFP4 else None,
        "ref_exp": np.zeros(1, np.int32) if fmt.scale == SC_E3M0 else None,
    }
    del nsc
    qt = _QT(_ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["offsets"]),
             _ptr(out["macro_scales"]), _ptr(out["tensor_scale"]), _ptr(out["ref_exp"]),
             rows, cols)
    dq = np.zeros((rows, cols), np.float32 if dq_dtype == F32 else np.uint16)
    st = _Stats()
    f = fmt._c()
    rc = lib().ref_quantize(ctypes.byref(f), in_dtype, _ptr(x), rows, cols, cols,
                            ctypes.byref(qt), _ptr(dq), dq_dtype, ctypes.byref(st))
    if rc != 0:
        raise ValueError(f"ref_quantize failed with status {rc}")
    out["dequant"] = dq
    out["stats"] = stats_dict(st)
    return out


def dequantize(fmt: Format, q: dict, rows, cols, out_dtype=F32):
    qt = _QT(_ptr(q["codes"]), _ptr(q["scales"]), _ptr(q.get("offsets")),
             _ptr(q.get("macro_scales")), _ptr(q.get("tensor_scale")),
             _ptr(q.get("ref_exp")), rows, cols)
    y = np.zeros((rows, cols), np.float32 if out_dtype == F32 else np.uint16)
    f = fmt._c()
    rc = lib().ref_dequantize(ctypes.byref(f), ctypes.byref(qt), out_dtype, _ptr(y), cols)
    if rc != 0:
        raise ValueError(f"ref_dequantize failed with status {rc}")
    return y


def stats_dict(st):
    return {"sig2": st.sig2, "err2": st.err2, "n": st.n, "nonzero": st.nonzero,
            "flushed": st.flushed, "zero_blocks": st.zero_blocks}


def qsnr_db(stats):
    """QSNR of eq. (1) of "Unveiling the Potential of Quantization with MXFP4"
    (Sec. 3) from the two squared Frobenius norms."""
    if stats["err2"] == 0:
        return float("inf")
    return 10.0 * np.log10(stats["sig2"] / stats["err2"])


def qsnr(ref, approx):
    ref = np.ascontiguousarray(ref)
    approx = np.ascontiguousarray(approx)
    dtype = BF16 if ref.dtype == np.uint16 else F32
    assert approx.dtype == ref.dtype and approx.size == ref.size
    st = _Stats()
    d = ctypes.c_double()
    rc = lib().ref_qsnr(dtype, _ptr(ref), _ptr(approx), ref.size, ctypes.byref(st), ctypes.byref(d))
    if rc != 0:
        raise ValueError(f"ref_qsnr failed with status {rc}")
    return stats_dict(st), d.value


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, np.uint32)
    k = np.asarray(key, np.uint32)
    o = np.zeros(4, np.uint32)
    lib().ref_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return [int(v) for v in o]


def r16(seed, offset, idx):
    return int(lib().ref_r16(seed, offset, idx))


def round_code(elem, asym, mode, v, r=0):
    return int(lib().ref_round_code(elem, asym, mode, float(np.float32(v)), r))


def code_value(elem, asym, code):
    return float(lib().ref_code_value(elem, asym, code))


def fp8_scale_code(kind, t):
    return int(lib().ref_fp8_scale_code(kind, float(np.float32(t))))


def fp8_scale_value(kind, code):
    return float(lib().ref_fp8_scale_value(kind, code))


def e8m0_exponent(rule, tau, elem, asym, amax):
    return int(lib().ref_e8m0_exponent(rule, float(np.float32(tau)), elem, asym,
                                       float(np.float32(amax))))


def hadamard_const(h):
    return float(lib().ref_hadamard_const(h))


def hadamard_rows(x, h):
    """Rotate every contiguous chunk of h values of a float32 array in place."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    flat = y.reshape(-1, h)
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        lib().ref_hadamard_row(h, _ptr(row))
        flat[i] = row
    return y


def bf16_bits_to_f32(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def gemm_f64(deq_a, deq_b):
    """C = A . B^T of two dequantized operands (each row-major, K contiguous),
    accumulated in float64: the plain definition of the block-scaled product
    once each block's scale has been applied to its elements."""
    return np.asarray(deq_a, np.float64) @ np.asarray(deq_b, np.float64).T


def gemm_f64_sampled(deq_a, deq_b, m_idx, n_idx):
    """C[m, n] for listed (m, n) pairs, one float64 dot product each."""
    a = np.asarray(deq_a[m_idx], np.float64)
    b = np.asarray(deq_b[n_idx], np.float64)
    return np.einsum("ik,ik->i", a, b)


def f32_to_bf16_bits(x):
    """Round fp32 values to the nearest bf16 (ties to even); NaN kept quiet."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r
