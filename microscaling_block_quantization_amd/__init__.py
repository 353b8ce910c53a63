"""Python binding of libmx.so, the gfx950 microscaling block-quantization library.

Argument marshalling only: the functions below take torch tensors (device
memory and streams come from PyTorch), pass raw pointers through the C ABI of
``include/mx.h`` and return.  Every step of quantization, dequantization, the
QSNR reduction and the block-scaled GEMM runs in the library's HIP kernels.
There is no fallback: if ``libmx.so`` is missing or fails to load, importing
the entry points raises.

The method (cited by page title and section): MXFP4 = E2M1 elements + one
E8M0 scale per 32; NVFP4 = E2M1 + E4M3 per 16 + an fp32 per-tensor scale
("Unveiling the Potential of Quantization with MXFP4", Sec. 2); QSNR eq. (1),
(2) (same page, Sec. 3); OAS and Macro Block Scaling (Sec. 4); UE5M3 scales
("Is Finer Better?", technical summary); block Hadamard rotation ("Bridging
the Gap ... Microscaling FP4 Quantization", Sec. 2.2); INT4 / E3M0 elements,
RTNE / stochastic / ceil rounding, asymmetric scaling and row / column / 2D
blocks (ARITH 2025 MX-training report, main results).
"""
import ctypes
import os
from dataclasses import dataclass, field

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmx.so")

MX_OK, MX_ERR_ARG, MX_ERR_UNSUPPORTED, MX_ERR_ALIGN, MX_ERR_WORKSPACE, MX_ERR_HIP, MX_ERR_TOO_LARGE = range(7)
NOALLOC_SCRATCH_BYTES = 4 << 20      # MX_NOALLOC_SCRATCH_BYTES of include/mx.h
ELEM_E2M1, ELEM_INT4, ELEM_FP6_E2M3, ELEM_FP6_E3M2, ELEM_E3M0, ELEM_FP8_E4M3, ELEM_FP8_E5M2 = range(7)
SCALE_E8M0, SCALE_UE4M3, SCALE_NVFP4, SCALE_UE5M3, SCALE_E3M0 = range(5)
RULE_FLOOR, RULE_CEIL, RULE_OAS = range(3)
ROUND_RTNE, ROUND_SR, ROUND_CEIL = range(3)
DTYPE_F32, DTYPE_BF16 = range(2)

EXPORTS = ["mx_query_sizes", "mx_quantize", "mx_quantize_noalloc", "mx_quantize_many", "mx_dequantize",
           "mx_qsnr_workspace_size", "mx_qsnr", "mx_gemm", "mx_status_string"]


class MxFormat(ctypes.Structure):
    _fields_ = [("elem", ctypes.c_int32), ("scale", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("round", ctypes.c_int32), ("block_rows", ctypes.c_int32),
                ("block_cols", ctypes.c_int32), ("asymmetric", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("macro_cols", ctypes.c_int32),
                ("oas_tau", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("rng_offset", ctypes.c_uint64)]


class MxQTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("macro_scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("ref_exp", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class MxStats(ctypes.Structure):
    _fields_ = [("sig2", ctypes.c_double), ("err2", ctypes.c_double), ("n", ctypes.c_int64),
                ("nonzero", ctypes.c_int64), ("flushed", ctypes.c_int64),
                ("zero_blocks", ctypes.c_int64)]


class MxQJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("out", ctypes.POINTER(MxQTensor)), ("stats", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


class MxSizes(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_size_t), ("scales", ctypes.c_size_t),
                ("offsets", ctypes.c_size_t), ("macro_scales", ctypes.c_size_t),
                ("tensor_scale", ctypes.c_size_t), ("ref_exp", ctypes.c_size_t),
                ("workspace", ctypes.c_size_t)]


class MxError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {mx_status_string(status)} (status {status})")


_lib = None


def lib():
    """Load libmx.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "python microscaling_block_quantization_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        P = ctypes.POINTER
        L.mx_query_sizes.argtypes = [P(MxFormat), i64, i64, P(MxSizes)]
        L.mx_quantize.argtypes = [P(MxFormat), i32, vp, i64, i64, i64, P(MxQTensor), vp, i32, vp,
                                  vp, ctypes.c_size_t, vp]
        L.mx_quantize_noalloc.argtypes = [P(MxFormat), i32, vp, i64, i64, i64, P(MxQTensor), vp, i32, vp, vp]
        L.mx_quantize_many.argtypes = [P(MxFormat), i32, P(MxQJob), i32, vp]
        L.mx_dequantize.argtypes = [P(MxFormat), P(MxQTensor), i32, vp, i64, vp]
        L.mx_qsnr_workspace_size.argtypes = [i64]
        L.mx_qsnr_workspace_size.restype = ctypes.c_size_t
        L.mx_qsnr.argtypes = [i32, vp, vp, i64, P(MxStats), P(ctypes.c_double), vp,
                              ctypes.c_size_t, vp]
        L.mx_gemm.argtypes = [P(MxFormat), P(MxQTensor), P(MxFormat), P(MxQTensor), vp, i64, i32, vp]
        L.mx_status_string.argtypes = [i32]
        L.mx_status_string.restype = ctypes.c_char_p
        for name in ("mx_query_sizes", "mx_quantize", "mx_quantize_noalloc", "mx_quantize_many",
                     "mx_dequantize", "mx_qsnr", "mx_gemm"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def mx_status_string(status):
    return lib().mx_status_string(int(status)).decode()


@dataclass
class Format:
    elem: int = ELEM_E2M1
    scale: int = SCALE_E8M0
    rule: int = RULE_FLOOR
    round: int = ROUND_RTNE
    block_rows: int = 1
    block_cols: int = 32
    asymmetric: int = 0
    hadamard: int = 0
    macro_cols: int = 0
    oas_tau: float = 0.0
    seed: int = 0
    rng_offset: int = 0

    def c(self):
        return MxFormat(self.elem, self.scale, self.rule, self.round, self.block_rows,
                        self.block_cols, self.asymmetric, self.hadamard, self.macro_cols,
                        self.oas_tau, self.seed, self.rng_offset)


MXFP4 = Format()
MXFP6_E2M3 = Format(elem=ELEM_FP6_E2M3)
MXFP6_E3M2 = Format(elem=ELEM_FP6_E3M2)
MXFP8_E4M3 = Format(elem=ELEM_FP8_E4M3)
MXFP8_E5M2 = Format(elem=ELEM_FP8_E5M2)


@dataclass
class QTensor:
    """A quantized tensor: device buffers laid out as include/mx.h describes."""
    rows: int
    cols: int
    codes: torch.Tensor
    scales: torch.Tensor
    offsets: torch.Tensor = None
    macro_scales: torch.Tensor = None
    tensor_scale: torch.Tensor = None
    ref_exp: torch.Tensor = None
    _keep: list = field(default_factory=list)

    def c(self):
        p = lambda t: None if t is None else t.data_ptr()
        return MxQTensor(p(self.codes), p(self.scales), p(self.offsets), p(self.macro_scales),
                         p(self.tensor_scale), p(self.ref_exp), self.rows, self.cols)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, where):
    if rc != MX_OK:
        raise MxError(rc, where)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _empty(nbytes, device):
    # 16-byte aligned: the caching allocator hands out 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def mx_query_sizes(fmt: Format, rows, cols):
    s = MxSizes()
    f = fmt.c()
    _check(lib().mx_query_sizes(ctypes.byref(f), rows, cols, ctypes.byref(s)), "mx_query_sizes")
    return {k: getattr(s, k) for k, _ in MxSizes._fields_}


def alloc_qtensor(fmt: Format, rows, cols, device="cuda"):
    s = mx_query_sizes(fmt, rows, cols)
    q = QTensor(rows, cols, _empty(s["codes"], device), _empty(s["scales"], device))
    if s["offsets"]:
        q.offsets = torch.empty(s["offsets"] // 2, dtype=torch.int16, device=device)
    if s["macro_scales"]:
        q.macro_scales = _empty(s["macro_scales"], device)
    if s["tensor_scale"]:
        q.tensor_scale = torch.empty(1, dtype=torch.float32, device=device)
    if s["ref_exp"]:
        q.ref_exp = torch.empty(1, dtype=torch.int32, device=device)
    return q


def alloc_workspace(fmt: Format, rows, cols, device="cuda"):
    return _empty(mx_query_sizes(fmt, rows, cols)["workspace"], device)


def stats_to_dict(t):
    """Read a device mx_stats (48 bytes) into a dict."""
    raw = t.detach().to("cpu").numpy().tobytes()[:ctypes.sizeof(MxStats)]
    st = MxStats.from_buffer_copy(raw)
    return {k: getattr(st, k) for k, _ in MxStats._fields_}


def mx_quantize(fmt: Format, x: torch.Tensor, out: QTensor = None, dequant=None, stats=None,
                workspace=None, stream=None):
    """Quantize a 2-D fp32 / bf16 device tensor.

    dequant: None, a dtype (torch.float32 / torch.bfloat16) to allocate, or a tensor.
    stats: None, True (allocate), or a 48-byte device uint8 tensor.
    Returns (qtensor, dequant tensor or None, stats tensor or None)."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    assert x.stride(1) == 1
    if out is None:
        out = alloc_qtensor(fmt, rows, cols, x.device)
    if isinstance(dequant, torch.dtype):
        dequant = torch.empty((rows, cols), dtype=dequant, device=x.device)
    if stats is True:
        stats = _empty(ctypes.sizeof(MxStats), x.device)
    need_ws = stats is not None or fmt.scale in (SCALE_NVFP4, SCALE_E3M0)
    if workspace is None and need_ws:
        workspace = alloc_workspace(fmt, rows, cols, x.device)
    f = fmt.c()
    q = out.c()
    rc = lib().mx_quantize(ctypes.byref(f), _dtype_code(x), _ptr(x), rows, cols, ld, ctypes.byref(q),
                           _ptr(dequant), DTYPE_F32 if dequant is None else _dtype_code(dequant),
                           _ptr(stats), _ptr(workspace),
                           0 if workspace is None else workspace.numel(), _stream(stream))
    _check(rc, "mx_quantize")
    return out, dequant, stats


def mx_quantize_noalloc(fmt: Format, x: torch.Tensor, out: QTensor, dequant=None, stats=None, stream=None):
    """mx_quantize without a workspace: the library's static scratch array on
    this GPU holds what its kernels need beyond the outputs (at most
    NOALLOC_SCRATCH_BYTES; larger calls raise MxError MX_ERR_TOO_LARGE).  The
    outputs are the caller's: `out` (a QTensor), `dequant` (None or a tensor)
    and `stats` (None or a 48-byte device tensor).  Calls that overlap on one
    GPU share the array and race."""
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    f = fmt.c()
    q = out.c()
    rc = lib().mx_quantize_noalloc(ctypes.byref(f), _dtype_code(x), _ptr(x), rows, cols, ld, ctypes.byref(q),
                                   _ptr(dequant), DTYPE_F32 if dequant is None else _dtype_code(dequant),
                                   _ptr(stats), _stream(stream))
    _check(rc, "mx_quantize_noalloc")
    return out, dequant, stats


def mx_quantize_many(fmt: Format, xs, outs=None, stats=None, workspaces=None, stream=None):
    """Quantize several 2-D device tensors of one dtype in one format (one
    call of mx_quantize_many).  outs: None or a list of QTensors; stats: None,
    True (allocate one per tensor) or a list of 48-byte device tensors (or
    None entries); workspaces: None (allocated where needed) or a list.
    Returns (list of qtensors, list of stats tensors or None)."""
    xs = list(xs)
    n = len(xs)
    outs = [None] * n if outs is None else list(outs)
    if stats is True:
        stats = [_empty(ctypes.sizeof(MxStats), x.device) for x in xs]
    stats = [None] * n if stats is None else list(stats)
    workspaces = [None] * n if workspaces is None else list(workspaces)
    assert len(outs) == n and len(stats) == n and len(workspaces) == n
    dt = _dtype_code(xs[0]) if n else DTYPE_BF16
    keep = []
    jobs = (MxQJob * max(n, 1))()
    for i, x in enumerate(xs):
        assert x.dim() == 2 and x.is_cuda and _dtype_code(x) == dt
        assert x.numel() == 0 or x.stride(1) == 1
        rows, cols = x.shape
        if outs[i] is None:
            outs[i] = alloc_qtensor(fmt, rows, cols, x.device)
        if workspaces[i] is None and (stats[i] is not None or fmt.scale in (SCALE_NVFP4, SCALE_E3M0)):
            workspaces[i] = alloc_workspace(fmt, rows, cols, x.device)
        q = outs[i].c()
        keep.append(q)
        ws = workspaces[i]
        jobs[i] = MxQJob(x.data_ptr(), rows, cols, x.stride(0) if rows > 1 and x.numel() else cols,
                         ctypes.pointer(q),
                         None if stats[i] is None else stats[i].data_ptr(),
                         None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel())
    f = fmt.c()
    rc = lib().mx_quantize_many(ctypes.byref(f), dt, jobs, n, _stream(stream))
    _check(rc, "mx_quantize_many")
    return outs, stats


def mx_dequantize(fmt: Format, q: QTensor, out_dtype=torch.float32, y=None, stream=None):
    if y is None:
        y = torch.empty((q.rows, q.cols), dtype=out_dtype, device=q.codes.device)
    f = fmt.c()
    qc = q.c()
    ld = y.stride(0) if q.rows > 1 else q.cols
    rc = lib().mx_dequantize(ctypes.byref(f), ctypes.byref(qc), _dtype_code(y), _ptr(y), ld, _stream(stream))
    _check(rc, "mx_dequantize")
    return y


def mx_qsnr_workspace_size(n):
    return int(lib().mx_qsnr_workspace_size(int(n)))


def mx_qsnr(ref: torch.Tensor, approx: torch.Tensor, workspace=None, stream=None):
    """QSNR (dB) of eq. (1)/(2) between two device tensors; returns (stats, dB)."""
    assert ref.dtype == approx.dtype and ref.numel() == approx.numel()
    assert ref.is_contiguous() and approx.is_contiguous()
    n = ref.numel()
    if workspace is None:
        workspace = _empty(mx_qsnr_workspace_size(n), ref.device)
    st = MxStats()
    d = ctypes.c_double()
    rc = lib().mx_qsnr(_dtype_code(ref), _ptr(ref), _ptr(approx), n, ctypes.byref(st), ctypes.byref(d),
                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "mx_qsnr")
    return {k: getattr(st, k) for k, _ in MxStats._fields_}, d.value


def mx_gemm(fa: Format, a: QTensor, fb: Format, b: QTensor, c=None, out_dtype=torch.bfloat16, stream=None):
    """C = deq(A) . deq(B)^T for A (M x K) and B (N x K): MXFP4, MXFP6 (E2M3 /
    E3M2) or MXFP8 (E4M3 / E5M2) with E8M0 scales per 1 x 32 block, in any pairing (MXFP4 operands may
    carry 1 x 128 macro-block scales, macro_cols=128); or E2M1 under UE4M3,
    NVFP4, UE5M3 or E8M0 scales on other row blocks.  c: an M x N view (any
    row stride) to write into, else a new tensor of out_dtype."""
    if c is None:
        c = torch.empty((a.rows, b.rows), dtype=out_dtype, device=a.codes.device)
    ldc = c.stride(0) if a.rows > 1 else b.rows
    f1, f2 = fa.c(), fb.c()
    qa, qb = a.c(), b.c()
    rc = lib().mx_gemm(ctypes.byref(f1), ctypes.byref(qa), ctypes.byref(f2), ctypes.byref(qb), _ptr(c), ldc,
                       _dtype_code(c), _stream(stream))
    _check(rc, "mx_gemm")
    return c
