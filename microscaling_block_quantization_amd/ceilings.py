"""Binding of libmx_ceilings.so (include/mx_ceilings.h): the context kernels the
benchmark compares the hot path with -- a device copy, a read-mostly stream
with the quantizer's 4:1 byte mix, the FP4 matrix-instruction loop fed from
LDS like the tiled GEMM, and the GEMM's LDS-DMA operand stream on its own.
Argument marshalling only; each function enqueues on the current torch
stream and returns."""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmx_ceilings.so")
EXPORTS = ["mxc_copy", "mxc_read4_write1", "mxc_mfma_loop_grid", "mxc_mfma_loop_flops", "mxc_mfma_loop",
           "mxc_lds_dma"]
LOOP_OPERAND_BYTES = 32768
DMA_STAGE_BYTES = 32768

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "python microscaling_block_quantization_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
        L.mxc_copy.argtypes = [vp, vp, sz, vp]
        L.mxc_read4_write1.argtypes = [vp, vp, sz, vp]
        L.mxc_mfma_loop_grid.argtypes = []
        L.mxc_mfma_loop_flops.argtypes = [i32, i64]
        L.mxc_mfma_loop_flops.restype = ctypes.c_double
        L.mxc_mfma_loop.argtypes = [vp, vp, i32, i64, vp]
        L.mxc_lds_dma.argtypes = [vp, sz, vp, i32, i32, vp]
        for n in ("mxc_copy", "mxc_read4_write1", "mxc_mfma_loop_grid", "mxc_mfma_loop", "mxc_lds_dma"):
            getattr(L, n).restype = i32
        _lib = L
    return _lib


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(rc, where):
    if rc != 0:
        raise RuntimeError(f"{where} failed with status {rc}")


def copy(src, dst):
    _ok(lib().mxc_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), _s()), "mxc_copy")


def read4_write1(src, dst):
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n // 4
    _ok(lib().mxc_read4_write1(src.data_ptr(), dst.data_ptr(), n, _s()), "mxc_read4_write1")


def mfma_loop_grid():
    return int(lib().mxc_mfma_loop_grid())


def mfma_loop_flops(grid, iters):
    return float(lib().mxc_mfma_loop_flops(grid, iters))


def mfma_loop(operands, out, grid, iters):
    assert operands.numel() * operands.element_size() >= LOOP_OPERAND_BYTES
    assert out.numel() >= grid * 512 and out.dtype == torch.float32
    _ok(lib().mxc_mfma_loop(operands.data_ptr(), out.data_ptr(), grid, iters, _s()), "mxc_mfma_loop")


def lds_dma(src, out, grid, stages):
    n = src.numel() * src.element_size()
    assert out.numel() >= grid * 512 and out.element_size() == 4
    _ok(lib().mxc_lds_dma(src.data_ptr(), n, out.data_ptr(), grid, stages, _s()), "mxc_lds_dma")
