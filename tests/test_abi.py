"""The C-ABI library loads, exports every entry point include/mx.h declares, and
its host-side logic (validation, size queries, status strings) behaves as the
header documents.  No kernel is launched: every call here is rejected before
the first launch, or is a pure size query."""
import ctypes
import os
import re

import pytest

import microscaling_block_quantization_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mx_quantize", "mx_dequantize", "mx_qsnr", "mx_gemm", "mx_query_sizes"):
        assert n in names
    assert set(names) == set(mx.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = mx.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    nm = os.popen(f"nm -D --defined-only {mx.LIB_PATH}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}\b", nm), n


def test_struct_layouts_match_header():
    assert ctypes.sizeof(mx.MxFormat) == 56
    assert mx.MxFormat.seed.offset == 40
    assert ctypes.sizeof(mx.MxQTensor) == 64
    assert ctypes.sizeof(mx.MxStats) == 48
    assert ctypes.sizeof(mx.MxSizes) == 56
    assert ctypes.sizeof(mx.MxQJob) == 64


def test_status_strings():
    assert mx.mx_status_string(mx.MX_OK) == "ok"
    for s in range(1, 7):
        assert mx.mx_status_string(s) != "unknown status"
    assert mx.mx_status_string(99) == "unknown status"


def sizes(**kw):
    return mx.mx_query_sizes(mx.Format(**kw), kw.pop("_rows", 64), 256)


def test_query_sizes_mxfp4_and_nvfp4():
    s = mx.mx_query_sizes(mx.Format(), 64, 256)
    assert s["codes"] == 64 * 128 and s["scales"] == 64 * 8
    assert s["offsets"] == 0 and s["tensor_scale"] == 0 and s["workspace"] > 0
    # 4 + 8/b bits per element ("Unveiling ... MXFP4", Sec. 3)
    assert 8 * (s["codes"] + s["scales"]) / (64 * 256) == 4.25
    s = mx.mx_query_sizes(mx.Format(scale=mx.SCALE_NVFP4, block_cols=16), 64, 256)
    assert 8 * (s["codes"] + s["scales"]) / (64 * 256) == 4.5 and s["tensor_scale"] == 4
    s = mx.mx_query_sizes(mx.Format(elem=mx.ELEM_FP6_E2M3), 64, 256)
    assert s["codes"] == 64 * 192
    s = mx.mx_query_sizes(mx.Format(elem=mx.ELEM_INT4, asymmetric=1, rule=1), 64, 256)
    assert s["offsets"] == 2 * s["scales"]
    s = mx.mx_query_sizes(mx.Format(macro_cols=128, block_cols=16), 64, 256)
    assert s["macro_scales"] == 64 * 2 and s["scales"] == 64 * 16
    s = mx.mx_query_sizes(mx.Format(block_rows=32, block_cols=32), 64, 256)
    assert s["scales"] == 2 * 8
    s = mx.mx_query_sizes(mx.Format(scale=mx.SCALE_E3M0, rule=1), 64, 256)
    assert s["ref_exp"] == 4


STAT_PART_BYTES = 48          # one statistics partial per workgroup of the quantizer


def _rows_grid(rows, cols):
    """workgroups of the general row kernel: 256 threads of 16 (8 when cols is
    8 mod 16) consecutive elements each"""
    ch = 16 if cols % 16 == 0 else 8
    return -(-rows * (cols // ch) // 256)


def _tiles_grid(rows, cols, br, in_bf16):
    """workgroups of the column / 2D kernel: one per band of br rows and 1 KiB
    of each row (512 bf16 or 256 fp32 columns)"""
    tc = 512 if in_bf16 else 256
    return (rows // br) * -(-cols // tc)


@pytest.mark.parametrize("rows,cols,kw", [
    (8192, 4096, {}), (4096, 14336, {}), (14336, 4096, {}), (256, 1032, dict(block_cols=8)),
    (1024, 1024, dict(block_cols=16)), (8192, 4096, dict(scale=mx.SCALE_NVFP4, block_cols=16)),
    (96, 512, dict(block_rows=32, block_cols=1)), (4096, 14336, dict(block_rows=32, block_cols=32)),
    (4096, 14336, dict(block_rows=8, block_cols=8)),
])
def test_workspace_covers_every_kernel_route(rows, cols, kw):
    """The statistics partials of whichever kernel a call takes fit in the
    queried workspace: a dequant output or a strided input sends MXFP4 to the
    general row kernel, whose grid is not capped like the fast kernel's."""
    s = mx.mx_query_sizes(mx.Format(**kw), rows, cols)
    br = kw.get("block_rows", 1)
    if br == 1:
        need = _rows_grid(rows, cols) * STAT_PART_BYTES
    else:
        need = max(_tiles_grid(rows, cols, br, b) for b in (0, 1)) * STAT_PART_BYTES
    if kw.get("scale") == mx.SCALE_NVFP4:
        need += _rows_grid(rows, cols) * 4       # the tensor pre-pass maxima
    assert s["workspace"] >= need


@pytest.mark.parametrize("kw,status", [
    (dict(elem=7), mx.MX_ERR_ARG),
    (dict(block_cols=24), mx.MX_ERR_ARG),
    (dict(block_cols=4), mx.MX_ERR_UNSUPPORTED),
    (dict(block_rows=64, block_cols=1), mx.MX_ERR_UNSUPPORTED),
    (dict(block_rows=16, block_cols=8), mx.MX_ERR_UNSUPPORTED),
    (dict(rule=2, oas_tau=5.0), mx.MX_ERR_ARG),
    (dict(rule=2, oas_tau=12.0), mx.MX_ERR_ARG),
    (dict(hadamard=8), mx.MX_ERR_UNSUPPORTED),
    (dict(hadamard=32, block_rows=32, block_cols=1), mx.MX_ERR_UNSUPPORTED),
    (dict(macro_cols=64), mx.MX_ERR_ARG),
    (dict(macro_cols=128, scale=1), mx.MX_ERR_UNSUPPORTED),
    (dict(asymmetric=1, scale=2), mx.MX_ERR_UNSUPPORTED),
    (dict(asymmetric=1, elem=2), mx.MX_ERR_UNSUPPORTED),
    (dict(asymmetric=2), mx.MX_ERR_ARG),
])
def test_query_rejects_bad_formats(kw, status):
    with pytest.raises(mx.MxError) as e:
        mx.mx_query_sizes(mx.Format(**kw), 64, 256)
    assert e.value.status == status


def test_shape_rules():
    with pytest.raises(mx.MxError):
        mx.mx_query_sizes(mx.Format(), 64, 100)          # cols not a multiple of the block
    with pytest.raises(mx.MxError):
        mx.mx_query_sizes(mx.Format(block_rows=32, block_cols=1), 40, 256)
    with pytest.raises(mx.MxError):
        mx.mx_query_sizes(mx.Format(), -1, 256)
    s = mx.mx_query_sizes(mx.Format(), 0, 256)          # empty tensors are valid
    assert s["codes"] == 0 and s["scales"] == 0


def _call_quantize(fmt, x=1024, codes=2048, scales=4096, rows=4, cols=64, ld=64, ws=None, wsb=0,
                   stats=None, dtype=mx.DTYPE_F32):
    q = mx.MxQTensor(codes, scales, None, None, None, None, rows, cols)
    f = fmt.c()
    return mx.lib().mx_quantize(ctypes.byref(f), dtype, x, rows, cols, ld, ctypes.byref(q), None,
                                mx.DTYPE_F32, stats, ws, wsb, None)


def test_quantize_rejects_before_launch():
    # fake (never dereferenced) addresses: every call below fails validation
    assert _call_quantize(mx.Format(), x=None) == mx.MX_ERR_ARG
    assert _call_quantize(mx.Format(), ld=32) == mx.MX_ERR_ARG
    assert _call_quantize(mx.Format(), x=1032) == mx.MX_ERR_ALIGN
    assert _call_quantize(mx.Format(), ld=66) == mx.MX_ERR_ALIGN
    assert _call_quantize(mx.Format(), dtype=5) == mx.MX_ERR_ARG
    assert _call_quantize(mx.Format(), stats=4096, ws=None) == mx.MX_ERR_WORKSPACE
    assert _call_quantize(mx.Format(), stats=4096, ws=8192, wsb=16) == mx.MX_ERR_WORKSPACE
    assert _call_quantize(mx.Format(scale=mx.SCALE_NVFP4, block_cols=16)) == mx.MX_ERR_ARG  # no tensor_scale


def test_gemm_rejects_before_launch():
    f = mx.Format().c()
    bad = mx.Format(elem=mx.ELEM_INT4).c()
    a = mx.MxQTensor(1024, 2048, None, None, None, None, 64, 256)
    b = mx.MxQTensor(4096, 8192, None, None, None, None, 32, 256)
    b_k = mx.MxQTensor(4096, 8192, None, None, None, None, 32, 512)
    b_k80 = mx.MxQTensor(4096, 8192, None, None, None, None, 32, 80)
    L = mx.lib()
    assert L.mx_gemm(ctypes.byref(bad), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_UNSUPPORTED
    assert L.mx_gemm(ctypes.byref(f), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b_k), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ARG
    assert L.mx_gemm(ctypes.byref(f), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 16,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ARG
    # K = 80 breaks the 1 x 32 block shape of the operands themselves
    assert L.mx_gemm(ctypes.byref(f), ctypes.byref(b_k80), ctypes.byref(f), ctypes.byref(b_k80), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ARG
    assert L.mx_gemm(ctypes.byref(f), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10008, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ALIGN
    # element types outside E2M1 / E2M3 / E3M2, and non-E8M0 scales, are not run
    for e in (mx.ELEM_INT4, mx.ELEM_E3M0):
        g = mx.Format(elem=e).c()
        assert L.mx_gemm(ctypes.byref(g), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 32,
                         mx.DTYPE_BF16, None) == mx.MX_ERR_UNSUPPORTED
    nv = mx.Format(elem=mx.ELEM_E3M0, scale=mx.SCALE_UE5M3).c()
    assert L.mx_gemm(ctypes.byref(f), ctypes.byref(a), ctypes.byref(nv), ctypes.byref(b), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_UNSUPPORTED
    # macro-block scales: MXFP4 only, and the macro_scales buffer is required
    g6m = mx.Format(elem=mx.ELEM_FP6_E2M3, macro_cols=128).c()
    assert L.mx_gemm(ctypes.byref(g6m), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_UNSUPPORTED
    fm = mx.Format(macro_cols=128).c()
    assert L.mx_gemm(ctypes.byref(fm), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ARG
    am = mx.MxQTensor(1024, 2048, None, 4096, None, None, 64, 256)
    assert L.mx_gemm(ctypes.byref(fm), ctypes.byref(am), ctypes.byref(f), ctypes.byref(b), 0x10008, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ALIGN
    # macro scales over 1 x 16 E8M0 sub-blocks (the decode route): against fp8
    # block scales not run; without the macro buffer an argument error;
    # otherwise through validation (misaligned C, so no launch)
    fm16 = mx.Format(macro_cols=128, block_cols=16).c()
    a16 = mx.MxQTensor(1024, 2048, None, None, None, None, 64, 256)
    b16 = mx.MxQTensor(4096, 8192, None, 12288, None, None, 32, 256)
    a16m = mx.MxQTensor(1024, 2048, None, 4096, None, None, 64, 256)
    nv16 = mx.Format(scale=mx.SCALE_UE4M3, block_cols=16).c()
    assert L.mx_gemm(ctypes.byref(fm16), ctypes.byref(a16m), ctypes.byref(nv16), ctypes.byref(b16), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_UNSUPPORTED
    assert L.mx_gemm(ctypes.byref(fm16), ctypes.byref(a16), ctypes.byref(fm16), ctypes.byref(b16), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ARG
    assert L.mx_gemm(ctypes.byref(fm16), ctypes.byref(a16m), ctypes.byref(fm16), ctypes.byref(b16), 0x10008, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ALIGN
    # FP6 elements need E8M0 scales on 1 x 32 blocks; NVFP4 needs its tensor scale
    g6u = mx.Format(elem=mx.ELEM_FP6_E2M3, scale=mx.SCALE_UE4M3, block_cols=16).c()
    assert L.mx_gemm(ctypes.byref(g6u), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_UNSUPPORTED
    nvf = mx.Format(scale=mx.SCALE_NVFP4, block_cols=16).c()
    assert L.mx_gemm(ctypes.byref(nvf), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10000, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ARG
    a_t = mx.MxQTensor(1024, 2048, None, None, 8192, None, 64, 256)
    assert L.mx_gemm(ctypes.byref(nvf), ctypes.byref(a_t), ctypes.byref(f), ctypes.byref(b), 0x10008, 32,
                     mx.DTYPE_BF16, None) == mx.MX_ERR_ALIGN
    # FP6 operands pass validation (checked here with a misaligned C, so no launch)
    for e in (mx.ELEM_FP6_E2M3, mx.ELEM_FP6_E3M2):
        g = mx.Format(elem=e).c()
        assert L.mx_gemm(ctypes.byref(g), ctypes.byref(a), ctypes.byref(f), ctypes.byref(b), 0x10008, 32,
                         mx.DTYPE_BF16, None) == mx.MX_ERR_ALIGN


def test_qsnr_rejects_before_launch():
    L = mx.lib()
    d = ctypes.c_double()
    assert L.mx_qsnr(mx.DTYPE_F32, 1024, 2048, 0, None, ctypes.byref(d), 4096, 1 << 20, None) == mx.MX_ERR_ARG
    assert L.mx_qsnr(mx.DTYPE_F32, 1024, 2048, 100, None, ctypes.byref(d), None, 0, None) == mx.MX_ERR_WORKSPACE
    assert L.mx_qsnr(mx.DTYPE_F32, 1028, 2048, 100, None, ctypes.byref(d), 4096, 1 << 20, None) == mx.MX_ERR_ALIGN
    assert mx.mx_qsnr_workspace_size(100) > 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it says so and exits with 2
    before touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU only" in out["error"]


def test_noalloc_rejects_before_launch():
    """The no-allocation entry point checks its arguments like mx_quantize, and
    refuses (before any HIP call) a tensor whose workspace would not fit its
    static scratch array; a call that needs no workspace has no size limit."""
    L = mx.lib()

    def call(fmt, rows, cols, stats=None, x=1024):
        q = mx.MxQTensor(2048, 4096, None, None, 8192, None, rows, cols)
        f = fmt.c()
        return L.mx_quantize_noalloc(ctypes.byref(f), mx.DTYPE_BF16, x, rows, cols, cols, ctypes.byref(q), None,
                                     mx.DTYPE_F32, stats, None)

    assert call(mx.Format(), 4, 64, x=None) == mx.MX_ERR_ARG
    assert call(mx.Format(), 4, 64, x=1032) == mx.MX_ERR_ALIGN
    assert call(mx.Format(block_cols=24), 4, 96) == mx.MX_ERR_ARG
    big = (1 << 15, 1 << 15)                       # 2^30 elements: workspace far above 4 MiB
    assert mx.mx_query_sizes(mx.MXFP4, *big)["workspace"] > mx.NOALLOC_SCRATCH_BYTES
    assert call(mx.MXFP4, *big, stats=4096) == mx.MX_ERR_TOO_LARGE
    assert call(mx.Format(scale=mx.SCALE_NVFP4, block_cols=16), *big) == mx.MX_ERR_TOO_LARGE
    # the largest configured tensors fit
    for rows, cols, kw in ((16384, 4096, {}), (4096, 14336, dict(block_rows=8, block_cols=8)),
                           (16384, 4096, dict(scale=mx.SCALE_NVFP4, block_cols=16))):
        assert mx.mx_query_sizes(mx.Format(**kw), rows, cols)["workspace"] <= mx.NOALLOC_SCRATCH_BYTES


def test_quantize_many_rejects_before_launch():
    """mx_quantize_many checks every job before its first launch: a bad count
    or job array, the first failing job's own status (even after valid jobs,
    which would otherwise have been launched and, with no GPU, reported
    MX_ERR_HIP), and two jobs whose workspaces overlap."""
    L = mx.lib()
    f = mx.MXFP4.c()
    rows, cols = 64, 256
    ws = mx.mx_query_sizes(mx.MXFP4, rows, cols)["workspace"]
    qt = [mx.MxQTensor(0x100000 * (i + 1), 0x100000 * (i + 1) + 0x40000, None, None, None, None, rows, cols)
          for i in range(3)]

    def job(i, x=0x1000, stats=None, wsp=None, wsb=0, r=rows):
        return mx.MxQJob(x, r, cols, cols, ctypes.pointer(qt[i]), stats, wsp, wsb)

    def call(*jobs, count=None, dtype=mx.DTYPE_BF16):
        arr = (mx.MxQJob * max(len(jobs), 1))(*jobs)
        return L.mx_quantize_many(ctypes.byref(f), dtype, arr if jobs else None,
                                  len(jobs) if count is None else count, None)

    assert call(count=0) == mx.MX_OK                      # nothing to do, nothing launched
    assert call(count=0, dtype=7) == mx.MX_ERR_ARG
    assert call(count=-1) == mx.MX_ERR_ARG
    assert call(count=2) == mx.MX_ERR_ARG                 # jobs NULL
    assert call(job(0), job(1, x=None)) == mx.MX_ERR_ARG
    assert call(job(0), job(1, x=0x1008)) == mx.MX_ERR_ALIGN
    assert call(job(0), job(1, r=-1)) == mx.MX_ERR_ARG
    assert call(job(0), job(1, stats=0x9000)) == mx.MX_ERR_WORKSPACE
    assert call(job(0, stats=0x9000, wsp=0x10000, wsb=ws),
                job(1, stats=0x9100, wsp=0x10000 + ws - 256, wsb=ws)) == mx.MX_ERR_ARG
    assert call(job(0, stats=0x9000, wsp=0x10000, wsb=ws), job(1, stats=0x9100, wsp=0x10000, wsb=ws),
                job(2)) == mx.MX_ERR_ARG


def test_ceilings_library_exports_its_header():
    """libmx_ceilings.so (the measurement's context kernels) exports what
    include/mx_ceilings.h declares, and libmx.so exports none of it."""
    from microscaling_block_quantization_amd import ceilings
    src = open(os.path.join(ROOT, "include", "mx_ceilings.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(mxc_[a-z0-9_]+)\s*\(", src)))
    assert names == sorted(ceilings.EXPORTS)
    nm = os.popen(f"nm -D --defined-only {ceilings.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", nm), n
    assert "mxc_" not in os.popen(f"nm -D --defined-only {mx.LIB_PATH}").read()
    L = ceilings.lib()
    assert L.mxc_mfma_loop_flops(256, 10) == 2.0 * 32 * 32 * 64 * 16 * 8 * 256 * 10
    assert L.mxc_copy(None, None, 16, None) == 1 and L.mxc_mfma_loop(None, None, 1, 1, None) == 1


def test_header_sizes_match_the_binding():
    """The sizes include/mx.h states are the ones the Python binding uses."""
    import re
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    defs = {m.group(1): m.group(2) for m in re.finditer(r"#define\s+(MX_\w+)\s+\(?([0-9u<\s]+)\)?", src)}
    assert eval(defs["MX_NOALLOC_SCRATCH_BYTES"].replace("u", "")) == mx.NOALLOC_SCRATCH_BYTES
