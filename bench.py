#!/usr/bin/env python3
"""Benchmark of the microscaling hot path on one MI355X.

One step = one W4A4 linear layer at Llama-8B MLP shape, on synthetic data:
  quantize A (bf16 8192 x 4096 ~ N(0, 1))      -> MXFP4 codes + E8M0 scales + stats
  quantize B (bf16 14336 x 4096 ~ N(0, .02^2)) -> MXFP4 codes + E8M0 scales + stats
    (both in one mx_quantize_many call: one quantize launch, one statistics
    finalize launch)
  C = deq(A) . deq(B)^T on the block-scaled FP4 MFMA, fp32 accumulate, bf16 out
(MXFP4 = 1x32 E2M1 blocks with E8M0 scales, floor rule, round-to-nearest-even).

Timing: W warm-up steps, then K timed steps with HIP events at the phase
boundaries (the quantize phase, then the GEMM), on the stream every call is
enqueued on; 4 input sets (704 MB) rotate so that no step finds its inputs
in the 256 MB Infinity Cache.  Reported: quantizer GB/s (algorithmic bytes:
2 B read + 0.5 B codes + 1/32 B scale per element) over the timed steps as
`value`, GEMM TFLOP/s (2 M N K per product), mean and median of each, their
fractions of the MI355X peaks, QSNR of A, B (eq. (1)) and of the product
(eq. (2)) against the bf16 product, and the CPU oracle timed on this host.

For information, after the timed steps (none of it is part of `value`):
  ceilings         copy bandwidth, the quantizer's 4:1 read/write byte mix,
                   and the FP4 matrix-instruction loop on random and constant
                   operands (libmx_ceilings.so)
  quantize_formats every quantizer cell of the pages' configurations at full
                   size (fp32 1024x1024 MXFP4 with dequant; the bf16 8192x4096
                   NVFP4 / MXFP4 / UE5M3 / UE4M3 block sweep; the bf16
                   4096x14336 gradient formats over 1x32, 32x1, 32x32 blocks;
                   the bf16 16384x4096 activation formats: Hadamard, OAS, MBS,
                   NVFP4; MXFP6 / MXFP8 operands of bf16 8192x4096), each timed
                   alone after an Infinity Cache flush, with its QSNR, MSE,
                   flush and zero-block fractions
  gemm_formats     the step's product in the other block formats
  parity           the step's codes, scales, statistics and 256 rows of its
                   product against the CPU oracle

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                       [--no-formats] [--no-ceilings]
"""
import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

M, N, K = 8192, 14336, 4096
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0        # MI355X dense MXFP4 (and FP6) MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0         # MI355X dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 / fp16 MFMA, TFLOP/s
QUANT_BYTES_PER_ELEM = 2 + 0.5 + 1.0 / 32
FLUSH_BYTES = 512 << 20          # written (and read) between timed cells: evicts the 256 MB Infinity Cache

HERE = os.path.dirname(os.path.abspath(__file__))


def sources_hash(srcs):
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(HERE, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted(name, key):
    """A figure measured with rocprofv3 counters (profiles/<name>.json), or None
    when the kernel's sources changed since it was taken."""
    try:
        with open(os.path.join(HERE, "profiles", name)) as f:
            k = json.load(f)["kernels"][key]
        return k if sources_hash(k["sources"]) == k["sha"] else None
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated to defeat the 256 MB Infinity Cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the other quantizer cells and GEMM formats (not part of the step)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the context ceilings")
    ap.add_argument("--only-gemm-formats", action="store_true",
                    help="only the products in the other block formats (gemm_formats), for a kernel trace")
    ap.add_argument("--only-formats", action="store_true",
                    help="run only the quantizer cells (for profiling them)")
    return ap.parse_args()


def timed(torch, fn, reps, flush=None):
    """median and mean (ms) of `reps` event-timed calls of fn on the current
    stream; flush() (untimed) runs before each call"""
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts), sum(ts) / len(ts)


def ceilings(torch, dev):
    """context ceilings from the tracked context kernels (libmx_ceilings.so)"""
    from microscaling_block_quantization_amd import ceilings as cl
    out = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.random_(0, 256)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    med, _ = timed(torch, lambda: cl.copy(src, dst), 10)
    out["copy"] = {"bytes": 2 * n, "ms": round(med, 4), "gbs": round(2 * n / med / 1e6, 1),
                   "frac_hbm_peak": round(2 * n / med / 1e6 / HBM_PEAK_GBS, 4),
                   "note": "1 GiB read + 1 GiB written, 16-byte non-temporal accesses"}
    med, _ = timed(torch, lambda: cl.read4_write1(src, dst), 10)
    b = n + n // 4
    out["read4_write1"] = {"bytes": b, "ms": round(med, 4), "gbs": round(b / med / 1e6, 1),
                           "frac_hbm_peak": round(b / med / 1e6 / HBM_PEAK_GBS, 4),
                           "note": "1 GiB read, 256 MiB written: the bf16 -> MXFP4 quantizer's byte mix"}
    del src, dst
    grid = cl.mfma_loop_grid()
    iters = 4000
    res = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    ops = torch.empty(cl.LOOP_OPERAND_BYTES, dtype=torch.uint8, device=dev)
    for kind in ("random", "constant"):
        if kind == "random":
            ops.random_(0, 256)
        else:
            ops.fill_(0x5A)
        cl.mfma_loop(ops, res, grid, 100)
        med, _ = timed(torch, lambda: cl.mfma_loop(ops, res, grid, iters), 5)
        tf = cl.mfma_loop_flops(grid, iters) / med / 1e9
        out[f"fp4_mfma_loop_{kind}"] = {
            "ms": round(med, 4), "tflops": round(tf, 1), "frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4),
            "note": f"{grid} workgroups x 8 waves, 4x2 tiles of the 32x32x64 scaled FP4 instruction fed by "
                    f"ds_read_b128 (6 per 8 instructions), {kind} operand bytes"}
    # the GEMM's operand stream alone: as many 32 KiB stages per CU as the step's
    # product moves (7 tiles of 256 x 256 per CU, 32 stages of K = 128 each)
    tiles_per_cu = -(-((M // 256) * (N // 256)) // grid)
    stages = tiles_per_cu * (K // 128)
    src = torch.empty(4 << 20, dtype=torch.uint8, device=dev)
    src.random_(0, 256)
    words = torch.empty(grid * 512, dtype=torch.int32, device=dev)
    cl.lds_dma(src, words, grid, stages)
    med, _ = timed(torch, lambda: cl.lds_dma(src, words, grid, stages), 10)
    byt = grid * stages * cl.DMA_STAGE_BYTES
    out["lds_dma_stream"] = {
        "ms": round(med, 4), "gbs": round(byt / med / 1e6, 1), "gbs_per_cu": round(byt / grid / med / 1e6, 2),
        "note": f"{grid} workgroups x {stages} stages of 32 KiB (512 rows x 64 B) into LDS by buffer_load_dwordx4 ... "
                f"lds, two stages in flight, a barrier per stage: the step's GEMM operand stream without its "
                f"arithmetic, so its time is a floor for that GEMM on this tiling"}
    return out


# ---- the quantizer cells of the pages' configurations -------------------------
def cell_bytes(mx, fmt, rows, cols, in_bytes, dq_bytes=0):
    s = mx.mx_query_sizes(fmt, rows, cols)
    out = s["codes"] + s["scales"] + s["offsets"] + s["macro_scales"] + s["tensor_scale"] + s["ref_exp"]
    return rows * cols * in_bytes + out + dq_bytes


def quantize_formats(mx, torch, np, synth, dev, flush):
    F = mx.Format
    cells = []

    def run(config, name, fmt, x, dq_dtype=None):
        rows, cols = x.shape
        esz = x.element_size()
        q = mx.alloc_qtensor(fmt, rows, cols, dev)
        ws = mx.alloc_workspace(fmt, rows, cols, dev)
        st = torch.empty(48, dtype=torch.uint8, device=dev)
        dq = torch.empty((rows, cols), dtype=dq_dtype, device=dev) if dq_dtype is not None else None
        call = lambda: mx.mx_quantize(fmt, x, out=q, dequant=dq, stats=st, workspace=ws)
        call()
        med, mean = timed(torch, call, 10, flush)
        s = mx.stats_to_dict(st)
        b = cell_bytes(mx, fmt, rows, cols, esz, 0 if dq is None else dq.numel() * dq.element_size())
        nblk = (rows // fmt.block_rows) * (cols // fmt.block_cols)
        c = {"config": config, "format": name, "shape": [rows, cols], "us": round(med * 1e3, 2),
             "gbs": round(b / med / 1e6, 1), "frac_hbm_peak": round(b / med / 1e6 / HBM_PEAK_GBS, 4),
             "bytes": b,
             "qsnr_db": round(10 * math.log10(s["sig2"] / s["err2"]), 4) if s["err2"] > 0 else None,
             "mse": s["err2"] / s["n"],
             "flush_frac": round(s["flushed"] / max(s["nonzero"], 1), 6),
             "zero_block_frac": round(s["zero_blocks"] / nblk, 6)}
        if fmt.scale in (mx.SCALE_NVFP4, mx.SCALE_E3M0):
            c["prepass_read_bytes"] = rows * cols * esz
            c["gbs_with_prepass_read"] = round((b + rows * cols * esz) / med / 1e6, 1)
        cells.append(c)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # c1: fp32 1024 x 1024 N(0, 0.02^2), MXFP4 with the fp32 dequantized tensor
    x = up(synth.w1())
    run("fp32 1024x1024 N(0,0.02^2)", "MXFP4 1x32 + fp32 dequant", mx.MXFP4, x, torch.float32)
    # c2: bf16 8192 x 4096 N(0, sigma^2), block-size sweep of four scale formats
    for sigma in (1e-3, 2e-2):
        x = up(synth.w2(sigma))
        for sname, sc in (("MXFP4 (E8M0)", mx.SCALE_E8M0), ("NVFP4 (UE4M3 + fp32)", mx.SCALE_NVFP4),
                          ("UE5M3", mx.SCALE_UE5M3), ("UE4M3 (no tensor scale)", mx.SCALE_UE4M3)):
            for b in (8, 16, 32, 64, 128, 256):
                run(f"bf16 8192x4096 N(0,{sigma}^2)", f"{sname} 1x{b}", F(scale=sc, block_cols=b), x)
        del x
    # c3: bf16 4096 x 14336 gradients, Laplace(0, 1e-4) + 0.1% x50
    x = up(synth.w3())
    for shape, (br, bc) in (("1x32", (1, 32)), ("32x1", (32, 1)), ("32x32", (32, 32))):
        run("bf16 4096x14336 gradient", f"E2M1 SR (Philox) E8M0 {shape}",
            F(round=mx.ROUND_SR, seed=synth.SR_SEED, block_rows=br, block_cols=bc), x)
        run("bf16 4096x14336 gradient", f"E2M1 E3M0-scale ceil {shape}",
            F(scale=mx.SCALE_E3M0, rule=mx.RULE_CEIL, block_rows=br, block_cols=bc), x)
        run("bf16 4096x14336 gradient", f"INT4 asymmetric min/max {shape}",
            F(elem=mx.ELEM_INT4, asymmetric=1, rule=mx.RULE_CEIL, block_rows=br, block_cols=bc), x)
    del x
    # c4: bf16 16384 x 4096 activations, Laplace(0, 1) + 8 channels x100
    x = up(synth.w4())
    act = [("MXFP4 1x32", F()), ("H32 -> MXFP4", F(hadamard=32)), ("H128 -> MXFP4", F(hadamard=128))]
    for tau in (6.0, 7.0, 7.5, 8.0):
        for b in (32, 16):
            act.append((f"MXFP4 OAS tau={tau} 1x{b}", F(rule=mx.RULE_OAS, oas_tau=tau, block_cols=b)))
    act += [("MBS 1x128 UE4M3 / 1x16 E8M0 (ceil)", F(macro_cols=128, block_cols=16, rule=mx.RULE_CEIL)),
            ("MBS + OAS tau=7.5 (1x16)", F(macro_cols=128, block_cols=16, rule=mx.RULE_OAS, oas_tau=7.5)),
            ("NVFP4 1x16", F(scale=mx.SCALE_NVFP4, block_cols=16)),
            ("H16 -> NVFP4", F(scale=mx.SCALE_NVFP4, block_cols=16, hadamard=16)),
            ("H32 -> NVFP4", F(scale=mx.SCALE_NVFP4, block_cols=16, hadamard=32))]
    for name, fmt in act:
        run("bf16 16384x4096 activation", name, fmt, x)
    del x
    # operands of the 6- and 8-bit products (gemm_formats): bf16 8192 x 4096 N(0, 1)
    x = up(synth.w2(1.0))
    for name, el in (("MXFP6 E2M3 1x32", mx.ELEM_FP6_E2M3), ("MXFP6 E3M2 1x32", mx.ELEM_FP6_E3M2),
                     ("MXFP8 E4M3 1x32", mx.ELEM_FP8_E4M3), ("MXFP8 E5M2 1x32", mx.ELEM_FP8_E5M2)):
        run("bf16 8192x4096 N(0,1) operand", name, F(elem=el), x)
    del x
    # the counted VALU work of the ALU-heavy cells, where it was measured
    for c in cells:
        v = counted("quantize_formats_valu.json", f"{c['format']} @ {c['config']}")
        if v is not None:
            c["alu"] = {k: v[k] for k in ("valu_insts_per_elem", "alu_bound_gbs", "note") if k in v}
    return cells


def gemm_formats(mx, torch, a, b, C, R, dev, reps=5):
    """The same product with operands in the other block formats the library
    multiplies, for information (not part of the step): A and B quantized on the
    GPU in each format, the product timed with events (median of `reps`), its
    QSNR (eq. (2)) against the bf16 product R, and the fraction of the matrix
    peak of the instruction the path runs on (FP4/FP6 10.1 PFLOP/s; the FP4
    formats with fp8 block scales decode to fp16 or bf16: 2.5 PFLOP/s)."""
    F = mx.Format
    fp6, fp6b = F(elem=mx.ELEM_FP6_E2M3), F(elem=mx.ELEM_FP6_E3M2)
    nv = F(scale=mx.SCALE_NVFP4, block_cols=16)
    cases = [
        ("MXFP4 x MXFP4", mx.MXFP4, mx.MXFP4, "fp4 MFMA, persistent LDS-staged (the step's kernel)", FP4_PEAK_TFLOPS),
        ("MXFP6 E2M3 x MXFP6 E2M3", fp6, fp6, "fp6 MFMA, LDS-staged 256x256 tiles", FP4_PEAK_TFLOPS),
        ("MXFP6 E3M2 x MXFP6 E3M2", fp6b, fp6b, "fp6 MFMA, LDS-staged 256x256 tiles", FP4_PEAK_TFLOPS),
        ("MXFP6 E2M3 x MXFP4", fp6, mx.MXFP4, "fp6 x fp4 MFMA, LDS-staged 256x256 tiles", FP4_PEAK_TFLOPS),
        ("MXFP4-MBS x MXFP4-MBS", F(macro_cols=128), F(macro_cols=128), "fp4 MFMA + per-stage macro-scale fold, LDS-staged 256x256 tiles",
         FP4_PEAK_TFLOPS),
        ("NVFP4 x NVFP4", nv, nv, "fp16 MFMA after exact decode, LDS-staged 256x256 tiles", BF16_PEAK_TFLOPS),
        ("UE5M3/16 x UE5M3/16", F(scale=mx.SCALE_UE5M3, block_cols=16), F(scale=mx.SCALE_UE5M3, block_cols=16),
         "bf16 MFMA after exact decode, LDS-staged 256x256 tiles", BF16_PEAK_TFLOPS),
        ("MBS/16 x MBS/16", F(block_cols=16, macro_cols=128), F(block_cols=16, macro_cols=128),
         "bf16 MFMA after exact decode with the macro scale folded into each 1x16 block's, LDS-staged 256x256 tiles",
         BF16_PEAK_TFLOPS),
        ("MXFP8 E4M3 x MXFP8 E4M3", mx.MXFP8_E4M3, mx.MXFP8_E4M3, "fp8 MFMA, LDS-staged 256x256 tiles", FP8_PEAK_TFLOPS),
        ("MXFP8 E4M3 x MXFP4", mx.MXFP8_E4M3, mx.MXFP4, "fp8 x fp4 MFMA, LDS-staged 256x256 tiles", FP8_PEAK_TFLOPS),
    ]
    out = []
    for name, fa, fb, path, peak in cases:
        qa, _, _ = mx.mx_quantize(fa, a)
        qb, _, _ = mx.mx_quantize(fb, b)
        mx.mx_gemm(fa, qa, fb, qb, c=C)
        torch.cuda.synchronize()
        ms, _ = timed(torch, lambda: mx.mx_gemm(fa, qa, fb, qb, c=C), reps)
        _, db = mx.mx_qsnr(R, C.float())
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out.append({"operands": name, "path": path, "ms": round(ms, 4), "tflops": round(tf, 1),
                    "frac_peak": round(tf / peak, 4), "peak_tflops": peak, "qsnr_ab_db": round(db, 4)})
        del qa, qb
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the quantizer and the GEMM shard by rows without "
                          "communication, and no multi-GPU figure is produced",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_block_quantization_amd as mx
    from microscaling_block_quantization_amd import ceilings as cl
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush_src = torch.empty(FLUSH_BYTES // 2, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    flush = lambda: cl.copy(flush_src, flush_dst)

    if args.only_formats:
        print(json.dumps({"quantize_formats": quantize_formats(mx, torch, np, synth, dev, flush)}), flush=True)
        return

    a_np, b_np = synth.w5(M, N, K)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    if args.only_gemm_formats:
        a_t, b_t = up(a_np), up(b_np)
        c_t = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        r_t = torch.matmul(a_t, b_t.t().contiguous()).float()
        print(json.dumps({"gemm_formats": gemm_formats(mx, torch, a_t, b_t, c_t, r_t, dev)}), flush=True)
        return

    A = [up(a_np)]
    B = [up(b_np)]
    for _ in range(args.sets - 1):
        A.append(A[0].clone())
        B.append(B[0].clone())
    fmt = mx.MXFP4
    qa = mx.alloc_qtensor(fmt, M, K, dev)
    qb = mx.alloc_qtensor(fmt, N, K, dev)
    wsa = mx.alloc_workspace(fmt, M, K, dev)
    wsb = mx.alloc_workspace(fmt, N, K, dev)
    sta = torch.empty(64, dtype=torch.uint8, device=dev)
    stb = torch.empty(64, dtype=torch.uint8, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # events only at the boundaries of the two phases (an event between two
    # kernels costs the stream a few microseconds of its own); every call and
    # event goes to the current stream
    # A and B go to the quantizer in one call (one shared launch, then one
    # launch that finalizes both tensors' statistics)
    def quantize(s, stats=True):
        mx.mx_quantize_many(fmt, [A[s], B[s]], outs=[qa, qb], stats=[sta, stb] if stats else None,
                            workspaces=[wsa, wsb])

    def step(i, ev=None):
        s = i % args.sets
        if ev: ev[0].record()
        quantize(s)
        if ev: ev[1].record()
        mx.mx_gemm(fmt, qa, fmt, qb, c=C)
        if ev: ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i, events[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    q_t = [e[0].elapsed_time(e[1]) for e in events]
    g_t = [e[1].elapsed_time(e[2]) for e in events]
    q_ms, g_ms = sum(q_t) / len(q_t), sum(g_t) / len(g_t)
    q_med, g_med = statistics.median(q_t), statistics.median(g_t)

    quant_bytes = (M + N) * K * QUANT_BYTES_PER_ELEM
    flops = 2.0 * M * N * K
    gbs = lambda ms: quant_bytes / (ms * 1e-3) / 1e9
    tfs = lambda ms: flops / (ms * 1e-3) / 1e12

    # for information, outside the timed steps: the quantizer alone (codes and
    # scales, no statistics), the form a layer uses when fidelity is not wanted
    # (enqueued back to back like the steps, events at the boundaries)
    reps = 20

    def timed(call):
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            ev2[i][0].record()
            call(i % args.sets)
            ev2[i][1].record()
        torch.cuda.synchronize()
        t = [e[0].elapsed_time(e[1]) for e in ev2]
        return sum(t) / reps, statistics.median(t)

    q0, q0_med = timed(lambda s: quantize(s, stats=False))

    # also for information: the same quantization as two mx_quantize calls
    # (four launches with statistics, two without)
    def separate(s, stats=True):
        mx.mx_quantize(fmt, A[s], out=qa, stats=sta if stats else None, workspace=wsa)
        mx.mx_quantize(fmt, B[s], out=qb, stats=stb if stats else None, workspace=wsb)

    qs, qs_med = timed(separate)
    qs0, qs0_med = timed(lambda s: separate(s, stats=False))
    # the step left A's and B's codes of the last input set; recompute them (and
    # the product) for the fidelity figures and the parity check below
    s_last = (args.steps - 1) % args.sets
    quantize(s_last)
    mx.mx_gemm(fmt, qa, fmt, qb, c=C)
    torch.cuda.synchronize()

    # fidelity: eq. (1) for A and B from the fused statistics, eq. (2) for the product
    st_a, st_b = mx.stats_to_dict(sta), mx.stats_to_dict(stb)
    qsnr = lambda st: 10 * np.log10(st["sig2"] / st["err2"])
    R = torch.matmul(A[0], B[0].t().contiguous()).float()     # bf16 reference product (hipBLASLt)
    _, qsnr_ab = mx.mx_qsnr(R, C.float())
    c_rows = C[:256].view(torch.int16).cpu().numpy().view(np.uint16)
    codes_a, scales_a = qa.codes.cpu().numpy(), qa.scales.cpu().numpy()
    codes_b, scales_b = qb.codes.cpu().numpy(), qb.scales.cpu().numpy()
    variants = [] if args.no_formats else gemm_formats(mx, torch, A[0], B[0], C, R, dev)
    del R
    del A, B, C
    torch.cuda.empty_cache()
    ceil = None if args.no_ceilings else ceilings(torch, dev)
    qcells = [] if args.no_formats else quantize_formats(mx, torch, np, synth, dev, flush)

    gt, qt = counted("traffic.json", "gemm"), counted("traffic.json", "quantize")
    out = {
        "metric": "quantize GB/s (% HBM peak) + MXFP4 GEMM TFLOP/s (% MFMA peak) on 1 MI355X",
        "value": round(gbs(q_ms), 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (quantizer arithmetic), e2m1 x e2m1 -> f32 (MFMA)",
        "data": "synthetic",
        "config": {"workload": "W4A4 linear layer: MXFP4-quantize A bf16 8192x4096 N(0,1) and "
                               "B bf16 14336x4096 N(0,0.02^2) (1x32 E2M1, E8M0 floor, RTNE, fused stats), "
                               "then C = A.B^T on block-scaled FP4 MFMA, bf16 out",
                   "M": M, "N": N, "K": K, "quant_bytes_per_step": quant_bytes, "input_sets": args.sets},
        "quantize": {"gbs": round(gbs(q_ms), 1), "frac_hbm_peak": round(gbs(q_ms) / HBM_PEAK_GBS, 4),
                     "ms": round(q_ms, 4), "median_ms": round(q_med, 4),
                     "median_gbs": round(gbs(q_med), 1)},
        "quantize_codes_only": {"gbs": round(gbs(q0), 1), "frac_hbm_peak": round(gbs(q0) / HBM_PEAK_GBS, 4),
                                "ms": round(q0, 4), "median_gbs": round(gbs(q0_med), 1),
                                "note": "same quantizer without the fused statistics; not part of the step"},
        "quantize_separate_calls": {"gbs": round(gbs(qs), 1), "median_gbs": round(gbs(qs_med), 1),
                                    "codes_only_gbs": round(gbs(qs0), 1),
                                    "codes_only_median_gbs": round(gbs(qs0_med), 1),
                                    "note": "A and B by two mx_quantize calls instead of one "
                                            "mx_quantize_many; not part of the step"},
        "gemm": {"tflops": round(tfs(g_ms), 1), "frac_fp4_peak": round(tfs(g_ms) / FP4_PEAK_TFLOPS, 4),
                 "ms": round(g_ms, 4), "median_ms": round(g_med, 4), "median_tflops": round(tfs(g_med), 1)},
        "roofline": {"bound": "mfma", "kernel": "block-scaled MXFP4 GEMM (k_gemm_tiled)",
                     "achieved": round(tfs(g_ms), 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfs(g_ms) / FP4_PEAK_TFLOPS, 4),
                     "traffic": None if gt is None else round(gt["traffic_bytes"])},
        "quantize_roofline": {"bound": "hbm", "kernel": "MXFP4 row quantizer with fused statistics, A and B in one "
                                                        "launch (k_rows_fast_many), + one statistics finalize",
                              "achieved": round(gbs(q_ms), 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(gbs(q_ms) / HBM_PEAK_GBS, 4),
                              "traffic": None if qt is None else round(qt["fetch_bytes"] + qt["write_bytes"])},
        "qsnr_db": {"A": round(qsnr(st_a), 4), "B": round(qsnr(st_b), 4), "AB": round(qsnr_ab, 4)},
        "ceilings": ceil,
        "quantize_formats": qcells,
        "gemm_formats": variants,
        "parity": None,
        "cpu_baseline": None,
    }
    if ceil is not None:
        out["roofline"]["frac_of_mfma_loop_random"] = round(
            tfs(g_ms) / ceil["fp4_mfma_loop_random"]["tflops"], 4)
        out["quantize_roofline"]["frac_of_read4_write1"] = round(gbs(q_ms) / ceil["read4_write1"]["gbs"], 4)
        # the operand stream alone takes this long: the product's time over it
        out["roofline"]["ms_over_lds_dma_stream"] = round(g_ms / ceil["lds_dma_stream"]["ms"], 3)

    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        # repeat the full quantization of A and B until about 10 s of CPU work
        reps, tq = 0, 0.0
        while tq < 10.0 and reps < 50:
            t0 = time.perf_counter()
            ra = oracle.quantize(a_np, oracle.Format())
            rb = oracle.quantize(b_np, oracle.Format())
            tq += time.perf_counter() - t0
            reps += 1
        tq /= reps
        rows = 256
        t0 = time.perf_counter()
        c_ref = oracle.gemm_f64(ra["dequant"][:rows], rb["dequant"])
        tg = time.perf_counter() - t0
        # the fp32 1024 x 1024 configuration, one thread and all threads
        w1 = synth.w1()
        c1 = {}
        for nt in (1, threads):
            oracle.set_threads(nt)
            t0 = time.perf_counter()
            oracle.quantize(w1, oracle.Format())
            c1[nt] = time.perf_counter() - t0
        oracle.set_threads(threads)
        out["cpu_baseline"] = {
            "value": round(quant_bytes / tq / 1e9, 4), "unit": "GB/s", "cores": oracle.get_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"full quantize of A and B ({(M + N) * K} elements), {reps} times, {tq:.3f} s each; "
                      f"GEMM sample {rows}x{N}x{K} float64 in {tg:.2f} s; fp32 1024x1024 MXFP4 with dequant "
                      f"and stats: {c1[1] * 1e3:.1f} ms on 1 thread, {c1[threads] * 1e3:.1f} ms on {threads}",
            "gemm_tflops": round(2.0 * rows * N * K / tg / 1e12, 5),
            "c1_fp32_1024x1024_ms": {"1_thread": round(c1[1] * 1e3, 2), f"{threads}_threads": round(c1[threads] * 1e3, 2)},
        }
        # the step's outputs against the oracle on the same inputs
        want_c = oracle.f32_to_bf16_bits(c_ref.astype(np.float32))
        out["parity"] = {
            "codes_scales_bit_exact": bool(
                np.array_equal(codes_a[:ra["codes"].size], ra["codes"].reshape(-1)) and
                np.array_equal(scales_a[:ra["scales"].size], ra["scales"].reshape(-1)) and
                np.array_equal(codes_b[:rb["codes"].size], rb["codes"].reshape(-1)) and
                np.array_equal(scales_b[:rb["scales"].size], rb["scales"].reshape(-1))),
            "stats_counts_exact": all(st[k] == r["stats"][k] for st, r in ((st_a, ra), (st_b, rb))
                                      for k in ("n", "nonzero", "flushed", "zero_blocks")),
            "qsnr_abs_diff_db": max(abs(qsnr(st_a) - oracle.qsnr_db(ra["stats"])),
                                    abs(qsnr(st_b) - oracle.qsnr_db(rb["stats"]))),
            "gemm_rows_checked": rows,
            "gemm_bf16_bit_exact": bool(np.array_equal(c_rows, want_c)),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
