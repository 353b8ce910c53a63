#!/usr/bin/env python3
"""Benchmark of the microscaling hot path on one MI355X.

One step = one W4A4 linear layer at Llama-8B MLP shape, on synthetic data:
  quantize A (bf16 8192 x 4096 ~ N(0, 1))      -> MXFP4 codes + E8M0 scales + stats
  quantize B (bf16 14336 x 4096 ~ N(0, .02^2)) -> MXFP4 codes + E8M0 scales + stats
  C = deq(A) . deq(B)^T on the block-scaled FP4 MFMA, fp32 accumulate, bf16 out
(MXFP4 = 1x32 E2M1 blocks with E8M0 scales, floor rule, round-to-nearest-even).

Reported: quantizer GB/s (algorithmic bytes: 2 B read + 0.5 B codes + 1/32 B
scale per element) as `value`, GEMM TFLOP/s (2 M N K per product), each with
its fraction of the MI355X peak, QSNR of A, B (eq. (1)) and of the product
(eq. (2)) against the bf16 product, and the CPU oracle timed on this host.

After the timed steps, the same product in the other block formats (MXFP6,
mixed 6-/4-bit, MXFP4 with macro-block scales, NVFP4, UE5M3) is timed for
information under "gemm_formats", with its QSNR (eq. (2)).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-formats]
"""
import argparse
import hashlib
import json
import os
import sys
import time

M, N, K = 8192, 14336, 4096
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0        # MI355X dense MXFP4 (and FP6) MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, TFLOP/s
QUANT_BYTES_PER_ELEM = 2 + 0.5 + 1.0 / 32


HERE = os.path.dirname(os.path.abspath(__file__))


def counted_traffic(key):
    """HBM bytes per launch measured with the FETCH_SIZE / WRITE_SIZE counters
    (profiles/traffic.json), or None when the kernel's sources changed since."""
    try:
        with open(os.path.join(HERE, "profiles", "traffic.json")) as f:
            k = json.load(f)["kernels"][key]
        h = hashlib.sha256()
        for src in k["sources"]:
            with open(os.path.join(HERE, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] != k["sha"]:
            return None
        return k
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated to defeat the 256 MB MALL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the products in the other block formats (not part of the step)")
    return ap.parse_args()


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
    ]
    out = []
    for name, fa, fb, path, peak in cases:
        qa, _, _ = mx.mx_quantize(fa, a)
        qb, _, _ = mx.mx_quantize(fb, b)
        mx.mx_gemm(fa, qa, fb, qb, c=C)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record()
            mx.mx_gemm(fa, qa, fb, qb, c=C)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        ms = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps))[reps // 2]
        _, db = mx.mx_qsnr(R, C.float())
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out.append({"operands": name, "path": path, "ms": round(ms, 4), "tflops": round(tf, 1),
                    "frac_peak": round(tf / peak, 4), "peak_tflops": peak, "qsnr_ab_db": round(db, 4)})
        del qa, qb
    return out


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
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a_np, b_np = synth.w5(M, N, K)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

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

    # events only at the boundaries of the two phases: an event between two
    # kernels costs the stream a few microseconds of its own
    nev = 3
    def step(i, ev=None):
        s = i % args.sets
        if ev: ev[0].record()
        mx.mx_quantize(fmt, A[s], out=qa, stats=sta, workspace=wsa)
        mx.mx_quantize(fmt, B[s], out=qb, stats=stb, workspace=wsb)
        if ev: ev[1].record()
        mx.mx_gemm(fmt, qa, fmt, qb, c=C)
        if ev: ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i, events[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    q_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    g_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps

    quant_bytes = (M + N) * K * QUANT_BYTES_PER_ELEM
    quant_gbs = quant_bytes / (q_ms * 1e-3) / 1e9
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12

    # for information, outside the timed steps: the quantizer alone (codes and
    # scales, no statistics), the form a layer uses when fidelity is not wanted
    reps = 10
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        s = i % args.sets
        ev2[i][0].record()
        mx.mx_quantize(fmt, A[s], out=qa, workspace=wsa)
        mx.mx_quantize(fmt, B[s], out=qb, workspace=wsb)
        ev2[i][1].record()
    torch.cuda.synchronize()
    q0 = sum(e[0].elapsed_time(e[1]) for e in ev2) / reps
    quant0_gbs = quant_bytes / (q0 * 1e-3) / 1e9
    # the step left A's and B's codes of the last input set; recompute them (and
    # the product) for the fidelity figures below
    s_last = (args.steps - 1) % args.sets
    mx.mx_quantize(fmt, A[s_last], out=qa, stats=sta, workspace=wsa)
    mx.mx_quantize(fmt, B[s_last], out=qb, stats=stb, workspace=wsb)
    mx.mx_gemm(fmt, qa, fmt, qb, c=C)
    torch.cuda.synchronize()

    # fidelity: eq. (1) for A and B from the fused statistics, eq. (2) for the product
    st_a, st_b = mx.stats_to_dict(sta), mx.stats_to_dict(stb)
    qsnr = lambda st: 10 * np.log10(st["sig2"] / st["err2"])
    R = torch.matmul(A[0], B[0].t().contiguous()).float()     # bf16 reference product (hipBLASLt)
    _, qsnr_ab = mx.mx_qsnr(R, C.float())
    variants = [] if args.no_formats else gemm_formats(mx, torch, A[0], B[0], C, R, dev)
    del R

    gt, qt = counted_traffic("gemm"), counted_traffic("quantize")
    out = {
        "metric": "quantize GB/s (% HBM peak) + MXFP4 GEMM TFLOP/s (% MFMA peak) on 1 MI355X",
        "value": round(quant_gbs, 1),
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
                   "M": M, "N": N, "K": K, "quant_bytes_per_step": quant_bytes},
        "quantize": {"gbs": round(quant_gbs, 1), "frac_hbm_peak": round(quant_gbs / HBM_PEAK_GBS, 4),
                     "ms": round(q_ms, 4)},
        "quantize_codes_only": {"gbs": round(quant0_gbs, 1), "frac_hbm_peak": round(quant0_gbs / HBM_PEAK_GBS, 4),
                                "ms": round(q0, 4),
                                "note": "same quantizer without the fused statistics; not part of the step"},
        "gemm": {"tflops": round(gemm_tflops, 1), "frac_fp4_peak": round(gemm_tflops / FP4_PEAK_TFLOPS, 4),
                 "ms": round(g_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": "block-scaled MXFP4 GEMM",
                     "achieved": round(gemm_tflops, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / FP4_PEAK_TFLOPS, 4),
                     "traffic": None if gt is None else round(gt["traffic_bytes"])},
        "quantize_roofline": {"bound": "hbm", "kernel": "MXFP4 row quantizer with fused statistics "
                                                        "(+ statistics finalize), A and B",
                              "achieved": round(quant_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(quant_gbs / HBM_PEAK_GBS, 4),
                              "traffic": None if qt is None else round(
                                  sum(qt[t]["fetch_bytes"] + qt[t]["write_bytes"] for t in ("A", "B")))},
        "qsnr_db": {"A": round(qsnr(st_a), 4), "B": round(qsnr(st_b), 4), "AB": round(qsnr_ab, 4)},
        "gemm_formats": variants,
        "cpu_baseline": None,
    }

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
        oracle.gemm_f64(ra["dequant"][:rows], rb["dequant"])
        tg = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": round(quant_bytes / tq / 1e9, 4), "unit": "GB/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"full quantize of A and B ({(M + N) * K} elements), {reps} times, {tq:.3f} s each; "
                      f"GEMM sample {rows}x{N}x{K} float64 in {tg:.2f} s",
            "gemm_tflops": round(2.0 * rows * N * K / tg / 1e12, 5),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
