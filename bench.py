#!/usr/bin/env python3
"""Benchmark of the N:M sparse GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
nm_compress (magnitude prune + pack of W) followed by nm_spmm (Y = W_nm X),
with every input resident in HBM before the timed region starts.

Default workload: a LLaMA-2-7B projection at prefill, W 4096 x 4096 bf16
N(0, 0.02) pruned 2:4 along K, activations 2048 x 4096 bf16 N(0, 1), fp32 Y.

Prints one JSON line (rank 0, N = 1):
  value        dense-equivalent TFLOP/s of the step, 2*R*K*T / t_step
  roofline     the sparse GEMM kernel against the MI355X dense MFMA peak for
               its dtype (decode: against HBM bandwidth): achieved =
               algorithmic FLOP (2*R*S*T, S = K*N/M stored weights per row) or
               bytes / mean kernel duration, from HIP events on its stream
               around the timed region's GEMM phase (the timed steps run their
               compressions first, then their products)
  cpu_baseline the CPU oracle (NumPy, fp64) timed on this host over the same
               workload
  kernels      per-kernel means (sparse GEMM, compress, dense hipBLASLt GEMM
               of the same shape) and the speedup over the dense GEMM
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "2:4 sparse GEMM dense-equivalent TFLOP/s and HBM GB/s; speedup vs dense"
PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0,
                    "f8e4m3": 5000.0}  # MI355X dense MFMA (int8: TOP/s), published
PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="dense-matmul load before the warmup, so the clock has settled "
                         "(an idle GPU takes about a second of load to reach it)")
    ap.add_argument("--workload", type=int, default=2,
                    help="1..7 (default 2: prefill 4096x4096x2048; 6, 7: the same shape in INT8, FP8)")
    ap.add_argument("--T", type=int, default=None, help="tokens (decode workload: 1, 8 or 16)")
    ap.add_argument("--pattern", default=None, help="n:m (workload 4: 1:4 or 1:8)")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "half"])
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=None,
                    help="copies of the inputs cycled through (defeats the 256 MB last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / matmul peaks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy, the reference a counter "
                         "profile of this command scales HBM byte counters against")
    return ap.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key, hsh):
    """HBM bytes per launch from a committed counter summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != hsh:
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(wl, n, m, T, reps):
    """The oracle as it stands, timed on the host: prune+pack, decompress, fp64 GEMM
    (int8: the exact int64 product, on a sample of rows; NumPy has no BLAS for it;
    fp8: the decoded values' fp64 product)."""
    import numpy as np
    from oracle import nm_oracle as O
    w = wl.weights()
    act = wl.activations(T)
    perm = wl.permutation()
    i8 = wl.dtype == "i8"
    f8 = wl.dtype == "f8e4m3"
    rows = 512 if i8 else wl.R  # about 6 s of int64 matmul at 4096 x 2048
    times, t_pack, t_gemm = [], [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        vals, idx = (O.prune_pack_i8(w, n, m) if i8 else O.prune_pack_fp8(w, n, m) if f8 else
                     O.prune_pack(w, n, m))
        t1 = time.perf_counter()
        if i8:
            O.spmm_ref_i8(vals[:rows], idx[:rows], wl.K, n, m, act, perm=perm)
        elif f8:
            O.spmm_ref_fp8(vals, idx, wl.K, n, m, act, perm=perm)
        else:
            O.spmm_ref(vals, idx, wl.K, n, m, act, wl.dtype, perm=perm)
        t2 = time.perf_counter()
        times.append(t2 - t0)
        t_pack.append(t1 - t0)
        t_gemm.append(t2 - t1)
    t = statistics.median(times)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            cores = min(cores, int(os.environ[var]))
            break
    tg = statistics.median(t_gemm)
    tp = statistics.median(t_pack)
    gemm_flops = 2.0 * rows * wl.K * T
    if i8:
        # whole-workload time: the pack as timed, the product scaled from its row sample
        t = tp + tg * wl.R / rows
        sample = (f"{wl.R}x{wl.K}x{T} int8 2:4: prune+pack of all of W, decompress and exact int64 "
                  f"product of its first {rows} rows, scaled to R; median of {reps} runs")
    else:
        sample = (f"whole workload ({wl.R}x{wl.K}x{T}, {n}:{m}): prune+pack, decompress and "
                  f"fp64 matmul; median of {reps} runs, {t:.2f} s each")
    flops = 2.0 * wl.R * wl.K * T
    return {"value": flops / t / 1e12, "unit": "TOP/s" if i8 else "TFLOP/s", "cores": cores,
            "kind": "oracle", "sample": sample, "prune_pack_s": tp, "decompress_gemm_s": tg,
            "gemm_dense_eq_gflops": gemm_flops / tg / 1e9}


def measured_peaks(torch):
    """Peaks measured on this GPU with plain library calls (context for the
    roofline fractions): a 1 GiB device-to-device copy (read + write bytes)
    and a dense bf16 8192^3 matmul (hipBLASLt)."""
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_copy = timed(lambda: dst.copy_(src), 10)
    t_mm = timed(lambda: torch.matmul(a, b), 10)
    out = {"copy_gbps": 2.0 * src.numel() * 2 / t_copy / 1e9,
           "dense_bf16_matmul_tflops": 2.0 * 8192 ** 3 / t_mm / 1e12,
           "how": "1 GiB torch copy (read+write bytes / t); torch.matmul bf16 8192^3"}
    del src, dst, a, b
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the per-GPU kernel is what --gpus 1 times); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nm_inputs
    import structured_sparse_gemm_nm_amd as nm

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    nm.lib()  # fails loudly if the library is not built

    wl = nm_inputs.WORKLOADS[args.workload]
    T = args.T if args.T is not None else wl.Ts[-1] if args.workload == 3 else wl.Ts[0]
    if args.pattern:
        n, m = (int(v) for v in args.pattern.split(":"))
    else:
        n, m = wl.patterns[0]
    R, K = wl.R, wl.K
    S = K // m * n
    dt = wl.dtype
    i8 = dt == "i8"
    f8 = dt == "f8e4m3"
    b8 = i8 or f8  # one-byte weights and activations
    tdt = (torch.int8 if i8 else torch.float8_e4m3fn if f8 else torch.float16 if dt == "f16" else
           torch.bfloat16)
    # int8 weights give the exact int32 product, fp8 ones an fp32 product
    out_dtype = (torch.int32 if i8 else torch.float32 if f8 or args.out_dtype == "f32" else tdt)
    out_name = "i32" if i8 else "f32" if f8 else args.out_dtype
    nm.nm_set_variant(args.variant)

    def dev(bits):
        if b8:
            return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(tdt)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

    W = dev(wl.weights())
    act = dev(wl.activations(T))
    perm_np = wl.permutation()
    perm = torch.from_numpy(perm_np).cuda() if perm_np is not None else None
    dcode = nm.NM_I8 if i8 else nm.NM_FP8 if f8 else nm.NM_F16 if dt == "f16" else nm.NM_BF16
    vb, ib, words = nm.nm_packed_sizes(R, K, n, m, dcode)
    esz = 1 if b8 else 2
    ybytes = T * R * (4 if out_dtype in (torch.float32, torch.int32) else 2)
    step_bytes = vb + ib + T * K * esz + ybytes  # the GEMM's algorithmic bytes

    # Rotation: enough copies that one pass over them exceeds the 256 MB cache.
    rotate = args.rotate if args.rotate is not None else (1 if args.workload == 2 else
                                                          max(1, min(64, -(-320_000_000 // step_bytes))))
    copies = []
    for c in range(rotate):
        Wc = W if c == 0 else W.clone()
        Ac = act if c == 0 else act.clone()
        vals = torch.empty((R, S), dtype=tdt, device="cuda")
        idx = torch.empty((R, words), dtype=torch.int32, device="cuda")
        Y = torch.empty((T, R), dtype=out_dtype, device="cuda")
        copies.append((Wc, Ac, vals, idx, Y))

    def gemm(c):
        _, Ac, vals, idx, Y = copies[c]
        if perm is None:
            nm.nm_spmm(vals, idx, Ac, K, n, m, out_dtype=out_dtype, out=Y)
        else:
            nm.nm_spmm_perm(vals, idx, Ac, perm, K, n, m, out_dtype=out_dtype, out=Y)

    def compress(c):
        Wc, _, vals, idx, _ = copies[c]
        nm.nm_compress(Wc, n, m, values=vals, idx=idx)

    # ---- clock settling: an idle GPU starts at a low clock and takes about a
    # second of load to reach its steady state; that load is a dense torch
    # matmul, so no launch of the kernels under test happens outside the
    # warmup, the timed region and the per-kernel loops below
    settle = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    tw = time.perf_counter()
    while (time.perf_counter() - tw) * 1e3 < args.settle_ms:
        for _ in range(8):
            torch.matmul(settle, settle)
        torch.cuda.synchronize()
    del settle

    # ---- warmup: W steps in the timed region's order (their compressions,
    # then their products)
    for i in range(args.warmup):
        compress(i % rotate)
    for i in range(args.warmup):
        gemm(i % rotate)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps.  Every step compresses one copy
    # of W and multiplies with it; the steps' compressions run first, then
    # their products, so one event between the two phases times each kernel's
    # mean launch on the stream they run on (an event pair around every launch
    # adds its own cost to each), and with several copies a product reads
    # weights the later compressions have pushed out of the last-level cache.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    mid = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        compress(i % rotate)
    mid.record()
    for i in range(args.steps):
        gemm(i % rotate)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    compress_mean_us = start.elapsed_time(mid) * 1e3 / args.steps
    gemm_mean_us = mid.elapsed_time(end) * 1e3 / args.steps

    # ---- per-kernel breakdown (back-to-back launches of one kernel)
    def time_loop(fn, iters):
        for i in range(5):
            fn(i % rotate)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(iters):
            fn(i % rotate)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    iters = max(20, args.steps)
    gemm_loop_us = time_loop(gemm, iters)
    compress_us = time_loop(compress, iters)
    dense = []
    for c in range(rotate):
        dense.append(nm.nm_decompress(copies[c][2], copies[c][3], K, n, m))
    actp = [copies[c][1] if perm is None else copies[c][1][:, perm.long()].contiguous()
            for c in range(rotate)]

    if i8:
        # dense int8 GEMM with an int32 result (hipBLASLt through torch._int_mm)
        dense_t = [d.t() for d in dense]  # [K, R], column-major view of the row-major W

        def dense_gemm(c):
            torch._int_mm(actp[c], dense_t[c])
    elif f8:
        # dense fp8 GEMM with an fp32 result (hipBLASLt through torch._scaled_mm, unit scales)
        dense_t = [d.t() for d in dense]
        one = torch.ones((), dtype=torch.float32, device="cuda")

        def dense_gemm(c):
            torch._scaled_mm(actp[c], dense_t[c], scale_a=one, scale_b=one, out_dtype=torch.float32)
    else:
        def dense_gemm(c):
            torch.nn.functional.linear(actp[c], dense[c])

    try:
        dense_us = time_loop(dense_gemm, iters)
    except RuntimeError as e:  # no dense 8-bit GEMM for this shape / build
        print(f"dense reference unavailable: {e}", file=sys.stderr)
        dense_us = None
    gemm_half_us = None
    if not b8:  # a rounded half-precision output (8-bit weights have a 4-byte one only)
        y_half = torch.empty((T, R), dtype=tdt, device="cuda")

        def gemm_half(c):
            _, Ac, vals, idx, _ = copies[c]
            if perm is None:
                nm.nm_spmm(vals, idx, Ac, K, n, m, out_dtype=tdt, out=y_half)
            else:
                nm.nm_spmm_perm(vals, idx, Ac, perm, K, n, m, out_dtype=tdt, out=y_half)

        gemm_half_us = time_loop(gemm_half, iters)

    dense_eq_flop = 2.0 * R * K * T
    alg_flop = 2.0 * R * S * T
    achieved_tflops = alg_flop / (gemm_mean_us * 1e-6) / 1e12
    lib_src = [os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "csrc", f)
               for f in sorted(os.listdir(os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "csrc")))]
    hsh = source_hash(lib_src)
    kernel_key = f"spmm_w{args.workload}_{n}of{m}_T{T}_{out_name}"
    roofline_bound = "mfma" if args.workload in (1, 2, 4, 6, 7) else "hbm"
    unit = "TOP/s" if i8 else "TFLOP/s"
    if roofline_bound == "mfma":
        roofline = {"bound": "mfma", "achieved": achieved_tflops, "peak": PEAK_MFMA_TFLOPS[dt],
                    "unit": unit, "frac": achieved_tflops / PEAK_MFMA_TFLOPS[dt],
                    "traffic": traffic_from_profile(kernel_key, hsh)}
    else:
        gbps = step_bytes / (gemm_mean_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": gbps / PEAK_HBM_GBPS, "traffic": traffic_from_profile(kernel_key, hsh)}
    roofline["kernel"] = "nm_spmm" if perm is None else "nm_spmm_perm"
    roofline["per_launch"] = {"flop": alg_flop, "bytes": step_bytes, "mean_us": gemm_mean_us}
    # roofline times: the algorithmic bound (stored weights only) and the bound
    # at the 2:4 smfmac rate (1:4 / 1:8 widened to the 2:4 operand), each the
    # larger of the MFMA time and the HBM time of the algorithmic bytes
    peak_f = PEAK_MFMA_TFLOPS[dt] * 1e12
    t_hbm = step_bytes / (PEAK_HBM_GBPS * 1e9)
    t_alg = max(alg_flop / peak_f, t_hbm)
    t_24 = max(dense_eq_flop / 2.0 / peak_f, t_hbm)
    roofline["t_roof_us"] = {"algorithmic": t_alg * 1e6, "at_2of4_rate": t_24 * 1e6}
    roofline["frac_of_t_roof"] = {"algorithmic": t_alg / (gemm_mean_us * 1e-6),
                                  "at_2of4_rate": t_24 / (gemm_mean_us * 1e-6)}

    extra = {}
    if perm is not None:
        y_plain = torch.empty((T, R), dtype=out_dtype, device="cuda")
        ident = torch.arange(K, dtype=torch.int32, device="cuda")

        def plain(c):
            _, Ac, vals, idx, _ = copies[c]
            nm.nm_spmm(vals, idx, Ac, K, n, m, out_dtype=out_dtype, out=y_plain)

        def identity(c):
            _, Ac, vals, idx, _ = copies[c]
            nm.nm_spmm_perm(vals, idx, Ac, ident, K, n, m, out_dtype=out_dtype, out=y_plain)

        plain_us = time_loop(plain, iters)
        ident_us = time_loop(identity, iters)
        extra = {"nm_spmm_no_perm_us": plain_us, "nm_spmm_perm_identity_us": ident_us,
                 "perm_overhead_vs_no_perm": gemm_loop_us / plain_us - 1.0,
                 "perm_overhead_vs_identity_perm": gemm_loop_us / ident_us - 1.0}

    out = {
        "metric": METRIC,
        "value": dense_eq_flop / (ms_step * 1e-3) / 1e12,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": ("synthetic (seeded N(0,1)*32 rounded to int8, the workload's shapes)" if i8 else
                 "synthetic (seeded N(0,1) rounded to E4M3, the workload's shapes)" if f8 else
                 "synthetic (seeded N(0,sigma) inputs of the workload's shapes)"),
        "config": {"workload": wl.name, "R": R, "K": K, "T": T, "pattern": f"{n}:{m}",
                   "out_dtype": out_name, "permuted": perm is not None,
                   "rotate": rotate,
                   "step": "nm_compress + nm_spmm", "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {
            "nm_spmm_us_in_step": gemm_mean_us,
            "nm_compress_us_in_step": compress_mean_us,
            "nm_spmm_us_loop": gemm_loop_us,
            "nm_spmm_dense_eq_tflops": dense_eq_flop / (gemm_loop_us * 1e-6) / 1e12,
            "nm_spmm_packed_gbps": (vb + ib) / (gemm_loop_us * 1e-6) / 1e9,
            "nm_spmm_alg_gbps": step_bytes / (gemm_loop_us * 1e-6) / 1e9,
            "nm_spmm_half_out_us": gemm_half_us,
            "nm_compress_us": compress_us,
            "nm_compress_gbps": (R * K * esz + vb + ib) / (compress_us * 1e-6) / 1e9,
            "dense_linear_us": dense_us,
            "speedup_vs_dense_half_out": dense_us / gemm_half_us if dense_us and gemm_half_us else None,
            "speedup_vs_dense_f32_out": dense_us / gemm_loop_us if dense_us else None,
            **extra,
        },
        "wall_s_timed": wall,
        "source_hash": hsh,
    }
    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel() * 4
    if not args.no_peaks:
        pk = measured_peaks(torch)
        out["measured_peaks"] = pk
        if roofline["bound"] == "hbm":
            roofline["frac_of_measured_copy"] = roofline["achieved"] / pk["copy_gbps"]
        elif not b8:
            roofline["frac_of_measured_dense_matmul"] = roofline["achieved"] / pk["dense_bf16_matmul_tflops"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, n, m, T, args.cpu_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
