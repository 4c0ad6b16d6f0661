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
  kernels      per-kernel means (sparse GEMM with fp32 and with half output,
               compress, dense hipBLASLt GEMMs of the same shape with the same
               output dtypes), timed in alternating blocks, and the speedup
               over the dense GEMM at equal output dtype
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
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (FMA = 2 FLOP), published


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="dense-matmul load before the warmup, so the clock has settled "
                         "(an idle GPU takes about a second of load to reach it)")
    ap.add_argument("--workload", type=int, default=2,
                    help="1..11 (default 2: prefill 4096x4096x2048; 6, 7: the same shape in INT8, FP8; "
                         "8: the same shape in hybrid dense / 2:4 tiles; 9: its training-side "
                         "products dX and dW; 10, 11: workload 5's permuted layer on a block-sparse and a "
                         "diagonal-sparse weight)")
    ap.add_argument("--T", type=int, default=None, help="tokens (decode workload: 1, 8 or 16)")
    ap.add_argument("--pattern", default=None, help="n:m (workload 4: 1:4 or 1:8)")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "half"])
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=None,
                    help="copies of the inputs cycled through (defeats the 256 MB last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / matmul peaks")
    ap.add_argument("--print-source-hash", choices=sorted(KERNEL_SOURCES), default=None,
                    help="print the source hash of one family of kernels (the key a counter "
                         "summary is filed under) and exit")
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


CSRC = os.path.join(ROOT, "structured_sparse_gemm_nm_amd", "csrc")
# The sources each family of kernels is built from: its own translation units,
# plus the shared device and host headers, the C ABI's dispatch and the public
# header.  Counters taken on one family stay valid while only another changes.
KERNEL_SOURCES = {
    "spmm": ["nm_spmm.hip", "nm_spmm_lds.hip", "nm_spmm_lds_nm.hip", "nm_spmm_decode.hip",
             "nm_spmm_pipe.hip", "nm_spmm_resident.hip", "nm_permute.hip", "nm_int8.hip"],
    "hybrid": ["nm_hybrid.hip", "nm_select.h"],
    "host": ["nm_hosts.hip"],
    "train": ["nm_train.hip"],
}
SHARED_SOURCES = ["nm_device.h", "nm_internal.h", "nm_api.cpp"]


def kernel_source_hash(family):
    files = [os.path.join(CSRC, f) for f in KERNEL_SOURCES[family] + SHARED_SOURCES]
    return source_hash(files + [os.path.join(ROOT, "include", "nmsparse.h")])


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


def cpu_baseline_hybrid(wl, T, reps):
    """The hybrid-tile oracle as it stands (pack, decompress, fp64 GEMM) on the first
    eight tile-rows of W, scaled to all of them."""
    from oracle import nm_hybrid as H
    tr, tc, _ = wl.hybrid
    flags = wl.tile_flags()
    rb = 8
    w = wl.weights()[:rb * tr]
    act = wl.activations(T)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        v, i = H.hybrid_pack(w, tr, tc, flags[:rb])
        H.hybrid_spmm_ref(v, i, rb * tr, wl.K, tr, tc, flags[:rb], act, wl.dtype)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times) * flags.shape[0] / rb
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"value": 2.0 * wl.R * wl.K * T / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"{wl.R}x{wl.K}x{T} hybrid {tr}x{tc} tiles: pack, decompress and fp64 matmul of "
                       f"the first {rb} of {flags.shape[0]} tile-rows, scaled; median of {reps} runs")}


def bench_hybrid(args, wl):
    """Hybrid dense / 2:4 tiles: one step = nm_hybrid_compress + nm_hybrid_spmm."""
    import numpy as np
    import torch

    import structured_sparse_gemm_nm_amd as nm

    R, K = wl.R, wl.K
    T = args.T if args.T is not None else wl.Ts[0]
    tr, tc, frac = wl.hybrid
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
    out_dtype = torch.float32 if args.out_dtype == "f32" else tdt
    flags = wl.tile_flags()
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

    W = dev(wl.weights())
    act = dev(wl.activations(T))
    vals = torch.empty(L.values_count, dtype=tdt, device="cuda")
    idx = torch.zeros(max(L.idx_bytes, 16), dtype=torch.uint8, device="cuda")
    Y = torch.empty((T, R), dtype=out_dtype, device="cuda")
    y_half = torch.empty((T, R), dtype=tdt, device="cuda")

    def compress(_c=0):
        nm.nm_hybrid_compress(W, L, values=vals, idx=idx)

    def gemm(_c=0):
        nm.nm_hybrid_spmm(vals, idx, L, act, out_dtype=out_dtype, out=Y)

    settle = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    tw = time.perf_counter()
    while (time.perf_counter() - tw) * 1e3 < args.settle_ms:
        for _ in range(8):
            torch.matmul(settle, settle)
        torch.cuda.synchronize()
    del settle
    for _ in range(args.warmup):
        compress()
    for _ in range(args.warmup):
        gemm()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    start.record()
    for _ in range(args.steps):
        compress()
    mid.record()
    for _ in range(args.steps):
        gemm()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    compress_mean_us = start.elapsed_time(mid) * 1e3 / args.steps
    gemm_mean_us = mid.elapsed_time(end) * 1e3 / args.steps

    # per-kernel blocks, alternating (see main): the hybrid product with both
    # output dtypes, the dense GEMMs with the same ones, and the all-2:4 product
    v24, i24 = nm.nm_compress(W, 2, 4)
    # dense operand: the weight as the hybrid pruning leaves it (W_hat^T, row-major)
    W_hat_t = _hybrid_dense_operand(nm, torch, W, L, flags, tdt)
    loops = {"gemm": gemm, "compress": compress,
             "gemm_half": lambda c: nm.nm_hybrid_spmm(vals, idx, L, act, out_dtype=tdt, out=y_half),
             "dense_half": lambda c: torch.mm(act, W_hat_t),
             "dense_f32": lambda c: torch.mm(act, W_hat_t, out_dtype=torch.float32),
             "all_2of4": lambda c: nm.nm_spmm(v24, i24, act, K, 2, 4, out_dtype=out_dtype)}
    iters = max(20, args.steps)
    for name in list(loops):
        try:
            for _ in range(3):
                loops[name](0)
            torch.cuda.synchronize()
        except RuntimeError as e:
            print(f"{name} unavailable: {e}", file=sys.stderr)
            del loops[name]
    samples = {name: [] for name in loops}
    for _ in range(5):
        for name, fn in loops.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(iters):
                fn(0)
            b.record()
            torch.cuda.synchronize()
            samples[name].append(a.elapsed_time(b) * 1e3 / iters)
    loop_us = {name: float(np.median(v)) for name, v in samples.items()}

    def ratio(x, y):
        return loop_us[x] / loop_us[y] if x in loop_us and y in loop_us else None

    alg_flop = 2.0 * T * L.values_count           # one MAC per stored weight and token
    dense_eq_flop = 2.0 * R * K * T
    achieved = alg_flop / (gemm_mean_us * 1e-6) / 1e12
    hsh = kernel_source_hash("hybrid")
    out_name = args.out_dtype
    kernel_key = f"hybrid_w{wl.wid}_{tr}x{tc}_T{T}_{out_name}"
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_TFLOPS[wl.dtype], "traffic": traffic_from_profile(kernel_key, hsh),
                "kernel": "nm_hybrid_spmm",
                "per_launch": {"flop": alg_flop, "mean_us": gemm_mean_us,
                               "bytes": L.values_count * 2 + L.idx_bytes + T * K * 2 +
                               T * R * (4 if out_name == "f32" else 2)}}
    dense_tiles = float(flags.mean())
    out = {
        "metric": METRIC, "value": dense_eq_flop / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,sigma) inputs of the workload's shapes; seeded tile flags)",
        "config": {"workload": wl.name, "R": R, "K": K, "T": T, "tiles": f"{tr}x{tc}",
                   "dense_tile_fraction": dense_tiles, "zero_fraction": 0.5 * (1.0 - dense_tiles),
                   "out_dtype": out_name, "step": "nm_hybrid_compress + nm_hybrid_spmm",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {
            "nm_hybrid_spmm_us_in_step": gemm_mean_us, "nm_hybrid_compress_us_in_step": compress_mean_us,
            "nm_hybrid_spmm_us_loop": loop_us.get("gemm"), "nm_hybrid_spmm_half_out_us": loop_us.get("gemm_half"),
            "nm_hybrid_compress_us": loop_us.get("compress"),
            "dense_half_out_us": loop_us.get("dense_half"), "dense_f32_out_us": loop_us.get("dense_f32"),
            "all_2of4_nm_spmm_us": loop_us.get("all_2of4"),
            "speedup_vs_dense_same_out_dtype": {k: v for k, v in {
                "f32": ratio("dense_f32", "gemm") if out_name == "f32" else None,
                "half": ratio("dense_half", "gemm_half")}.items() if v is not None},
        },
        "wall_s_timed": wall, "source_hash": hsh,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_hybrid(wl, T, args.cpu_reps)
    print(json.dumps(out), flush=True)


def cpu_baseline_host(wl, T, reps):
    """The host-structure oracle as it stands (pack + the dense fp64 product of
    the stored matrix with act read through perm) on the first 16384 tokens
    (all of them at the workload's size), scaled to all T (the product is
    linear in the token count)."""
    from oracle import nm_hosts as H
    kind, _ = wl.host
    w = wl.weights()
    perm = wl.permutation()
    ts = min(T, 16384)
    act = wl.activations(T)[:ts]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        if kind == "block":
            row_ptr, col = H.block_structure(wl.block_mask())
            vals = H.block_pack(w, row_ptr, col)
            H.block_spmm_ref(vals, row_ptr, col, wl.R, wl.K, act, wl.dtype, perm=perm)
        else:
            offs = wl.diag_offsets()
            vals = H.diag_pack(w, offs)
            H.diag_spmm_ref(vals, offs, wl.R, wl.K, act, wl.dtype, perm=perm)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times) * T / ts
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"value": 2.0 * wl.R * wl.K * T / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"{wl.R}x{wl.K}x{T} {kind}: pack, densify and fp64 product through perm over the first "
                       f"{ts} of {T} tokens, scaled; median of {reps} runs")}


def bench_host(args, wl):
    """The permutation on a block-sparse or diagonal-sparse weight: one step =
    nm_block_compress + nm_block_spmm (or the diagonal pair) with act read
    through perm."""
    import numpy as np
    import torch

    import structured_sparse_gemm_nm_amd as nm

    kind, param = wl.host
    R, K = wl.R, wl.K
    T = args.T if args.T is not None else wl.Ts[0]
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
    out_dtype = torch.float32 if args.out_dtype == "f32" else tdt
    out_name = args.out_dtype
    ob = 4 if out_name == "f32" else 2

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    W = dev(wl.weights())
    perm = i32(wl.permutation())
    if kind == "block":
        row_ptr, col = nm.nm_block_structure(R, K, wl.block_mask())
        rp, cl = i32(row_ptr), i32(col)
        nnz = int(col.size)
        vals = nm.nm_block_compress(W, rp, cl)
        stored = nnz * 1024
        struct_bytes = rp.numel() * 4 + cl.numel() * 4
    else:
        offs = i32(wl.diag_offsets())
        nnz = int(offs.numel())
        vals = nm.nm_diag_compress(W, offs)
        stored = nnz * R
        struct_bytes = nnz * 4
    step_bytes = stored * 2 + T * K * 2 + T * R * ob
    rotate = args.rotate if args.rotate is not None else max(1, min(64, -(-320_000_000 // step_bytes)))
    acts = [dev(wl.activations(T))]
    for _ in range(rotate - 1):
        acts.append(acts[0].clone())
    outs = [torch.empty((T, R), dtype=out_dtype, device="cuda") for _ in range(rotate)]
    vbuf = torch.empty_like(vals)

    def compress(c=0):
        if kind == "block":
            nm.nm_block_compress(W, rp, cl, values=vbuf)
        else:
            nm.nm_diag_compress(W, offs, values=vbuf)

    def product(c=0, p=perm, odt=out_dtype, out=None):
        o = outs[c % rotate] if out is None else out
        if kind == "block":
            return nm.nm_block_spmm(vals, rp, cl, acts[c % rotate], perm=p, out_dtype=odt, out=o)
        return nm.nm_diag_spmm(vals, offs, acts[c % rotate], perm=p, out_dtype=odt, out=o)

    settle = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    tw = time.perf_counter()
    while (time.perf_counter() - tw) * 1e3 < args.settle_ms:
        for _ in range(8):
            torch.matmul(settle, settle)
        torch.cuda.synchronize()
    del settle
    for i in range(args.warmup):
        compress(i)
    for i in range(args.warmup):
        product(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    start.record()
    for i in range(args.steps):
        compress(i)
    mid.record()
    for i in range(args.steps):
        product(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    compress_us = start.elapsed_time(mid) * 1e3 / args.steps
    spmm_us = mid.elapsed_time(end) * 1e3 / args.steps

    # dense hipBLASLt product on the stored matrix densified (act @ W_hat^T),
    # the same product without the map, and half output, in alternating blocks
    if kind == "block":
        W_hat = torch.zeros_like(W)
        mask = torch.from_numpy(np.kron(wl.block_mask(), np.ones((32, 32), dtype=np.uint8)).astype(bool)).cuda()
        W_hat[mask] = W[mask]
    else:
        cols = (torch.arange(R, device="cuda")[None, :] + offs.long()[:, None]) % K
        W_hat = torch.zeros_like(W)
        W_hat[torch.arange(R, device="cuda")[None, :].expand_as(cols), cols] = vals
    W_hat_t = W_hat.t().contiguous()
    half_out = torch.empty((T, R), dtype=tdt, device="cuda")
    loops = {"spmm": lambda c: product(c), "compress": compress,
             "spmm_no_perm": lambda c: product(c, p=None),
             "spmm_half": lambda c: product(c, odt=tdt, out=half_out),
             "dense_half": lambda c: torch.mm(acts[c % rotate], W_hat_t),
             "dense_f32": lambda c: torch.mm(acts[c % rotate], W_hat_t, out_dtype=torch.float32)}
    iters = max(20, args.steps)
    for name in list(loops):
        try:
            for i in range(3):
                loops[name](i)
            torch.cuda.synchronize()
        except RuntimeError as e:
            print(f"{name} unavailable: {e}", file=sys.stderr)
            del loops[name]
    samples = {name: [] for name in loops}
    for _ in range(5):
        for name, fn in loops.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(iters):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            samples[name].append(a.elapsed_time(b) * 1e3 / iters)
    loop_us = {name: float(np.median(v)) for name, v in samples.items()}

    def ratio(x, y):
        return loop_us[x] / loop_us[y] if x in loop_us and y in loop_us else None

    flop = 2.0 * stored * T                     # one MAC per stored weight and token
    nbytes = stored * 2 + struct_bytes + T * K * 2 + T * R * ob + K * 4
    kname = "nm_block_spmm" if kind == "block" else "nm_diag_spmm"
    hsh = kernel_source_hash("host")
    if kind == "block":
        ach = nbytes / (spmm_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS}
    else:
        ach = flop / (spmm_us * 1e-6) / 1e12
        roofline = {"bound": "alu", "achieved": ach, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                    "frac": ach / PEAK_FP32_VALU_TFLOPS}
    roofline.update({"traffic": traffic_from_profile(f"host_{kind}_w{wl.wid}_T{T}_{out_name}", hsh), "kernel": kname,
                     "per_launch": {"flop": flop, "bytes": nbytes, "mean_us": spmm_us}})
    out = {
        "metric": METRIC, "value": 2.0 * R * K * T / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,sigma) W and act, seeded structure and permutation)",
        "config": {"workload": wl.name, "R": R, "K": K, "T": T, "structure": kind,
                   ("kept_blocks" if kind == "block" else "diagonals"): nnz,
                   "density": stored / (R * K), "out_dtype": out_name, "rotate": rotate,
                   "step": f"{'nm_block_compress' if kind == 'block' else 'nm_diag_compress'} + {kname} (perm)",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {
            f"{kname}_us_in_step": spmm_us, "compress_us_in_step": compress_us,
            f"{kname}_us_loop": loop_us.get("spmm"), f"{kname}_no_perm_us": loop_us.get("spmm_no_perm"),
            f"{kname}_half_out_us": loop_us.get("spmm_half"), "compress_us": loop_us.get("compress"),
            "dense_half_out_us": loop_us.get("dense_half"), "dense_f32_out_us": loop_us.get("dense_f32"),
            "perm_overhead": (ratio("spmm", "spmm_no_perm") - 1.0) if ratio("spmm", "spmm_no_perm") else None,
            "speedup_vs_dense_same_out_dtype": {k: v for k, v in {
                "f32": ratio("dense_f32", "spmm") if out_name == "f32" else None,
                "half": ratio("dense_half", "spmm_half")}.items() if v is not None},
        },
        "wall_s_timed": wall, "source_hash": hsh,
    }
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_host(wl, T, args.cpu_reps)
    print(json.dumps(out), flush=True)


def cpu_baseline_train(wl, T, reps):
    """The training oracle as it stands (dX = G W_nm and the packed dW, fp64) on
    the first 2048 tokens of G and act (all of them at the workload's size),
    scaled to all T: both products are linear in the token count."""
    from oracle import nm_oracle as O
    from oracle import nm_train as TR
    n, m = wl.patterns[0]
    ts = min(T, 2048)
    vals, idx = O.prune_pack(wl.weights(), n, m)
    g = wl.gradient(T)[:ts]
    act = wl.activations(T)[:ts]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        TR.spmm_dx_ref(vals, idx, wl.K, n, m, g, wl.dtype)
        TR.spmm_dw_ref(idx, wl.K, n, m, g, act, wl.dtype)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times) * T / ts
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"value": 2.0 * 2.0 * wl.R * wl.K * T / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"{wl.R}x{wl.K}x{T} {n}:{m} dX and packed dW: fp64 decompress + G W_nm, G^T act "
                       f"sampled at the stored columns, over the first {ts} of {T} tokens, scaled; "
                       f"median of {reps} runs")}


def bench_train(args, wl):
    """Training-side products of a fixed-pattern layer: one step = nm_spmm_dx
    (dX = G W_nm from the packed weight) + nm_spmm_dw (dW at the stored
    positions, packed), the weight already packed."""
    import numpy as np
    import torch

    import structured_sparse_gemm_nm_amd as nm

    R, K = wl.R, wl.K
    T = args.T if args.T is not None else wl.Ts[0]
    n, m = wl.patterns[0]
    S = K // m * n
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
    out_dtype = torch.float32 if args.out_dtype == "f32" else tdt
    out_name = args.out_dtype

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

    W = dev(wl.weights())
    act = dev(wl.activations(T))
    G = dev(wl.gradient(T))
    vals, idx = nm.nm_compress(W, n, m)
    dX = torch.empty((T, K), dtype=out_dtype, device="cuda")
    dW = torch.empty((R, S), dtype=out_dtype, device="cuda")

    def dx(_c=0):
        nm.nm_spmm_dx(vals, idx, G, K, n, m, out_dtype=out_dtype, out=dX)

    def dw(_c=0):
        nm.nm_spmm_dw(idx, G, act, K, n, m, out_dtype=out_dtype, out=dW)

    settle = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    tw = time.perf_counter()
    while (time.perf_counter() - tw) * 1e3 < args.settle_ms:
        for _ in range(8):
            torch.matmul(settle, settle)
        torch.cuda.synchronize()
    del settle
    for _ in range(args.warmup):
        dx()
        dw()
    torch.cuda.synchronize()
    # the timed steps run their dX products first, then their dW products, so
    # each kernel's mean comes from events around its own phase
    t0 = time.perf_counter()
    start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    start.record()
    for _ in range(args.steps):
        dx()
    mid.record()
    for _ in range(args.steps):
        dw()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    dx_us = start.elapsed_time(mid) * 1e3 / args.steps
    dw_us = mid.elapsed_time(end) * 1e3 / args.steps

    # dense hipBLASLt products of the same shapes and output dtypes: dX = G W_hat
    # (W_hat the pruned weight, dense) and the full dense dW = G^T act (G^T
    # handed over row-major), in alternating blocks with the sparse ones
    W_hat = nm.nm_decompress(vals, idx, K, n, m).contiguous()
    Gt = G.t().contiguous()
    dxh = torch.empty((T, K), dtype=tdt, device="cuda")
    dwh = torch.empty((R, S), dtype=tdt, device="cuda")
    loops = {"dx": dx, "dw": dw,
             "dx_half": lambda c: nm.nm_spmm_dx(vals, idx, G, K, n, m, out_dtype=tdt, out=dxh),
             "dw_half": lambda c: nm.nm_spmm_dw(idx, G, act, K, n, m, out_dtype=tdt, out=dwh),
             "dense_dx_half": lambda c: torch.mm(G, W_hat),
             "dense_dx_f32": lambda c: torch.mm(G, W_hat, out_dtype=torch.float32),
             "dense_dw_half": lambda c: torch.mm(Gt, act),
             "dense_dw_f32": lambda c: torch.mm(Gt, act, out_dtype=torch.float32)}
    iters = max(20, args.steps)
    for name in list(loops):
        try:
            for _ in range(3):
                loops[name](0)
            torch.cuda.synchronize()
        except RuntimeError as e:
            print(f"{name} unavailable: {e}", file=sys.stderr)
            del loops[name]
    samples = {name: [] for name in loops}
    for _ in range(5):
        for name, fn in loops.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(iters):
                fn(0)
            b.record()
            torch.cuda.synchronize()
            samples[name].append(a.elapsed_time(b) * 1e3 / iters)
    loop_us = {name: float(np.median(v)) for name, v in samples.items()}

    def ratio(x, y):
        return loop_us[x] / loop_us[y] if x in loop_us and y in loop_us else None

    # algorithmic FLOP: one MAC per (token, stored weight) in each product; the
    # MFMA work of both kernels is the dense 2 R K T (neither product can skip
    # the zeros: in dX they do not lie along the reduction, in dW they are outputs)
    alg_flop = 2.0 * T * R * S
    mfma_flop = 2.0 * T * R * K
    dense_eq_flop = 2.0 * 2.0 * R * K * T
    ob = 4 if out_name == "f32" else 2
    hsh = kernel_source_hash("train")
    _, ib, _ = nm.nm_packed_sizes(R, K, n, m, nm.NM_BF16 if wl.dtype == "bf16" else nm.NM_F16)
    per = {"nm_spmm_dx": {"mean_us": dx_us, "flop": alg_flop, "mfma_flop": mfma_flop,
                          "bytes": R * S * 2 + ib + T * R * 2 + T * K * ob},
           "nm_spmm_dw": {"mean_us": dw_us, "flop": alg_flop, "mfma_flop": mfma_flop,
                          "bytes": ib + T * R * 2 + T * K * 2 + R * S * ob}}
    dom = max(per, key=lambda k: per[k]["mean_us"])
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    achieved = per[dom]["flop"] / (per[dom]["mean_us"] * 1e-6) / 1e12
    key = "dx" if dom == "nm_spmm_dx" else "dw"
    roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": traffic_from_profile(f"train_{key}_w{wl.wid}_T{T}_{out_name}", hsh),
                "kernel": dom, "per_launch": per[dom],
                "mfma_frac": per[dom]["mfma_flop"] / (per[dom]["mean_us"] * 1e-6) / 1e12 / peak}
    out = {
        "metric": METRIC, "value": dense_eq_flop / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,sigma) W, act and G of the workload's shapes)",
        "config": {"workload": wl.name, "R": R, "K": K, "T": T, "pattern": f"{n}:{m}", "out_dtype": out_name,
                   "step": "nm_spmm_dx + nm_spmm_dw", "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {
            "nm_spmm_dx_us_in_step": dx_us, "nm_spmm_dw_us_in_step": dw_us,
            "per_launch": per,
            "nm_spmm_dx_us_loop": loop_us.get("dx"), "nm_spmm_dw_us_loop": loop_us.get("dw"),
            "nm_spmm_dx_half_out_us": loop_us.get("dx_half"), "nm_spmm_dw_half_out_us": loop_us.get("dw_half"),
            "dense_dx_half_out_us": loop_us.get("dense_dx_half"), "dense_dx_f32_out_us": loop_us.get("dense_dx_f32"),
            "dense_dw_half_out_us": loop_us.get("dense_dw_half"), "dense_dw_f32_out_us": loop_us.get("dense_dw_f32"),
            "speedup_vs_dense_same_out_dtype": {k: v for k, v in {
                "dx_f32": ratio("dense_dx_f32", "dx") if out_name == "f32" else None,
                "dw_f32": ratio("dense_dw_f32", "dw") if out_name == "f32" else None,
                "dx_half": ratio("dense_dx_half", "dx_half"),
                "dw_half": ratio("dense_dw_half", "dw_half")}.items() if v is not None},
        },
        "wall_s_timed": wall, "source_hash": hsh,
    }
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
    if not args.no_peaks:
        pk = measured_peaks(torch)
        out["measured_peaks"] = pk
        roofline["frac_of_measured_dense_matmul"] = roofline["achieved"] / pk["dense_bf16_matmul_tflops"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_train(wl, T, args.cpu_reps)
    print(json.dumps(out), flush=True)


def _hybrid_dense_operand(nm, torch, W, L, flags, tdt):
    """W_hat^T [K, R] row-major for the dense reference GEMM: the weight as the
    hybrid pruning leaves it.  Dense tiles are W itself; a 2:4 tile keeps what
    the row-wise 2:4 pruning of W keeps on its columns (the same selection, as
    the GPU tests check bit for bit), so W_hat = where(dense tile, W,
    decompress(compress(W))).  Three launches, on the GPU."""
    import numpy as np
    R, K, tr, tc = L.R, L.K, L.tile_rows, L.tile_cols
    v24, i24 = nm.nm_compress(W, 2, 4)
    pruned = nm.nm_decompress(v24, i24, K, 2, 4)
    f = torch.from_numpy(np.ascontiguousarray(flags, dtype=np.bool_)).to(W.device)
    mask = f.repeat_interleave(tr, dim=0)[:R].repeat_interleave(tc, dim=1)
    return torch.where(mask, W, pruned).t().contiguous()


def copy_calibration(torch):
    """One plain 256 MiB device copy: the dispatch a counter profile of the
    same command scales its HBM byte counters against."""
    src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    return src.numel() * 4


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
    if args.print_source_hash:
        print(kernel_source_hash(args.print_source_hash))
        return
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
    if wl.hybrid:
        bench_hybrid(args, wl)
        return
    if wl.train:
        bench_train(args, wl)
        return
    if wl.host:
        bench_host(args, wl)
        return
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
    var = args.variant

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

    # the permuted product's workspace (the gather pass writes X' = act[:, perm]
    # there), allocated once like the outputs
    ws_need = nm.nm_spmm_perm_workspace_size(R, K, T, n, m, dcode) if perm is not None else 0
    ws = torch.empty(ws_need, dtype=torch.uint8, device="cuda") if ws_need else None

    def gemm(c):
        _, Ac, vals, idx, Y = copies[c]
        if perm is None:
            nm.nm_spmm(vals, idx, Ac, K, n, m, out_dtype=out_dtype, out=Y, variant=var)
        else:
            nm.nm_spmm_perm(vals, idx, Ac, perm, K, n, m, out_dtype=out_dtype, out=Y, variant=var, workspace=ws)

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

    # ---- per-kernel breakdown.  Each kernel is timed over blocks of `iters`
    # back-to-back launches, and the blocks of all kernels alternate round
    # robin (five rounds, median per kernel): a kernel timed right after a long
    # run of another one (a dense GEMM heats the chip and lowers its clock)
    # would otherwise carry that other kernel's after-effects.
    dense = []
    for c in range(rotate):
        dense.append(nm.nm_decompress(copies[c][2], copies[c][3], K, n, m))
    actp = [copies[c][1] if perm is None else copies[c][1][:, perm.long()].contiguous()
            for c in range(rotate)]
    # W^T as its own row-major [K, R] tensor (no transposed views in the dense calls)
    dense_t = [d.t().contiguous() for d in dense]

    loops = {"gemm": gemm, "compress": compress}
    if i8:
        # dense int8 GEMM with an int32 result (hipBLASLt through torch._int_mm)
        loops["dense_same_out"] = lambda c: torch._int_mm(actp[c], dense_t[c])
    elif f8:
        # dense fp8 GEMM with an fp32 result (hipBLASLt through torch._scaled_mm, unit scales;
        # its second operand must be column-major: the [K, R] view of the row-major W)
        one = torch.ones((), dtype=torch.float32, device="cuda")
        loops["dense_same_out"] = lambda c: torch._scaled_mm(actp[c], dense[c].t(), scale_a=one, scale_b=one,
                                                             out_dtype=torch.float32)
    else:
        y_half = torch.empty((T, R), dtype=tdt, device="cuda")

        def gemm_half(c):
            _, Ac, vals, idx, _ = copies[c]
            if perm is None:
                nm.nm_spmm(vals, idx, Ac, K, n, m, out_dtype=tdt, out=y_half, variant=var)
            else:
                nm.nm_spmm_perm(vals, idx, Ac, perm, K, n, m, out_dtype=tdt, out=y_half, variant=var,
                                workspace=ws)

        loops["gemm_half"] = gemm_half
        # dense GEMMs (hipBLASLt through torch) with the same output dtypes:
        # a half-precision result, and an fp32 one
        loops["dense_half"] = lambda c: torch.mm(actp[c], dense_t[c])
        loops["dense_f32"] = lambda c: torch.mm(actp[c], dense_t[c], out_dtype=torch.float32)
    if perm is not None:
        y_plain = torch.empty((T, R), dtype=out_dtype, device="cuda")
        ident = torch.arange(K, dtype=torch.int32, device="cuda")

        def plain(c):
            _, Ac, vals, idx, _ = copies[c]
            nm.nm_spmm(vals, idx, Ac, K, n, m, out_dtype=out_dtype, out=y_plain, variant=var)

        def identity(c):
            _, Ac, vals, idx, _ = copies[c]
            nm.nm_spmm_perm(vals, idx, Ac, ident, K, n, m, out_dtype=out_dtype, out=y_plain, variant=var,
                            workspace=ws)

        def in_kernel(c):
            _, Ac, vals, idx, _ = copies[c]
            nm.nm_spmm_perm(vals, idx, Ac, perm, K, n, m, out_dtype=out_dtype, out=y_plain, variant=var,
                            workspace=None)

        loops.update({"no_perm": plain, "identity_perm": identity, "perm_no_workspace": in_kernel})

    iters = max(20, args.steps)
    for name in list(loops):  # drop what this build of torch cannot run for the shape
        try:
            for i in range(3):
                loops[name](i % rotate)
            torch.cuda.synchronize()
        except RuntimeError as e:
            print(f"{name} unavailable: {e}", file=sys.stderr)
            del loops[name]
    samples = {name: [] for name in loops}
    for _ in range(5):
        for name, fn in loops.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(iters):
                fn(i % rotate)
            b.record()
            torch.cuda.synchronize()
            samples[name].append(a.elapsed_time(b) * 1e3 / iters)
    loop_us = {name: float(np.median(v)) for name, v in samples.items()}
    gemm_loop_us = loop_us["gemm"]
    compress_us = loop_us["compress"]
    gemm_half_us = loop_us.get("gemm_half")

    def ratio(a, b):
        return loop_us[a] / loop_us[b] if a in loop_us and b in loop_us else None

    if b8:
        speedup = {out_name: ratio("dense_same_out", "gemm")}
        dense_keys = {f"dense_{out_name}_out_us": loop_us.get("dense_same_out")}
    else:
        speedup = {out_name: ratio("dense_half" if out_name != "f32" else "dense_f32", "gemm"),
                   "half": ratio("dense_half", "gemm_half"),
                   "f32": ratio("dense_f32", "gemm") if out_name == "f32" else None}
        speedup = {k: v for k, v in speedup.items() if v is not None}
        dense_keys = {"dense_half_out_us": loop_us.get("dense_half"),
                      "dense_f32_out_us": loop_us.get("dense_f32")}

    dense_eq_flop = 2.0 * R * K * T
    alg_flop = 2.0 * R * S * T
    achieved_tflops = alg_flop / (gemm_mean_us * 1e-6) / 1e12
    hsh = kernel_source_hash("spmm")
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
        extra = {"nm_spmm_no_perm_us": loop_us.get("no_perm"),
                 "nm_spmm_perm_identity_us": loop_us.get("identity_perm"),
                 "nm_spmm_perm_no_workspace_us": loop_us.get("perm_no_workspace"),
                 "perm_overhead_vs_no_perm": ratio("gemm", "no_perm") - 1.0,
                 "perm_overhead_vs_identity_perm": ratio("gemm", "identity_perm") - 1.0}

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
            **dense_keys,
            # dense time / sparse time, both sides writing the same output dtype
            "speedup_vs_dense_same_out_dtype": speedup,
            **extra,
        },
        "wall_s_timed": wall,
        "source_hash": hsh,
    }
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
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
