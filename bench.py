"""Benchmark of the FP8 / 2:4-sparse GEMM layers on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only gemm] [--copy-calibration]

The timed step is one forward pass of the 2:4-sparse FP8 linear layer at
M = 2048, N = K = 4096 with inputs already resident in HBM: quantise the
fp32 activations to e4m3 with one scale per (row, 128-wide K block), then the
2:4-sparse FP8 groupwise GEMM (weight pre-pruned, compressed and quantised with
128 x 128 block scales) with its fused dequantisation and bf16 epilogue.
``value`` is the dense-equivalent throughput 2 M N K / step time.  Every other
row of the hot path (weight preparation, the dense GEMM, both output forms,
the decode shapes, the fused int4 + bf16 add) is timed in the same run and
reported under ``rows``.

``roofline`` describes the sparse GEMM kernel: its dense-equivalent FLOPs per
launch over its average launch time, taken with HIP events on the stream it
runs on, against MI355X's dense FP8 MFMA peak.  ``traffic`` comes from the
committed rocprofv3 counter summary when it was taken on the current kernel
source, else null.  ``cpu_baseline`` times the CPU oracle on the same workload.

One process, one GPU: ``--gpus`` above 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_gemm_layers_amd as sg  # noqa: E402
import workloads  # noqa: E402

METRIC = "dense-equiv FP8 TFLOP/s @M=2048 N=K=4096 2:4 W; % MFMA peak; M=16 GB/s"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_INT8_TOPS = 5000.0
PEAK_HBM_GBS = 8000.0
GEMM_SRC = os.path.join(ROOT, "sparse_gemm_layers_amd", "csrc", "gemm_fp8.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_gemm_2048x4096x4096_traffic.txt")
DEV = torch.device("cuda:0")
ROTATE = 8          # input sets cycled through in the headline loop (> MALL)
ROTATE_DECODE = 16  # weight copies cycled through in the decode rows
SLEEP_CYCLES = 4_000_000   # about 2 ms of GPU sleep ahead of a timed batch


def sparse_bytes(m, n, k, out_bytes=2):
    """Algorithmic bytes of the 2:4 GEMM: values K/2 and metadata K/8 per W row,
    W scales, X codes, X scales, Y."""
    return n * k // 2 + n * k // 8 + 4 * (-(-n // 128)) * (k // 128) + m * k + 4 * m * (k // 128) + m * n * out_bytes


def dense_bytes(m, n, k, out_bytes=2):
    return n * k + 4 * (-(-n // 128)) * (k // 128) + m * k + 4 * m * (k // 128) + m * n * out_bytes


def gen_layer(seed, m, n, k, on_gpu_rng=False):
    """fp32 X on the GPU and the prepared 2:4 weight (values, metadata, scales)."""
    if on_gpu_rng:
        g = torch.Generator(device=DEV)
        g.manual_seed(seed)
        x = torch.randn((m, k), generator=g, device=DEV)
        w = torch.randn((n, k), generator=g, device=DEV) * 0.02
    else:
        d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
        x, w = torch.from_numpy(d["x"]).to(DEV), torch.from_numpy(d["w"]).to(DEV)
    wv, meta = sg.sparse24_prune_compress(w)
    wq, sw = sg.fp8_quant_groupwise(wv, gr=128, gc=64)
    wp = sg.sparse24_pack_gfx950(wq, meta)
    return x, wq, meta, sw, wp


def time_fn(fn, reps=50, warm=5):
    """Mean GPU time of one call: `reps` calls are queued back to back behind a
    short GPU sleep (so that the host's launch cost, which exceeds the run time
    of the small kernels, stays outside the timed interval) and timed with one
    pair of HIP events; gaps between the kernels are included."""
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    torch.cuda._sleep(SLEEP_CYCLES)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(reps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def headline(steps, warmup):
    m, n, k = 2048, 4096, 4096
    sets = [gen_layer(3, m, n, k)] + [gen_layer(1000 + i, m, n, k, on_gpu_rng=True) for i in range(ROTATE - 1)]
    xq = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    sx = torch.empty((k // 128, m), dtype=torch.float32, device=DEV).t()
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def step(i):
        x, _, _, sw, wp = sets[i % ROTATE]
        sg.fp8_quant_groupwise(x, gr=1, gc=128, q=xq, s=sx)
        sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, wp, n, sw, 1, 128, y=y)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # The GEMM alone, launched back to back over the same rotating sets (X
    # quantised once per set): its mean launch duration, for the roofline.
    xqs = [sg.fp8_quant_groupwise(sets[i][0], gr=1, gc=128) for i in range(ROTATE)]
    gemm_ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed(
        xqs[i % ROTATE][0], xqs[i % ROTATE][1], sets[i % ROTATE][4], n, sets[i % ROTATE][3], 1, 128, y=y),
        reps=steps, warm=warmup)
    del xqs
    flops = 2.0 * m * n * k
    return {"ms_per_step": ms_step, "value": flops / (ms_step * 1e-3) / 1e12, "gemm_ms": gemm_ms,
            "gemm_tflops": flops / (gemm_ms * 1e-3) / 1e12, "m": m, "n": n, "k": k}


def rows_report():
    out = {}
    m, n, k = 2048, 4096, 4096
    x, wq, meta, sw, wp = gen_layer(3, m, n, k)
    w = torch.from_numpy(workloads.sparse_large(seed=3, m=8, n=n, k=k)["w"]).to(DEV)
    xq, sx = sg.fp8_quant_groupwise(x)
    # a1: activation quantisation (fp32 in, e4m3 + scales out)
    ms = time_fn(lambda i: sg.fp8_quant_groupwise(x, q=xq, s=sx))
    b = m * k * 4 + m * k + 4 * m * (k // 128)
    out["a1_quant_x_2048x4096"] = {"ms": ms, "GB/s": b / ms / 1e6}
    # a2 / a3: weight preparation
    wv = torch.empty((n, k // 2), dtype=torch.float32, device=DEV)
    mt = torch.empty((n, k // 8), dtype=torch.uint8, device=DEV)
    ms = time_fn(lambda i: sg.sparse24_prune_compress(w, vals=wv, meta=mt))
    b = n * k * 4 + n * k // 2 * 4 + n * k // 8
    out["a2_prune_compress_4096x4096"] = {"ms": ms, "GB/s": b / ms / 1e6}
    q = torch.empty((n, k // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((k // 128, n // 128), dtype=torch.float32, device=DEV).t()
    ms = time_fn(lambda i: sg.fp8_quant_groupwise(wv, gr=128, gc=64, q=q, s=s))
    b = n * k // 2 * 4 + n * k // 2 + 4 * (n // 128) * (k // 128)
    out["a3_quant_w_4096x2048_128x64"] = {"ms": ms, "GB/s": b / ms / 1e6}
    # packing the compressed weight into the gfx950 layout
    wpk = torch.empty_like(wp)
    ms = time_fn(lambda i: sg.sparse24_pack_gfx950(wq, meta, packed=wpk))
    b = n * k // 2 + n * k // 8 + wp.numel()
    out["a3b_pack_gfx950_4096x4096"] = {"ms": ms, "GB/s": b / ms / 1e6}
    # a5 + a6: sparse GEMM, both output forms, packed weight; and the canonical form
    flops = 2.0 * m * n * k
    for form in ("y", "yt"):
        y = torch.empty((m, n) if form == "y" else (n, m), dtype=torch.bfloat16, device=DEV)
        ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, wp, n, sw, 1, 128, form=form, y=y))
        out[f"a5_sparse_gemm_packed_2048x4096x4096_{form}"] = {
            "ms": ms, "TFLOP/s": flops / ms / 1e9, "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise(xq, sx, wq, meta, sw, 1, 128, y=y))
    out["a5_sparse_gemm_canonical_2048x4096x4096_y"] = {
        "ms": ms, "TFLOP/s": flops / ms / 1e9, "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    # a4: dense GEMM with outliers
    d = workloads.dense_outliers(seed=2, m=m, n=n, k=k)
    xd, wd = torch.from_numpy(d["x"]).to(DEV), torch.from_numpy(d["w"]).to(DEV)
    xdq, sxd = sg.fp8_quant_groupwise(xd)
    wdq, swd = sg.fp8_quant_groupwise(wd, gr=128, gc=128)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.fp8_gemm_groupwise(xdq, sxd, wdq, swd, 1, 128, y=y))
    out["a4_dense_gemm_2048x4096x4096"] = {"ms": ms, "TFLOP/s": flops / ms / 1e9,
                                           "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    del xd, wd, xdq, wdq
    # decode shapes, rotating weight copies so the 256 MB MALL cannot serve repeats
    for (dm, dn, dk) in workloads.DECODE_SHAPES:
        wsets = [gen_layer(2000 + i, 8, dn, dk, on_gpu_rng=True)[3:] for i in range(ROTATE_DECODE)]
        xdd = torch.from_numpy(workloads.decode(seed=4, m=dm, n=8, k=dk)["x"]).to(DEV)
        xq4, sx4 = sg.fp8_quant_groupwise(xdd)
        for form in ("y", "yt"):
            y = torch.empty((dm, dn) if form == "y" else (dn, dm), dtype=torch.bfloat16, device=DEV)
            ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed(
                xq4, sx4, wsets[i % ROTATE_DECODE][1], dn, wsets[i % ROTATE_DECODE][0], 1, 128, form=form, y=y),
                reps=64, warm=16)
            b = sparse_bytes(dm, dn, dk)
            out[f"decode_M{dm}_N{dn}_K{dk}_{form}"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                     "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
        del wsets
    # a7: fused int4 + bf16 add at L=2048, D1=4096, D2=64, D=4096
    dd = workloads.mixed_add(seed=5)
    x1, sx1 = sg.int4_quant_groupwise(torch.from_numpy(dd["x1"]).to(DEV))
    w1, sw1 = sg.int4_quant_groupwise(torch.from_numpy(dd["w1"]).to(DEV))
    x2 = torch.from_numpy(dd["x2"].view(np.int16)).to(DEV).view(torch.bfloat16)
    w2 = torch.from_numpy(dd["w2"].view(np.int16)).to(DEV).view(torch.bfloat16)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.mixed_gemm_add(x1, sx1, w1, sw1, x2, w2, y=y))
    ops = 2.0 * m * n * 4096 + 2.0 * m * n * 64
    out["a7_mixed_add_2048x4096x(4096+64)"] = {"ms": ms, "TOP/s": ops / ms / 1e9,
                                                "frac_int8_peak": ops / ms / 1e9 / PEAK_INT8_TOPS}
    return out


def cpu_baseline(min_seconds=8.0):
    import oracle
    from threadpoolctl import threadpool_info
    m, n, k = 2048, 4096, 4096
    d = workloads.sparse_large(seed=3, m=m, n=n, k=k)
    wv32, meta = oracle.prune_compress24(d["w"])
    wq, sw = oracle.fp8_quant_groupwise(wv32, 128, 64)
    xq, sx = oracle.fp8_quant_groupwise(d["x"], 1, 128)
    times = []
    t_all = time.perf_counter()
    while True:
        t = time.perf_counter()
        oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128)
        times.append(time.perf_counter() - t)
        if time.perf_counter() - t_all >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": 2.0 * m * n * k / float(np.mean(times)) / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full 2048x4096x4096 2:4 GEMM (fp64 NumPy oracle, {len(times)} runs, "
                      f"{np.mean(times):.2f} s each; quantisation/pruning done beforehand, untimed)"}


def traffic_from_profile():
    """HBM bytes per launch of the sparse GEMM from the committed counter
    summary, only if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != src:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE/WRITE_SIZE counters."""
    nbytes = 512 << 20
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["gemm"], default=None,
                    help="run only the headline loop (for counter collection)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs every kernel on a single MI355X "
              "and has no multi-GPU path (see how it would shard in the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    sg.lib()
    h = headline(args.steps, args.warmup)
    if args.only == "gemm":
        print(json.dumps({"headline": h}))
        return
    rows = rows_report()
    achieved = h["gemm_tflops"]
    tb = traffic_from_profile()
    line = {
        "metric": METRIC,
        "value": round(h["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {
            "workload": "2:4-sparse FP8 linear layer forward: fp32 X[2048,4096] quantised to e4m3 (1x128 "
                        "scales), W[4096,4096] pruned 2:4 + e4m3 (128x128 scales) in the gfx950 packed form, "
                        "Y=X.W^T bf16",
            "M": h["m"], "N": h["n"], "K": h["k"], "rotated_input_sets": ROTATE,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": tb,
            "kernel": "k_gemm_sparse_x2<packed> (2:4 FP8 GEMM, Y form)", "avg_launch_ms": round(h["gemm_ms"], 5),
        },
        "rows": {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in rows.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
