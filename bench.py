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
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# the sources the sparse GEMM kernel is compiled from (a change voids the recorded traffic)
# the sparse GEMM's sources and the build script (its compile flags shape the kernel too)
GEMM_SRCS = [os.path.join(ROOT, "sparse_gemm_layers_amd", "csrc", f)
             for f in ("gemm_fp8.hip", "gemm_common.h", "tile_epilogue.h", "common.h")] + \
            [os.path.join(ROOT, "sparse_gemm_layers_amd", "build.py")]
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


def k_constant(s, rows, k):
    """Scales s [rows] repeated over every 128-wide K block (K-block stride 0)."""
    return s[:, None].expand(rows, k // 128)


# Row markers for counter runs (--markers): before each timed row one launch
# of the streaming-read probe with 1000 + (row number) workgroups, after it
# one with 3000 + (row number), which the counter summary uses to take each
# row's own dispatches (not the set-up of the next row).
MARKERS = {"on": False, "n": 0, "buf": None, "sink": None}


def _mark_row():
    if not MARKERS["on"]:
        return
    if MARKERS["buf"] is None:
        MARKERS["buf"] = torch.zeros(16, dtype=torch.uint8, device=DEV)
        MARKERS["sink"] = torch.empty(4096 * 256, dtype=torch.float32, device=DEV)
    MARKERS["n"] += 1
    sg.probe_stream_read(MARKERS["buf"], 1000 + MARKERS["n"], MARKERS["sink"])
    print(f"row {MARKERS['n']}", file=sys.stderr, flush=True)   # progress of long counter runs


def _end_row():
    if MARKERS["on"]:
        sg.probe_stream_read(MARKERS["buf"], 3000 + MARKERS["n"], MARKERS["sink"])


def time_fn(fn, reps=50, warm=5):
    """Mean GPU time of one call: `reps` calls are queued back to back behind a
    short GPU sleep (so that the host's launch cost, which exceeds the run time
    of the small kernels, stays outside the timed interval) and timed with one
    pair of HIP events; gaps between the kernels are included."""
    _mark_row()
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
    _end_row()
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
    wq_dense = wdq
    del xd, wd, xdq
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
        # next row: the activation quantisation fused into the GEMM, against
        # quantise-then-GEMM (two launches); fp32 X in, bf16 Y out
        y = torch.empty((dm, dn), dtype=torch.bfloat16, device=DEV)
        bq = sparse_bytes(dm, dn, dk) - dm * dk - 4 * dm * (dk // 128) + 4 * dm * dk   # X read as fp32
        ms = time_fn(lambda i: sg.fp8_sparse24_gemm_packed_quant_x(
            xdd, wsets[i % ROTATE_DECODE][1], dn, wsets[i % ROTATE_DECODE][0], 128, y=y), reps=64, warm=16)
        out[f"next_fused_quant_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": bq / ms / 1e6,
                                                               "frac_hbm": bq / ms / 1e6 / PEAK_HBM_GBS}

        def separate(i):
            sg.fp8_quant_groupwise(xdd, q=xq4, s=sx4)
            sg.fp8_sparse24_gemm_groupwise_packed(xq4, sx4, wsets[i % ROTATE_DECODE][1], dn,
                                                  wsets[i % ROTATE_DECODE][0], 1, 128, y=y)
        ms = time_fn(separate, reps=64, warm=16)
        out[f"next_quant_then_gemm_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": bq / ms / 1e6,
                                                                   "frac_hbm": bq / ms / 1e6 / PEAK_HBM_GBS}
        del wsets
    # one GPU's share of an 8-way tensor-parallel layer (column-parallel
    # up-projection N = 14336 / 8, bf16 out; row-parallel down-projection
    # K = 14336 / 8, fp32 partial out), 64 weight copies (> 256 MB MALL)
    for (dm, dn, dk, odt) in ((16, 1792, 4096, torch.bfloat16), (16, 4096, 1792, torch.float32)):
        wsets = [gen_layer(2500 + i, 8, dn, dk, on_gpu_rng=True)[3:] for i in range(64)]
        xdd = torch.from_numpy(workloads.decode(seed=4, m=dm, n=8, k=dk)["x"]).to(DEV)
        xq4, sx4 = sg.fp8_quant_groupwise(xdd)
        y = torch.empty((dm, dn), dtype=odt, device=DEV)
        ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed(
            xq4, sx4, wsets[i % 64][1], dn, wsets[i % 64][0], 1, 128, y=y), reps=128, warm=64)
        b = sparse_bytes(dm, dn, dk, out_bytes=2 if odt == torch.bfloat16 else 4)
        out[f"tp8_share_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                       "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
        del wsets
    # next row: int8 x int8 2:4 GEMM, packed weight, 2048x4096x4096 and the M=16 decode shape
    d = workloads.sparse_large(seed=3, m=m, n=n, k=k)
    wv8, mt8 = sg.sparse24_prune_compress(torch.from_numpy(d["w"]).to(DEV))
    wq8, sw8 = sg.int8_quant_groupwise(wv8, gr=128, gc=64)
    wp8 = sg.sparse24_pack_gfx950(wq8, mt8)
    xq8, sx8 = sg.int8_quant_groupwise(torch.from_numpy(d["x"]).to(DEV))
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.int8_sparse24_gemm_groupwise_packed(xq8, sx8, wp8, n, sw8, 1, 128, y=y))
    out["next_int8_sparse_gemm_packed_2048x4096x4096_y"] = {
        "ms": ms, "TOP/s": flops / ms / 1e9, "frac_int8_peak": flops / ms / 1e9 / PEAK_INT8_TOPS}
    del wv8, mt8, wq8, wp8
    dm, dn, dk = 16, 14336, 4096
    wsets = []
    for i in range(ROTATE_DECODE):
        g = torch.Generator(device=DEV)
        g.manual_seed(3000 + i)
        wr = torch.randn((dn, dk), generator=g, device=DEV) * 0.02
        v, mt = sg.sparse24_prune_compress(wr)
        q8, s8 = sg.int8_quant_groupwise(v, gr=128, gc=64)
        wsets.append((s8, sg.sparse24_pack_gfx950(q8, mt)))
        del wr, v, mt, q8
    xq16, sx16 = sg.int8_quant_groupwise(torch.from_numpy(workloads.decode(seed=4, m=dm, n=8, k=dk)["x"]).to(DEV))
    y = torch.empty((dm, dn), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.int8_sparse24_gemm_groupwise_packed(
        xq16, sx16, wsets[i % ROTATE_DECODE][1], dn, wsets[i % ROTATE_DECODE][0], 1, 128, y=y), reps=64, warm=16)
    b = sparse_bytes(dm, dn, dk)
    out[f"next_int8_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    del wsets
    # next row: scales constant along K (rowwise), applied once after the K
    # loop, 2048x4096x4096 packed 2:4 and dense; and the batched ("L" mode)
    # 2:4 GEMM, 8 problems of 256x4096x4096 with distinct packed weights
    xqr = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    sxq = torch.empty((1, m), dtype=torch.float32, device=DEV).t()
    ms = time_fn(lambda i: sg.fp8_quant_groupwise(x, gr=1, gc=k, q=xqr, s=sxq))
    b = m * k * 4 + m * k + 4 * m
    out["next_rowwise_quant_x_2048x4096"] = {"ms": ms, "GB/s": b / ms / 1e6}
    st = torch.empty((1, 1), dtype=torch.float32, device=DEV)
    ms = time_fn(lambda i: sg.fp8_quant_groupwise(x, gr=m, gc=k, q=xqr, s=st))
    out["next_tensorwise_quant_x_2048x4096"] = {"ms": ms, "GB/s": (m * k * 4 + m * k + 4) / ms / 1e6}
    del xqr
    sxr = k_constant(sx[:, 0].contiguous(), m, k)
    swr = k_constant(sw[:, 0].repeat_interleave(128)[:n].contiguous(), n, k)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed(xq, sxr, wp, n, swr, 1, 1, y=y))
    out["next_rowwise_sparse_gemm_packed_2048x4096x4096_y"] = {
        "ms": ms, "TFLOP/s": flops / ms / 1e9, "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    ms = time_fn(lambda i: sg.fp8_gemm_groupwise(xq, sxr, wq_dense, swr, 1, 1, y=y))
    out["next_rowwise_dense_gemm_2048x4096x4096"] = {
        "ms": ms, "TFLOP/s": flops / ms / 1e9, "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    del wq_dense
    L, bm = 8, 256
    bsets = [gen_layer(4000 + i, 8, n, k, on_gpu_rng=True) for i in range(L)]
    wpb = torch.stack([b_[4] for b_ in bsets])
    swb = torch.stack([b_[3] for b_ in bsets])
    del bsets
    xb = xq[:L * bm].view(L, bm, k)
    sxb = torch.empty((L, k // 128, bm), dtype=torch.float32, device=DEV).transpose(1, 2)
    sxb.copy_(sx[:L * bm].view(L, bm, k // 128))
    yb = torch.empty((L, bm, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed_batched(xb, sxb, wpb, n, swb, 1, 128, y=yb))
    out[f"next_batched_sparse_gemm_packed_L{L}_{bm}x{n}x{k}_y"] = {
        "ms": ms, "TFLOP/s": flops / ms / 1e9, "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    # grouped: 8 groups of different M (summing to 2048 rows), one packed weight each
    sizes = [400, 120, 310, 256, 64, 380, 218, 300]
    ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed_grouped(xq, sx, sizes, wpb, n, swb, 128, y=y))
    out[f"next_grouped_sparse_gemm_packed_G8_ragged{m}x{n}x{k}_y"] = {
        "ms": ms, "TFLOP/s": flops / ms / 1e9, "frac_fp8_peak": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
    # grouped decode (MoE): 8 experts of at most 16 tokens each; 4 copies of
    # the 8 packed weights (4 x 84 MB) so the 256 MB MALL cannot serve repeats
    sizes = [3, 9, 16, 1, 12, 5, 16, 2]
    gm = sum(sizes)
    wrot = [wpb] + [wpb.clone() for _ in range(3)]
    yg = torch.empty((gm, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.fp8_sparse24_gemm_groupwise_packed_grouped(
        xq[:gm], sx[:gm], sizes, wrot[i % 4], n, swb, 128, y=yg), reps=64, warm=16)
    b = sum(sparse_bytes(mg, n, k) for mg in sizes if mg)
    out[f"next_grouped_decode_G8_M{gm}_N{n}_K{k}_y"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                       "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    del wpb, swb, yb, wrot, yg
    # next row: weight-only 2:4 (bf16 activations x e4m3 / int8 2:4 codes) at
    # the decode shapes (rotating weight copies) and at 2048x4096x4096
    dn, dk = 14336, 4096
    for codes in ("e4m3", "int8"):
        qf = sg.int8_quant_groupwise if codes == "int8" else sg.fp8_quant_groupwise
        wsets = []
        for i in range(ROTATE_DECODE):
            g = torch.Generator(device=DEV)
            g.manual_seed(5000 + i)
            v, mt = sg.sparse24_prune_compress(torch.randn((dn, dk), generator=g, device=DEV) * 0.02)
            q, s8 = qf(v, gr=128, gc=64)
            wsets.append((q, mt, s8))
            del v
        for dm in (16, 37, 64):
            xb = torch.from_numpy(workloads.decode(seed=4, m=dm, n=8, k=dk)["x"]).to(DEV).to(torch.bfloat16)
            y = torch.empty((dm, dn), dtype=torch.bfloat16, device=DEV)
            ms = time_fn(lambda i: sg.w8a16_sparse24_gemm_groupwise(
                xb, wsets[i % ROTATE_DECODE][0], wsets[i % ROTATE_DECODE][1], wsets[i % ROTATE_DECODE][2], 128, y=y),
                reps=64, warm=16)
            b = dn * dk // 2 + dn * dk // 8 + 4 * (dn // 128) * (dk // 128) + dm * dk * 2 + dm * dn * 2
            out[f"next_w8a16_{codes}_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                                   "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
            # the same weights in the gfx950 packed form (same bytes, same results)
            psets = [sg.sparse24_pack_gfx950(q, mt) for q, mt, _ in wsets]
            ms = time_fn(lambda i: sg.w8a16_sparse24_gemm_groupwise_packed(
                xb, psets[i % ROTATE_DECODE], dn, wsets[i % ROTATE_DECODE][2], 128, int8=codes == "int8", y=y),
                reps=64, warm=16)
            out[f"next_w8a16_{codes}_packed_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                                          "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
            del psets
        del wsets
    wsets = []
    for i in range(ROTATE_DECODE):
        g = torch.Generator(device=DEV)
        g.manual_seed(6000 + i)
        v, mt = sg.sparse24_prune_compress(torch.randn((dn, dk), generator=g, device=DEV) * 0.02)
        q4, s4 = sg.int4_quant_groupwise(v, gc=64)
        wsets.append((q4, mt, s4))
        del v
    for dm in (16, 37):
        xb = torch.from_numpy(workloads.decode(seed=4, m=dm, n=8, k=dk)["x"]).to(DEV).to(torch.bfloat16)
        y = torch.empty((dm, dn), dtype=torch.bfloat16, device=DEV)
        ms = time_fn(lambda i: sg.w4a16_sparse24_gemm_groupwise(
            xb, wsets[i % ROTATE_DECODE][0], wsets[i % ROTATE_DECODE][1], wsets[i % ROTATE_DECODE][2], y=y),
            reps=64, warm=16)
        b = dn * dk // 4 + dn * dk // 8 + 4 * dn * (dk // 128) + dm * dk * 2 + dm * dn * 2
        out[f"next_w4a16_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                        "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
        # the same weights in the blocked form (same bytes, same results)
        psets = [sg.sparse24_pack_w4(q4, mt) for q4, mt, _ in wsets]
        ms = time_fn(lambda i: sg.w4a16_sparse24_gemm_groupwise_packed(
            xb, psets[i % ROTATE_DECODE], dn, wsets[i % ROTATE_DECODE][2], y=y), reps=64, warm=16)
        out[f"next_w4a16_packed_decode_M{dm}_N{dn}_K{dk}_y"] = {"ms": ms, "GB/s": b / ms / 1e6,
                                                               "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
        del psets
    del wsets
    xb = x.to(torch.bfloat16)
    wv8, mt8 = sg.sparse24_prune_compress(torch.from_numpy(workloads.sparse_large(seed=3, m=8, n=n, k=k)["w"]).to(DEV))
    wq8, sw8 = sg.fp8_quant_groupwise(wv8, gr=128, gc=64)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ms = time_fn(lambda i: sg.w8a16_sparse24_gemm_groupwise(xb, wq8, mt8, sw8, 128, y=y), reps=10, warm=2)
    out["next_w8a16_e4m3_gemm_2048x4096x4096_y"] = {"ms": ms, "TFLOP/s": flops / ms / 1e9,
                                                    "frac_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
    wp8 = sg.sparse24_pack_gfx950(wq8, mt8)
    ms = time_fn(lambda i: sg.w8a16_sparse24_gemm_groupwise_packed(xb, wp8, n, sw8, 128, y=y), reps=10, warm=2)
    out["next_w8a16_e4m3_packed_gemm_2048x4096x4096_y"] = {"ms": ms, "TFLOP/s": flops / ms / 1e9,
                                                           "frac_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
    del wp8
    wq8, sw8 = sg.int8_quant_groupwise(wv8, gr=128, gc=64)
    ms = time_fn(lambda i: sg.w8a16_sparse24_gemm_groupwise(xb, wq8, mt8, sw8, 128, y=y), reps=10, warm=2)
    out["next_w8a16_int8_gemm_2048x4096x4096_y"] = {"ms": ms, "TFLOP/s": flops / ms / 1e9,
                                                    "frac_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
    q4, s4 = sg.int4_quant_groupwise(wv8, gc=64)
    ms = time_fn(lambda i: sg.w4a16_sparse24_gemm_groupwise(xb, q4, mt8, s4, y=y), reps=10, warm=2)
    out["next_w4a16_gemm_2048x4096x4096_y"] = {"ms": ms, "TFLOP/s": flops / ms / 1e9,
                                               "frac_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
    wp4 = sg.sparse24_pack_w4(q4, mt8)
    ms = time_fn(lambda i: sg.w4a16_sparse24_gemm_groupwise_packed(xb, wp4, n, s4, y=y), reps=10, warm=2)
    out["next_w4a16_packed_gemm_2048x4096x4096_y"] = {"ms": ms, "TFLOP/s": flops / ms / 1e9,
                                                      "frac_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
    del wp4
    del xb, wv8, mt8, wq8, q4, s4
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
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": 2.0 * m * n * k / float(np.mean(times)) / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "logical_cpus": os.cpu_count(),
            "scope": "the GEMM alone (the GPU value's step also quantises X; the GPU GEMM alone is "
                     "roofline.achieved)",
            "sample": f"full 2048x4096x4096 2:4 GEMM (fp64 NumPy oracle, {len(times)} runs, "
                      f"{np.mean(times):.2f} s each; quantisation/pruning done beforehand, untimed)"}


def measured_peaks():
    """What the chip sustains, next to the published peaks: each matrix-core
    instruction the kernels use (register operands, two waves per SIMD, eight
    independent chains), the shader clock during those runs, and a device copy."""
    out = {}
    sink = torch.empty(sg._binding.PROBE_WORKGROUPS * 512, dtype=torch.float32, device=DEV)
    clocks = torch.zeros(4 * sg._binding.PROBE_WORKGROUPS, dtype=torch.int64, device=DEV)
    for kind, iters in (("mfma_fp8", 2000), ("smfmac_fp8", 4000), ("mfma_i8", 4000), ("smfmac_promoted", 2000),
                        ("smfmac_rescaled", 2000), ("mfma_fp6", 4000)):
        best, ghz = None, None
        for _ in range(3):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            sg.probe_matrix_rate(kind, iters, sink, clocks)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e)
            if best is None or ms < best:
                c = clocks.cpu().numpy().reshape(-1, 4).astype(np.float64)
                ok = (c[:, 3] - c[:, 2]) > 0
                best = ms
                ghz = float(np.median((c[ok, 1] - c[ok, 0]) / (c[ok, 3] - c[ok, 2])) * 0.1)
        out[kind] = {"TFLOP/s" if kind != "mfma_i8" else "TOP/s": round(sg.probe_matrix_ops(kind, iters) / best / 1e9, 1),
                     "shader_GHz": round(ghz, 3)}
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    ms = time_fn(lambda i: b.copy_(a), reps=10, warm=2)
    out["device_copy_1GiB"] = {"GB/s": round(2 * nbytes / ms / 1e6, 1)}
    del a, b
    # a kernel that only streams (sg_probe_stream_read): the decode rows' weight
    # bytes (16 copies cycled, more than the MALL holds), the tensor-parallel
    # share rows' bytes (64 copies) and 1 GiB, timed like the rows (launch gaps
    # included)
    ssink = torch.empty(4096 * 256, dtype=torch.float32, device=DEV)
    for label, nb, copies in (("stream_read_37MB_16_copies", 37_240_000 // 16 * 16, 16),
                              ("stream_read_4.7MB_64_copies", 4_700_000 // 16 * 16, 64),
                              ("stream_read_1GiB", 1 << 30, 1)):
        bufs = [torch.empty(nb, dtype=torch.uint8, device=DEV).fill_(i + 1) for i in range(copies)]
        best = None
        for wg in (256, 512, 1024, 4096):
            ms = time_fn(lambda i: sg.probe_stream_read(bufs[i % copies], wg, ssink),
                         reps=64 if copies > 1 else 10, warm=8)
            if best is None or ms < best[0]:
                best = (ms, wg)
        out[label] = {"GB/s": round(nb / best[0] / 1e6, 1), "us": round(best[0] * 1e3, 2), "workgroups": best[1]}
        del bufs
    return out


def kernel_source_hash():
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def pmc_kib_per_dispatch(run_dir, counter, kernel_substr):
    """Mean value of one counter per dispatch of the kernels whose name
    contains kernel_substr, from a rocprofv3 --pmc database (KiB for the
    FETCH_SIZE / WRITE_SIZE derived counters)."""
    import glob
    import sqlite3
    db = sorted(glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True))[0]
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute(
        "select d.id, sum(p.value) from rocpd_pmc_event p join rocpd_kernel_dispatch d on p.event_id = d.event_id "
        "join rocpd_info_kernel_symbol s on d.kernel_id = s.id join rocpd_info_pmc i on p.pmc_id = i.id "
        "where i.name = ? and s.kernel_name like ? group by d.id", (counter, f"%{kernel_substr}%")).fetchall()
    return float(np.mean([v for _, v in rows]))


def pmc_kernel_names(run_dir, kernel_substr):
    """The distinct (demangled) names of the kernels a --pmc run measured whose
    name contains kernel_substr."""
    import glob
    import sqlite3
    db = sorted(glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True))[0]
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select distinct s.kernel_name from rocpd_kernel_dispatch d join rocpd_info_kernel_symbol s "
                       "on d.kernel_id = s.id where s.kernel_name like ?", (f"%{kernel_substr}%",)).fetchall()
    return sorted({_short(r[0]) for r in rows})


def write_traffic_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Writes the traffic file of the sparse GEMM from four counter runs (see
    its header for the commands): HBM bytes per launch, each counter scaled by
    what it reads for a plain device copy of known size."""
    kern = "k_gemm_sparse_wr"
    g_f = pmc_kib_per_dispatch(fetch_dir, "FETCH_SIZE", kern)
    g_w = pmc_kib_per_dispatch(write_dir, "WRITE_SIZE", kern)
    # the device-to-device copy (the HIP runtime's blit kernel behind tensor.copy_)
    c_f = pmc_kib_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    c_w = pmc_kib_per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    each_way_kib = (512 << 20) / 1024
    rs, ws = each_way_kib / c_f, each_way_kib / c_w
    rd, wr = round(g_f * 1024 * rs), round(g_w * 1024 * ws)   # whole bytes; the total is their sum
    m, n, k = 2048, 4096, 4096
    cmd = "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} -d <out>/prof_after/{d} -o run -- python3 -u <repo>/bench.py {a}"
    lines = [
        "# HBM traffic of the 2:4 sparse FP8 GEMM, 2048x4096x4096, packed weight, Y form, bf16 output",
        "# kernel (from the counter database): " + ", ".join(pmc_kernel_names(fetch_dir, kern)) +
        " (one launch = the whole GEMM)",
        "# FETCH_SIZE and WRITE_SIZE count the L2's traffic to and from memory behind it: L2 misses",
        "# (some of them served by the 256 MB MALL, not HBM) and write-backs; the copy calibration",
        "# converts the counts to bytes, so the figures below are an upper bound on HBM bytes",
        "# commands (from the repository root on an MI355X; one counter per run):",
        "#   " + cmd.format(c="FETCH_SIZE", d="FETCH_SIZE", a="--only gemm --steps 20 --warmup 5"),
        "#   " + cmd.format(c="WRITE_SIZE", d="WRITE_SIZE", a="--only gemm --steps 20 --warmup 5"),
        "# calibration (a plain 512 MiB device copy, same two counters):",
        "#   " + cmd.format(c="FETCH_SIZE", d="copy_FETCH_SIZE", a="--copy-calibration"),
        "#   " + cmd.format(c="WRITE_SIZE", d="copy_WRITE_SIZE", a="--copy-calibration"),
        "# this file: python bench.py --traffic-summary <out>/prof_after/{FETCH_SIZE,WRITE_SIZE,copy_FETCH_SIZE,"
        "copy_WRITE_SIZE}",
        "# counters are mean KiB per dispatch over the run's dispatches of the kernel",
        f"gemm_FETCH_SIZE_KiB: {g_f:.1f}",
        f"gemm_WRITE_SIZE_KiB: {g_w:.1f}",
        f"copy_FETCH_SIZE_KiB: {c_f:.1f}",
        f"copy_WRITE_SIZE_KiB: {c_w:.1f}",
        f"copy_bytes_each_way_KiB: {each_way_kib:.0f}",
        f"read_scale: {rs:.5f}",
        f"write_scale: {ws:.5f}",
        f"hbm_read_bytes_per_launch: {rd}",
        f"hbm_write_bytes_per_launch: {wr}",
        f"hbm_bytes_per_launch: {rd + wr}",
        f"algorithmic_bytes_per_launch: {sparse_bytes(m, n, k)}",
        "# reads are well above the algorithmic input bytes: each of the 8 XCDs' L2 fetches the X",
        "# row panels and W tiles its 32 workgroups use (4 n-tiles x 8 m-tiles per XCD)",
        f"kernel_source_sha256: {kernel_source_hash()}",
    ]
    open(TRAFFIC_FILE, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _dispatch_counters(run_dir):
    """Every kernel dispatch of a rocprofv3 --pmc run, in dispatch order:
    (kernel name, grid x, grid y, grid z, {counter: value summed over instances})."""
    import glob
    import sqlite3
    db = sorted(glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True))[0]
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute(
        "select d.id, s.kernel_name, d.grid_size_x, d.grid_size_y, d.grid_size_z, i.name, sum(p.value) "
        "from rocpd_pmc_event p join rocpd_kernel_dispatch d on p.event_id = d.event_id "
        "join rocpd_info_kernel_symbol s on d.kernel_id = s.id join rocpd_info_pmc i on p.pmc_id = i.id "
        "group by d.id, i.name order by d.id").fetchall()
    out = {}
    for did, name, gx, gy, gz, cname, v in rows:
        out.setdefault(did, [name, gx, gy, gz, {}])[4][cname] = float(v)
    return [tuple(v) for _, v in sorted(out.items())]


def _short(name):
    """Readable kernel name: demangled (c++filt, when present) without its argument list."""
    name = name[:-3] if name.endswith(".kd") else name
    if name.startswith("_Z"):
        import shutil
        import subprocess
        tool = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
        if tool:
            try:
                name = subprocess.run([tool, name], capture_output=True, text=True, timeout=10).stdout.strip() or name
            except (OSError, subprocess.SubprocessError):
                pass
    name = name.split("(")[0]
    return name[:-len(" [clone .kd]")] if name.endswith(" [clone .kd]") else name


def counter_summary(out_file, bench_json, title, command_lines, run_dirs):
    """Per benchmark row (split by the --markers probe launches) and kernel: the
    mean of every counter over the row's dispatches of that kernel, merged over
    the runs, with the derived figures used in the analysis."""
    order = json.load(open(bench_json))["row_order"]
    table = {}
    for rd in run_dirs:
        row = None
        for name, gx, gy, gz, cnt in _dispatch_counters(rd):
            if "k_probe_stream" in name and gx // 256 > 1000:
                row = order[gx // 256 - 1001] if gx // 256 < 3000 else None
                continue
            if row is None or not name.startswith("_ZN2sg"):   # the library's kernels only
                continue
            key = (row, _short(name), f"{gx}x{gy}x{gz}")
            t = table.setdefault(key, {"calls": 0, "sums": {}, "n": {}})
            for c, v in cnt.items():
                t["sums"][c] = t["sums"].get(c, 0.0) + v
                t["n"][c] = t["n"].get(c, 0) + 1
    lines = [f"# {title}", "# commands (from the repository root on an MI355X; one counter set per run):"]
    lines += ["#   " + c for c in command_lines]
    lines += ["# one line per benchmark row (its name gives the problem shape) and library kernel timed in it,",
              "# grid in work-items; means per dispatch of counters summed over hardware instances:",
              "#   mfma_util  = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs)",
              "#   valu_per_wave = SQ_INSTS_VALU / SQ_WAVES; lds_confl = SQ_LDS_BANK_CONFLICT / "
              "(SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT)",
              "#   read_MB / write_MB = FETCH_SIZE / WRITE_SIZE (KiB) x the plain-copy calibration of",
              "#   sparse_gemm_2048x4096x4096_traffic.txt (FETCH_SIZE counts half of a copy's read bytes,",
              "#   WRITE_SIZE all of its written bytes): L2-to-memory traffic, MALL hits included"]
    scales = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_FILE) if ":" in l and not l.startswith("#"))
        scales = {"FETCH_SIZE": float(kv["read_scale"]), "WRITE_SIZE": float(kv["write_scale"])}
    except (OSError, KeyError, ValueError):
        pass
    for (row, kern, grid), t in table.items():
        m = {c: t["sums"][c] / t["n"][c] for c in t["sums"]}
        d = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and m.get("GRBM_GUI_ACTIVE"):
            d.append(f"mfma_util={m['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * m['GRBM_GUI_ACTIVE'] / 8):.3f}")
        if "SQ_INSTS_VALU" in m and m.get("SQ_WAVES"):
            d.append(f"valu_per_wave={m['SQ_INSTS_VALU'] / m['SQ_WAVES']:.0f}")
        if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_LDS_IDX_ACTIVE"):
            d.append(f"lds_confl={m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_LDS_IDX_ACTIVE'] - m['SQ_LDS_BANK_CONFLICT'], 1):.3f}")
        if "FETCH_SIZE" in m:
            d.append(f"read_MB={m['FETCH_SIZE'] * 1024 * scales['FETCH_SIZE'] / 1e6:.1f}")
        if "WRITE_SIZE" in m:
            d.append(f"write_MB={m['WRITE_SIZE'] * 1024 * scales['WRITE_SIZE'] / 1e6:.1f}")
        lines.append(f"{row} | {kern} | {grid} | " + " ".join(d))
    open(out_file, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stall_summary(out_file, title, command_lines, run_dirs, kernel_substr):
    """Where the waves of one kernel spend their cycles (SQ counters, mean per
    dispatch over the runs): fractions of SQ_WAVE_CYCLES."""
    m, n = {}, {}
    for rd in run_dirs:
        for name, gx, gy, gz, cnt in _dispatch_counters(rd):
            if kernel_substr not in name:
                continue
            for c, v in cnt.items():
                m[c] = m.get(c, 0.0) + v
                n[c] = n.get(c, 0) + 1
    m = {c: m[c] / n[c] for c in m}
    wc = m.get("SQ_WAVE_CYCLES", 0.0)
    lines = [f"# {title}", "# commands (from the repository root on an MI355X; one counter set per run):"]
    lines += ["#   " + c for c in command_lines]
    lines += ["# mean per dispatch of each counter (summed over hardware instances); fractions are of",
              "# SQ_WAVE_CYCLES (wave-cycles the kernel's waves were resident; the SQ counts these in",
              "# units of 4 cycles, as it does the other *_CYCLES / WAIT / ACTIVE counters)"]
    for c in sorted(m):
        frac = f"  ({m[c] / wc:.3f} of wave cycles)" if wc and c != "SQ_WAVE_CYCLES" and \
            (c.startswith("SQ_WAIT") or c.startswith("SQ_ACTIVE") or c.endswith("_CYCLES")) else ""
        lines.append(f"{c}: {m[c]:.6g}{frac}")
    if m.get("SQ_WAVES"):
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU"):
            if c in m:
                lines.append(f"{c}_per_wave: {m[c] / m['SQ_WAVES']:.1f}")
    open(out_file, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_summary(out_file, title, command_lines, run_dir):
    """Per kernel of a rocprofv3 --kernel-trace run: calls and durations (us),
    registers and LDS, longest total first."""
    import glob
    import sqlite3
    db = sorted(glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True))[0]
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute(
        "select s.kernel_name, count(*), avg(d.end - d.start), min(d.end - d.start), max(d.end - d.start), "
        "sum(d.end - d.start), s.arch_vgpr_count, s.accum_vgpr_count, s.group_segment_size "
        "from rocpd_kernel_dispatch d join rocpd_info_kernel_symbol s on d.kernel_id = s.id "
        "group by s.kernel_name order by sum(d.end - d.start) desc").fetchall()
    durations = {}
    for name, dur in cur.execute("select s.kernel_name, d.end - d.start from rocpd_kernel_dispatch d "
                                 "join rocpd_info_kernel_symbol s on d.kernel_id = s.id"):
        durations.setdefault(name, []).append(dur)
    lines = [f"# {title}", "# command (from the repository root on an MI355X):"]
    lines += ["#   " + c for c in command_lines]
    lines += ["# source: rocprofv3 --kernel-trace (rocpd database), durations in microseconds",
              " calls    avg_us median_us    min_us    max_us   total_us vgpr agpr  lds_B  kernel"]
    for name, n, avg, mn, mx, tot, vg, ag, lds in rows:
        med = float(np.median(durations[name]))
        lines.append(f"{n:6d} {avg / 1e3:9.2f} {med / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f} {tot / 1e3:10.1f} "
                     f"{vg:4d} {ag:4d} {lds:6d}  {_short(name)[:110]}")
    open(out_file, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
    ap.add_argument("--only", choices=["gemm", "rows"], default=None,
                    help="run only the headline loop, or only the per-row kernels (for counter collection)")
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR", default=None,
                    help="write the sparse GEMM traffic file from FETCH_SIZE, WRITE_SIZE and the two copy "
                         "calibration counter runs")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--markers", action="store_true",
                    help="with --only rows: a marker launch before each row, for the counter summary")
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG", default=None,
                    help="OUT_FILE BENCH_JSON RUN_DIR...: per-row counter table of --only rows --markers runs")
    ap.add_argument("--stall-summary", nargs="+", metavar="ARG", default=None,
                    help="OUT_FILE KERNEL_SUBSTR RUN_DIR...: SQ cycle breakdown of one kernel")
    ap.add_argument("--trace-summary", nargs=2, metavar=("OUT_FILE", "RUN_DIR"), default=None,
                    help="per-kernel duration table of a rocprofv3 --kernel-trace run")
    ap.add_argument("--title", default="", help="first line of a summary file")
    ap.add_argument("--command", action="append", default=[], help="a command line recorded in a summary file")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs every kernel on a single MI355X "
              "and has no multi-GPU path. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_summary:
        write_traffic_summary(*args.traffic_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary[0], args.counter_summary[1], args.title, args.command,
                        args.counter_summary[2:])
        return
    if args.trace_summary:
        trace_summary(args.trace_summary[0], args.title, args.command, args.trace_summary[1])
        return
    if args.stall_summary:
        stall_summary(args.stall_summary[0], args.title, args.command, args.stall_summary[2:],
                      args.stall_summary[1])
        return
    sg.lib()
    if args.only == "rows":
        MARKERS["on"] = args.markers
        rows = rows_report()
        assert not args.markers or MARKERS["n"] == len(rows), "one marker per row"
        print(json.dumps({"rows": rows, "row_order": list(rows.keys()), "markers": MARKERS["n"]}))
        return
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
            "kernel": "k_gemm_sparse_wr<128, bf16, Y> (2:4 FP8 GEMM, packed weight, Y form)",
            "avg_launch_ms": round(h["gemm_ms"], 5),
        },
        "rows": {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in rows.items()},
        "measured_peaks": measured_peaks(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
