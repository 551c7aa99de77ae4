"""Non-finite values through the GEMMs: a NaN scale of one X row's K block
turns that output row into NaN, a NaN W scale block turns its output columns
into NaN, and the bf16 output keeps NaN as NaN (a rounding that carries into
the exponent would turn some NaN patterns into infinity).  Every other output
stays within the oracle's tolerance.  The pages say nothing of non-finite
inputs; the reading checked here is plain IEEE propagation through the
documented formula."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import down, say, up, up_scales

pytestmark = pytest.mark.gpu


def _check(got, ref, bound, what):
    gn, rn = np.isnan(got), np.isnan(ref)
    assert rn.any(), "the case must hold NaN outputs"
    assert np.array_equal(gn, rn), f"{what}: NaN at {np.argwhere(gn != rn)[:4].tolist()}"
    ok = oracle.within_tolerance(got[~rn], ref[~rn], bound[~rn])
    assert ok.all(), f"{what}: {(~ok).sum()} finite outputs outside tolerance"


@pytest.mark.parametrize("m", [300, 16, 37])
@pytest.mark.parametrize("path", ["dense", "sparse", "packed", "int8"])
@pytest.mark.parametrize("out,form", [(torch.float32, "y"), (torch.bfloat16, "y"), (torch.bfloat16, "yt")])
def test_nan_scales_give_nan_rows_and_columns(m, path, out, form):
    n, k = 384, 512
    say(f"NaN scales {path} M={m} {out} {form}")
    d = workloads.sparse_large(seed=60 + m, m=m, n=n, k=k)
    if path == "int8":
        xq, sx = oracle.int8_quant_groupwise(d["x"], 1, 128)
        wv32, meta = oracle.prune_compress24(d["w"])
        wq, sw = oracle.int8_quant_groupwise(wv32, 128, 64)
    else:
        xq, sx = oracle.fp8_quant_groupwise(d["x"], 1, 128)
        if path == "dense":
            wq, sw = oracle.fp8_quant_groupwise(d["w"], 128, 128)
            meta = None
        else:
            wv32, meta = oracle.prune_compress24(d["w"])
            wq, sw = oracle.fp8_quant_groupwise(wv32, 128, 64)
    sx = sx.copy()
    sw = sw.copy()
    sx[5, 1] = np.nan                  # row 5
    sw[2, 3] = np.nan                  # columns 256 .. 383
    if path == "dense":
        ref, bound = oracle.fp8_gemm_groupwise(xq, sx, 1, wq, sw, 128, bound=True)
        y = sg.fp8_gemm_groupwise(up(xq), up_scales(sx), up(wq), up_scales(sw), 1, 128, out, form)
    elif path == "int8":
        ref, bound = oracle.int8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
        y = sg.int8_sparse24_gemm_groupwise(up(xq), up_scales(sx), up(wq), up(meta), up_scales(sw), 1, 128,
                                            out, form)
    elif path == "sparse":
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
        y = sg.fp8_sparse24_gemm_groupwise(up(xq), up_scales(sx), up(wq), up(meta), up_scales(sw), 1, 128,
                                           out, form)
    else:
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
        wp = sg.sparse24_pack_gfx950(up(wq), up(meta))
        y = sg.fp8_sparse24_gemm_groupwise_packed(up(xq), up_scales(sx), wp, n, up_scales(sw), 1, 128, out, form)
    got = down(y).astype(np.float64)
    got = got.T if form == "yt" else got
    _check(got, ref, bound, f"{path} M={m}")
    assert np.isnan(got[5]).all() and np.isnan(got[:, 256:]).all()


def test_bf16_output_of_a_nan_stays_nan_for_every_payload():
    """Scales whose products are NaN with payloads that a carry would push into
    the exponent (0x7F800001-style): every such bf16 output is NaN, never inf."""
    m, n, k = 64, 256, 256
    d = workloads.sparse_large(seed=61, m=m, n=n, k=k)
    xq, sx = oracle.fp8_quant_groupwise(d["x"], 1, 128)
    wq, sw = oracle.fp8_quant_groupwise(d["w"], 128, 128)
    sx = sx.copy()
    payloads = np.array([0x7F800001, 0xFF800001, 0x7F807FFF, 0x7FFFFFFF], np.uint32).view(np.float32)
    sx[:4, 0] = payloads
    y = down(sg.fp8_gemm_groupwise(up(xq), up_scales(sx), up(wq), up_scales(sw), 1, 128, torch.bfloat16))
    assert np.isnan(y[:4]).all() and np.isfinite(y[4:]).all()
