"""GPU parity of the int8 x int8 2:4-sparse path against the oracle: the int8
quantiser bit-exactly, the GEMM (canonical and gfx950-packed weights) within
|y - y_ref| <= 1e-2 |y_ref| + 1e-3 T over ragged shapes, all scale modes, the
decode shapes and the full 2048 x 4096 x 4096 size in both output forms."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, assert_within_tolerance, down, say, up, up_scales

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gr,gc,rows,cols", [(1, 128, 37, 512), (1, 64, 300, 256), (128, 64, 300, 256),
                                             (128, 128, 130, 384)])
@pytest.mark.parametrize("bf16", [False, True])
def test_int8_quant_bit_exact(gr, gc, rows, cols, bf16):
    say(f"int8 quant gr={gr} gc={gc} {rows}x{cols} bf16={bf16}")
    x = workloads.sparse_large(seed=rows + cols, m=rows, n=8, k=cols)["x"]
    x[1, :gc] = 0.0                                          # an all-zero block
    x[2, 3] = 1e30                                           # a block dominated by one value
    xt = up(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
        x = xt.float().cpu().numpy()
    q, s = sg.int8_quant_groupwise(xt, gr=gr, gc=gc)
    rq, rs = oracle.int8_quant_groupwise(x, gr, gc)
    assert np.array_equal(down(q), rq)
    assert np.array_equal(down(s), rs)


def operands(m, n, k, gm, gn, seed):
    d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
    xq, sx = oracle.int8_quant_groupwise(d["x"], gm, 128)
    wv32, meta = oracle.prune_compress24(d["w"])
    wq, sw = oracle.int8_quant_groupwise(wv32, gn, 64)
    return xq, sx, wq, meta, sw


def check(m, n, k, gm=1, gn=128, out_dtype=torch.bfloat16, forms=("y", "yt"), seed=0, packed=False, m_major=True):
    say(f"int8 sparse M={m} N={n} K={k} gm={gm} gn={gn} {out_dtype} {forms} packed={packed} seed={seed}")
    xq, sx, wq, meta, sw = operands(m, n, k, gm, gn, seed)
    ref, bound = oracle.int8_sparse24_gemm_groupwise(xq, sx, gm, wq, meta, sw, gn, bound=True)
    outs = {}
    for form in forms:
        if packed:
            wp = sg.sparse24_pack_gfx950(up(wq), up(meta))
            y = sg.int8_sparse24_gemm_groupwise_packed(up(xq), up_scales(sx, m_major), wp, n, up_scales(sw, m_major),
                                                       gm, gn, out_dtype=out_dtype, form=form)
        else:
            y = sg.int8_sparse24_gemm_groupwise(up(xq), up_scales(sx, m_major), up(wq), up(meta),
                                                up_scales(sw, m_major), gm, gn, out_dtype=out_dtype, form=form)
        got = down(y)
        got = got.T if form == "yt" else got
        assert got.shape == (m, n)
        assert_within_tolerance(got.astype(np.float64), ref, bound, f"form={form}")
        outs[form] = got
    if len(outs) == 2:
        assert np.array_equal(outs["y"], outs["yt"])


RAGGED = [(1, 256, 128), (16, 256, 128), (17, 300, 384), (37, 512, 256), (64, 128, 256), (65, 256, 128),
          (129, 256, 256), (200, 700, 384), (300, 1000, 512)]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("m,n,k", RAGGED)
def test_int8_ragged_shapes(m, n, k, packed):
    check(m, n, k, seed=m * 5 + n, packed=packed)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("gm,gn", [(1, 1), (128, 1), (128, 128), (1, 128)])
@pytest.mark.parametrize("m", [37, 300])
def test_int8_granularity_modes(gm, gn, m, packed):
    check(m, 384, 256, gm=gm, gn=gn, seed=17 + gm + gn, packed=packed)


def test_int8_fp32_output_row_major_scales():
    check(257, 260, 256, out_dtype=torch.float32, seed=9, m_major=False, forms=("y",))
    check(20, 260, 256, out_dtype=torch.float32, seed=9, m_major=False, forms=("y",), packed=True)


@pytest.mark.parametrize("m,n,k", workloads.DECODE_SHAPES)
def test_int8_decode_shapes(m, n, k):
    check(m, n, k, seed=6, packed=True)


def test_int8_full_size_both_forms():
    check(2048, 4096, 4096, seed=3, packed=True)


def test_int8_gpu_prep_chain_matches_oracle_chain():
    """GPU prune + int8 quantisers + pack + GEMM on raw fp32 inputs against the
    oracle chain (the intermediate codes are bit-exact, so the GEMM inputs agree)."""
    d = workloads.sparse_large(seed=23, m=512, n=1024, k=1024)
    wv, meta = sg.sparse24_prune_compress(up(d["w"]))
    wq, sw = sg.int8_quant_groupwise(wv, gr=128, gc=64)
    wp = sg.sparse24_pack_gfx950(wq, meta)
    xq, sx = sg.int8_quant_groupwise(up(d["x"]), gr=1, gc=128)
    y = down(sg.int8_sparse24_gemm_groupwise_packed(xq, sx, wp, 1024, sw, 1, 128))
    oxq, osx, owq, ometa, osw = operands(512, 1024, 1024, 1, 128, 23)
    assert np.array_equal(down(wq), owq) and np.array_equal(down(xq), oxq)
    ref, bound = oracle.int8_sparse24_gemm_groupwise(oxq, osx, 1, owq, ometa, osw, 128, bound=True)
    assert_within_tolerance(y, ref, bound, "int8 end-to-end")
