"""GPU parity of the weight-only 2:4 GEMM (bf16 activations x e4m3 / int8 2:4
codes, groupwise weight scales) against the oracle: random codes over each
code type's whole finite range, ragged shapes, both scale granularities, both
output forms, fp32 and bf16 outputs, bias, and the M=16 decode shape."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, assert_within_tolerance, down, say, up

pytestmark = pytest.mark.gpu


def operands(m, n, k, gn, int8, seed):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(workloads.sparse_large(seed=seed, m=m, n=8, k=k)["x"]).to(DEV).to(torch.bfloat16)
    keep, _ = oracle.prune24(rng.standard_normal((n, k)).astype(np.float32))
    if int8:
        c = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    else:
        c = rng.integers(0, 256, size=(n, k)).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] ^= 1                              # every finite e4m3 code, no NaN
    wv, meta = oracle.compress24(c, keep)
    sw = (rng.uniform(0.5, 2.0, size=(-(-n // gn), k // 128)) * 2.0 ** -6).astype(np.float32)
    return x, wv, meta, sw


def check(m, n, k, gn=128, int8=False, out=torch.bfloat16, forms=("y", "yt"), bias=False, seed=0):
    say(f"w8a16 M={m} N={n} K={k} gn={gn} int8={int8} {out} bias={bias} seed={seed}")
    x, wv, meta, sw = operands(m, n, k, gn, int8, seed)
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, bound = oracle.w8a16_sparse24_gemm_groupwise(xbits, wv, meta, sw, gn, "int8" if int8 else "e4m3", bound=True)
    b = None
    if bias:
        bnp = np.random.default_rng(seed + 1).standard_normal(n).astype(np.float32)
        ref, bound = oracle.add_bias(ref, bound, bnp)
        b = up(bnp)
    outs = {}
    for form in forms:
        y = sg.w8a16_sparse24_gemm_groupwise(x, up(wv), up(meta), up(sw), gn, out_dtype=out, form=form, bias=b)
        got = down(y)
        got = got.T if form == "yt" else got
        assert got.shape == (m, n)
        assert_within_tolerance(got.astype(np.float64), ref, bound, f"form={form}")
        outs[form] = got
    if len(outs) == 2:
        assert np.array_equal(outs["y"], outs["yt"])


SHAPES = [(1, 256, 128), (16, 512, 256), (17, 300, 384), (37, 1000, 512), (64, 260, 256), (65, 256, 256),
          (200, 384, 640),
          # M = 49..64: two grid rows of 32 X rows (the second partial), with
          # 224+ workgroups, with the even split, and with one row block each
          (49, 14336, 256), (64, 11008, 256), (60, 4100, 384), (64, 1792, 256),
          # M = 17..48 over at most 128 row blocks: two grid rows of 2 or 1 sub-tiles
          (37, 1792, 384), (20, 1000, 256)]


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_w8a16_ragged(m, n, k, int8):
    check(m, n, k, int8=int8, seed=m + n + k + int8)


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("gn", [1, 128])
def test_w8a16_scales_fp32_bias(gn, int8):
    check(37, 300, 384, gn=gn, int8=int8, out=torch.float32, bias=True, seed=7 + gn)


@pytest.mark.parametrize("int8", [False, True])
def test_w8a16_decode_full_size(int8):
    """M = 16, N = 14336, K = 4096 (the benchmark's shape), every output."""
    check(16, 14336, 4096, int8=int8, forms=("y",), seed=21 + int8)


@pytest.mark.parametrize("int8", [False, True])
def test_w8a16_decode_m37_full_size(int8):
    """M = 37 (three 16-row sub-tiles, X in registers), N = 14336, K = 4096:
    four row blocks per workgroup."""
    check(37, 14336, 4096, int8=int8, forms=("y",), seed=23 + int8)


def test_w8a16_two_row_blocks_ragged_last():
    """M = 32, N = 7208: two row blocks per workgroup, the last one partial."""
    check(32, 7208, 512, out=torch.float32, bias=True, seed=25)


# More 16-row blocks than CUs but under 896: one workgroup per CU with an even
# share of two, three or four row blocks (the share's first row not a multiple
# of the share's size), for one, two and three 16-row sub-tiles of X.
EVEN_SPLIT = [(16, 5120, 1024, 128), (20, 11008, 512, 128), (37, 12288, 512, 128), (48, 13000, 256, 128),
              (33, 11000, 256, 1)]


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("m,n,k,gn", EVEN_SPLIT)
def test_w8a16_decode_even_row_split(m, n, k, gn, int8):
    check(m, n, k, gn=gn, int8=int8, out=torch.float32 if gn == 1 else torch.bfloat16, bias=gn == 1,
          seed=m + n + int8)


# Large M: the 256 x 128 tile kernel (taken from 192 tiles on), with the last
# tiles partly past M and N.
@pytest.mark.parametrize("int8", [False, True])
def test_w8a16_large_m_tiles(int8):
    check(1000, 12300, 256, int8=int8, seed=60 + int8)


def test_w8a16_mid_m_on_the_tile_kernel():
    """M = 130 over a wide weight: two m tiles, the second 2 rows tall."""
    check(130, 14336, 256, seed=66)


def test_w8a16_long_k_tile_kernel():
    """K = 8192 (64 K blocks) through the tile kernel's two-stage loop, M = 512,
    N = 4096; the oracle computes a sample of rows."""
    m, n, k = 512, 4096, 8192
    say(f"w8a16 long K M={m} N={n} K={k}")
    x, wv, meta, sw = operands(m, n, k, 128, False, seed=67)
    got = down(sg.w8a16_sparse24_gemm_groupwise(x, up(wv), up(meta), up(sw), 128))
    rows = np.array([0, 77, 128, 300, 511])
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref, bound = oracle.w8a16_sparse24_gemm_groupwise(xbits, wv, meta, sw, 128, "e4m3", bound=True)
    assert_within_tolerance(got[rows].astype(np.float64), ref, bound, "sampled rows")


def test_w8a16_large_m_per_row_scales_fp32_bias_single_k_block():
    check(300, 24580, 128, gn=1, out=torch.float32, bias=True, seed=62)


@pytest.mark.parametrize("int8", [False, True])
def test_w8a16_large_m_full_size_sampled_rows(int8):
    """2048 x 4096 x 4096 (the benchmark's shape) on the tile kernel; the
    oracle computes a sample of rows from every kind of tile position."""
    m, n, k = 2048, 4096, 4096
    say(f"w8a16 full size M={m} N={n} K={k} int8={int8}")
    x, wv, meta, sw = operands(m, n, k, 128, int8, seed=64 + int8)
    got = down(sg.w8a16_sparse24_gemm_groupwise(x, up(wv), up(meta), up(sw), 128))
    rows = np.array([0, 1, 63, 64, 127, 128, 1000, 1919, 2047])
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref, bound = oracle.w8a16_sparse24_gemm_groupwise(xbits, wv, meta, sw, 128, "int8" if int8 else "e4m3",
                                                      bound=True)
    assert_within_tolerance(got[rows].astype(np.float64), ref, bound, "sampled rows")


def test_w8a16_from_the_gpu_weight_pipeline():
    """GPU prune + compress + int8 / e4m3 quantisation of a weight, then the
    weight-only GEMM, against the oracle's chain."""
    m, n, k = 16, 512, 1024
    say(f"w8a16 pipeline M={m} N={n} K={k}")
    d = workloads.sparse_large(seed=30, m=m, n=n, k=k)
    x = up(d["x"]).to(torch.bfloat16)
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    v32, meta = sg.sparse24_prune_compress(up(d["w"]))
    ov32, ometa = oracle.prune_compress24(d["w"])
    for int8 in (False, True):
        q, s = (sg.int8_quant_groupwise if int8 else sg.fp8_quant_groupwise)(v32, gr=128, gc=64)
        oq, os_ = (oracle.int8_quant_groupwise if int8 else oracle.fp8_quant_groupwise)(ov32, 128, 64)
        got = down(sg.w8a16_sparse24_gemm_groupwise(x, q, meta, s, 128))
        ref, bound = oracle.w8a16_sparse24_gemm_groupwise(xbits, oq, ometa, os_, 128, "int8" if int8 else "e4m3",
                                                          bound=True)
        assert_within_tolerance(got, ref, bound, f"int8={int8}")


# ------------------------------------------------- W8A16, packed weight

def check_packed(m, n, k, gn=128, int8=False, out=torch.bfloat16, forms=("y", "yt"), bias=False, seed=0,
                 rows=None):
    """The packed weight-only GEMM against the oracle (on `rows` of the
    output only, when given), and bit for bit against the same call on the
    unpacked weight."""
    say(f"w8a16 packed M={m} N={n} K={k} gn={gn} int8={int8} {out} bias={bias} seed={seed}")
    x, wv, meta, sw = operands(m, n, k, gn, int8, seed)
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    sel = np.arange(m) if rows is None else np.asarray(rows)
    ref, bound = oracle.w8a16_sparse24_gemm_groupwise(xbits[sel], wv, meta, sw, gn, "int8" if int8 else "e4m3",
                                                      bound=True)
    b = None
    if bias:
        bnp = np.random.default_rng(seed + 1).standard_normal(n).astype(np.float32)
        ref, bound = oracle.add_bias(ref, bound, bnp)
        b = up(bnp)
    wvg, mg, swg = up(wv), up(meta), up(sw)
    wp = sg.sparse24_pack_gfx950(wvg, mg)
    for form in forms:
        y = sg.w8a16_sparse24_gemm_groupwise_packed(x, wp, n, swg, gn, int8=int8, out_dtype=out, form=form, bias=b)
        yc = sg.w8a16_sparse24_gemm_groupwise(x, wvg, mg, swg, gn, out_dtype=out, form=form, bias=b)
        assert torch.equal(y.view(torch.int16) if out == torch.bfloat16 else y.view(torch.int32),
                           yc.view(torch.int16) if out == torch.bfloat16 else yc.view(torch.int32)), f"form={form}"
        got = down(y)
        got = got.T if form == "yt" else got
        assert got.shape == (m, n)
        assert_within_tolerance(got[sel].astype(np.float64), ref, bound, f"form={form}")


# the LDS-streaming decode kernel (M <= 48: one, two, three 16-row sub-tiles;
# N not a multiple of 16, so the packer's zero rows are read; the even split),
# the register kernel (M = 49..64, and M > 64 where tiles do not pay) and
# the 256 x 128 tile kernel
PACKED_SHAPES = [(1, 256, 128), (16, 512, 256), (17, 300, 384), (37, 1000, 512), (48, 13000, 256),
                 (16, 5120, 1024), (20, 11008, 512), (64, 260, 256), (65, 256, 256), (200, 384, 640),
                 (1000, 12300, 256), (49, 14336, 256), (64, 11008, 256), (60, 4100, 384),
                 # fewer than 16 W rows: one partial row block (the packer's zero rows)
                 (5, 7, 128), (70, 9, 256)]


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("m,n,k", PACKED_SHAPES)
def test_w8a16_packed(m, n, k, int8):
    check_packed(m, n, k, int8=int8, seed=m + n + k + 3 * int8)


@pytest.mark.parametrize("m,n,k", [(37, 300, 384), (64, 260, 256), (300, 24580, 128)])
def test_w8a16_packed_per_row_scales_fp32_bias(m, n, k):
    check_packed(m, n, k, gn=1, out=torch.float32, bias=True, seed=70 + m)


@pytest.mark.parametrize("int8", [False, True])
def test_w8a16_packed_decode_full_size(int8):
    """M = 16 and 37, N = 14336, K = 4096 (the benchmark's decode shape)."""
    check_packed(16, 14336, 4096, int8=int8, forms=("y",), seed=80 + int8)
    check_packed(37, 14336, 4096, int8=int8, forms=("y",), seed=82 + int8)


def test_w8a16_packed_large_m_full_size_sampled_rows():
    """2048 x 4096 x 4096 on the tile kernel, K = 8192 on a 512-row X; the
    oracle computes sampled rows, the unpacked call all of them."""
    check_packed(2048, 4096, 4096, forms=("y",), seed=84, rows=[0, 1, 127, 128, 1000, 2047])
    check_packed(512, 4096, 8192, forms=("y",), seed=85, rows=[0, 77, 300, 511])


# --------------------------------------------------------------- W4A16

def check_w4(m, n, k, out=torch.bfloat16, forms=("y", "yt"), bias=False, seed=0):
    say(f"w4a16 M={m} N={n} K={k} {out} bias={bias} seed={seed}")
    d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
    x = up(d["x"]).to(torch.bfloat16)
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    v32, meta = oracle.prune_compress24(d["w"])
    q4, s4 = oracle.int4_quant_groupwise(v32, 64)
    ref, bound = oracle.w4a16_sparse24_gemm_groupwise(xbits, q4, meta, s4, bound=True)
    b = None
    if bias:
        bnp = np.random.default_rng(seed + 1).standard_normal(n).astype(np.float32) * 0.1
        ref, bound = oracle.add_bias(ref, bound, bnp)
        b = up(bnp)
    outs = {}
    for form in forms:
        got = down(sg.w4a16_sparse24_gemm_groupwise(x, up(q4), up(meta), up(s4), out_dtype=out, form=form, bias=b))
        got = got.T if form == "yt" else got
        assert_within_tolerance(got.astype(np.float64), ref, bound, f"form={form}")
        outs[form] = got
    if len(outs) == 2:
        assert np.array_equal(outs["y"], outs["yt"])


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_w4a16_ragged(m, n, k):
    check_w4(m, n, k, seed=40 + m + n)


def test_w4a16_fp32_bias():
    check_w4(37, 300, 384, out=torch.float32, bias=True, seed=41)


def test_w4a16_decode_full_size():
    check_w4(16, 14336, 4096, forms=("y",), seed=42)


def test_w4a16_decode_m37_full_size():
    check_w4(37, 14336, 4096, forms=("y",), seed=43)


@pytest.mark.parametrize("m,n,k", [(16, 5120, 512), (37, 11008, 256)])
def test_w4a16_decode_even_row_split(m, n, k):
    check_w4(m, n, k, seed=44 + m)


def test_w4a16_large_m_tiles():
    check_w4(1000, 12300, 256, seed=63)


def test_w4a16_from_the_gpu_weight_pipeline():
    """GPU prune + compress + int4 quantisation (64 compressed values per
    scale), bit-exact against the oracle's, then the GEMM."""
    m, n, k = 16, 512, 1024
    say(f"w4a16 pipeline M={m} N={n} K={k}")
    d = workloads.sparse_large(seed=43, m=m, n=n, k=k)
    x = up(d["x"]).to(torch.bfloat16)
    v32, meta = sg.sparse24_prune_compress(up(d["w"]))
    q4, s4 = sg.int4_quant_groupwise(v32, gc=64)
    ov32, ometa = oracle.prune_compress24(d["w"])
    oq4, os4 = oracle.int4_quant_groupwise(ov32, 64)
    assert np.array_equal(down(q4), oq4) and np.array_equal(down(s4), os4)
    got = down(sg.w4a16_sparse24_gemm_groupwise(x, q4, meta, s4))
    ref, bound = oracle.w4a16_sparse24_gemm_groupwise(x.view(torch.int16).cpu().numpy().view(np.uint16), oq4, ometa,
                                                      os4, bound=True)
    assert_within_tolerance(got, ref, bound, "pipeline")



# ------------------------------------------------- W4A16, blocked weight

def check_w4_packed(m, n, k, out=torch.bfloat16, forms=("y", "yt"), bias=False, seed=0, rows=None):
    """The GPU packer against the oracle's blocked layout byte for byte, then
    the blocked-weight W4A16 GEMM against the oracle (on `rows` only, when
    given) and bit for bit against the same call on the unpacked weight."""
    say(f"w4a16 blocked M={m} N={n} K={k} {out} bias={bias} seed={seed}")
    d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
    x = up(d["x"]).to(torch.bfloat16)
    xbits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    v32, meta = oracle.prune_compress24(d["w"])
    q4, s4 = oracle.int4_quant_groupwise(v32, 64)
    sel = np.arange(m) if rows is None else np.asarray(rows)
    ref, bound = oracle.w4a16_sparse24_gemm_groupwise(xbits[sel], q4, meta, s4, bound=True)
    b = None
    if bias:
        bnp = np.random.default_rng(seed + 1).standard_normal(n).astype(np.float32) * 0.1
        ref, bound = oracle.add_bias(ref, bound, bnp)
        b = up(bnp)
    qg, mg, sg4 = up(q4), up(meta), up(s4)
    wp = sg.sparse24_pack_w4(qg, mg)
    assert np.array_equal(down(wp), oracle.pack24_w4_blocked(q4, meta))
    for form in forms:
        y = sg.w4a16_sparse24_gemm_groupwise_packed(x, wp, n, sg4, out_dtype=out, form=form, bias=b)
        yc = sg.w4a16_sparse24_gemm_groupwise(x, qg, mg, sg4, out_dtype=out, form=form, bias=b)
        iv = torch.int16 if out == torch.bfloat16 else torch.int32
        assert torch.equal(y.view(iv), yc.view(iv)), f"form={form}"
        got = down(y)
        got = got.T if form == "yt" else got
        assert got.shape == (m, n)
        assert_within_tolerance(got[sel].astype(np.float64), ref, bound, f"form={form}")


@pytest.mark.parametrize("m,n,k", PACKED_SHAPES)
def test_w4a16_packed(m, n, k):
    check_w4_packed(m, n, k, seed=90 + m + n)


@pytest.mark.parametrize("m,n,k", [(37, 300, 384), (64, 260, 256), (300, 24580, 128)])
def test_w4a16_packed_fp32_bias(m, n, k):
    check_w4_packed(m, n, k, out=torch.float32, bias=True, seed=95 + m)


def test_w4a16_packed_decode_full_size():
    check_w4_packed(16, 14336, 4096, forms=("y",), seed=96)
    check_w4_packed(37, 14336, 4096, forms=("y",), seed=97)


def test_w4a16_packed_large_m_sampled_rows():
    check_w4_packed(2048, 4096, 4096, forms=("y",), seed=98, rows=[0, 1, 127, 128, 1000, 2047])
