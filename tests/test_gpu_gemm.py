"""GPU parity of the FP8 groupwise GEMMs (dense and 2:4-sparse W) against the
oracle, within |y - y_ref| <= 1e-2 |y_ref| + 1e-3 T (T = sum over K blocks of
the scale product times sum |x w|).  Operands are quantised (and pruned) by
the oracle, so these tests check the GEMM alone; the quantiser and pruning
kernels are checked bit-exactly in test_gpu_quant_prune.py."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, assert_within_tolerance, down, oracle_operands, say, up, up_scales

pytestmark = pytest.mark.gpu


def run_gemm(sparse, xq, sx, gm, wq, meta, sw, gn, out_dtype, form, m_major=True, packed=False):
    args = (up(xq), up_scales(sx, m_major))
    if packed:
        wp = up(oracle.pack24_gfx950(wq, meta))
        return sg.fp8_sparse24_gemm_groupwise_packed(*args, wp, wq.shape[0], up_scales(sw, m_major), gm, gn,
                                                     out_dtype=out_dtype, form=form)
    if sparse:
        return sg.fp8_sparse24_gemm_groupwise(*args, up(wq), up(meta), up_scales(sw, m_major), gm, gn,
                                              out_dtype=out_dtype, form=form)
    return sg.fp8_gemm_groupwise(*args, up(wq), up_scales(sw, m_major), gm, gn, out_dtype=out_dtype, form=form)


def check(sparse, m, n, k, gm=1, gn=128, out_dtype=torch.bfloat16, forms=("y", "yt"), seed=0, dist="sparse",
          m_major=True, packed=False):
    kind = "packed" if packed else ("sparse" if sparse else "dense")
    say(f"{kind} M={m} N={n} K={k} gm={gm} gn={gn} {out_dtype} {forms} seed={seed}")
    d = (workloads.dense_outliers if dist == "outliers" else workloads.sparse_large)(seed=seed, m=m, n=n, k=k)
    xq, sx, wq, meta, sw = oracle_operands(d["x"], d["w"], gm, gn, sparse)
    if sparse:
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, gm, wq, meta, sw, gn, bound=True)
    else:
        ref, bound = oracle.fp8_gemm_groupwise(xq, sx, gm, wq, sw, gn, bound=True)
    outs = {}
    for form in forms:
        y = run_gemm(sparse, xq, sx, gm, wq, meta, sw, gn, out_dtype, form, m_major, packed)
        got = down(y)
        got = got.T if form == "yt" else got
        assert got.shape == (m, n)
        assert_within_tolerance(got.astype(np.float64), ref, bound, f"form={form}")
        outs[form] = got
    if len(outs) == 2:   # both forms store the same numbers
        assert np.array_equal(outs["y"], outs["yt"])
    return outs


RAGGED = [(1, 256, 128), (15, 100, 256), (16, 256, 128), (17, 300, 384), (37, 512, 256), (64, 128, 256),
          (65, 256, 128), (127, 257, 256), (128, 512, 128), (129, 256, 256), (200, 700, 384), (300, 1000, 512)]


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("m,n,k", RAGGED)
def test_ragged_shapes(sparse, m, n, k):
    check(sparse, m, n, k, seed=m * 7 + n)


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("gm,gn", [(1, 1), (128, 1), (128, 128), (1, 128)])
@pytest.mark.parametrize("m", [37, 300])
def test_granularity_modes(sparse, gm, gn, m):
    check(sparse, m, 384, 256, gm=gm, gn=gn, seed=11 + gm + gn)


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("m", [20, 257])
def test_fp32_output_and_row_major_scales(sparse, m):
    check(sparse, m, 260, 256, out_dtype=torch.float32, seed=5, m_major=False)


def test_tiny_config_fp32():
    """64 x 128 x 256 2:4 FP8, fp32 out (the tiny workload), sparse and dense on
    the decompressed weight."""
    d = workloads.tiny_sparse()
    xq, sx, wq, meta, sw = oracle_operands(d["x"], d["w"], 1, 128, True)
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
    for form in ("y", "yt"):
        y = down(run_gemm(True, xq, sx, 1, wq, meta, sw, 128, torch.float32, form))
        assert_within_tolerance(y.T if form == "yt" else y, ref, bound, f"tiny sparse {form}")
    wd = oracle.decompress24(wq, meta)
    y = down(run_gemm(False, xq, sx, 1, wd, None, sw, 128, torch.float32, "y"))
    assert_within_tolerance(y, ref, bound, "tiny dense(decompressed)")


def test_dense_full_size_with_outliers():
    """2048 x 4096 x 4096, X with 1% outliers x20, X 1x128 / W 128x128 scales, bf16."""
    check(False, 2048, 4096, 4096, seed=2, dist="outliers", forms=("y",))


def test_sparse_full_size_both_forms():
    """2048 x 4096 x 4096 2:4 FP8: Y = X W^T and the swapped Y^T = W X^T."""
    check(True, 2048, 4096, 4096, seed=3)


@pytest.mark.parametrize("m,n,k", workloads.DECODE_SHAPES)
def test_decode_shapes(m, n, k):
    check(True, m, n, k, seed=4, forms=("y", "yt"))


# Packed decode with more 16-row blocks than CUs but too few for 224
# workgroups of four (on a 256-CU device): one workgroup per CU, each with an
# even share of 2, 3 or 4 row blocks (320, 688, 768 and 813 row blocks here;
# N = 13000 also ends in a partial row block).
@pytest.mark.parametrize("m,n,k", [(16, 5120, 1024), (20, 11008, 512), (37, 12288, 512), (64, 13000, 256)])
def test_packed_decode_even_row_split(m, n, k):
    check(True, m, n, k, seed=5 + m, forms=("y", "yt"), packed=True)


# Packed decode at M = 49..64 over no more row blocks than CUs: two grid rows
# of 32 X rows (the second 17..32 rows), per-row and 128-row X scales.
@pytest.mark.parametrize("m,n,k,gm", [(64, 4096, 512, 1), (50, 1000, 256, 1), (64, 300, 384, 128),
                                      (49, 4096, 1024, 128),
                                      # M = 17..48 over at most 128 row blocks: two rows of 2 or 1 sub-tiles
                                      (37, 1792, 512, 1), (20, 1000, 256, 1), (40, 300, 384, 128)])
def test_packed_decode_two_grid_rows(m, n, k, gm):
    check(True, m, n, k, gm=gm, seed=21 + m + n, forms=("y", "yt"), packed=True)
    check(True, m, n, k, gm=gm, seed=22 + m + n, forms=("y",), packed=True, out_dtype=torch.float32)


@pytest.mark.parametrize("kind", ["dense", "sparse", "packed_rows"])
@pytest.mark.parametrize("m,n,k,gm", [(64, 4096, 512, 1), (50, 1000, 256, 128), (37, 1792, 256, 1),
                                      (20, 1000, 384, 128)])
def test_register_decode_two_grid_rows(kind, m, n, k, gm):
    if kind == "packed_rows":
        check(True, m, n, k, gm=gm, gn=1, seed=31 + m, packed=True)
    else:
        check(kind == "sparse", m, n, k, gm=gm, seed=33 + m + n)


# The register decode kernel (dense, canonical 2:4, and packed with per-row W
# scales) with the same split: 2, 3 and 4 row blocks per workgroup for up to
# three 16-row X sub-tiles, 2 for four (N = 13000 ends in a partial row block).
@pytest.mark.parametrize("kind", ["dense", "sparse", "packed_rows"])
@pytest.mark.parametrize("m,n,k", [(16, 5120, 512), (9, 11008, 256), (16, 13000, 256), (20, 5120, 256),
                                   (20, 11008, 256), (37, 12288, 128), (64, 5120, 256)])
def test_register_decode_even_row_split(kind, m, n, k):
    if kind == "packed_rows":
        check(True, m, n, k, gn=1, seed=11 + m, packed=True)
    else:
        check(kind == "sparse", m, n, k, seed=13 + m + n)


def test_deterministic_and_all_zero_operands():
    d = workloads.sparse_large(seed=8, m=300, n=512, k=512)
    xq, sx, wq, meta, sw = oracle_operands(d["x"], d["w"], 1, 128, True)
    a = down(run_gemm(True, xq, sx, 1, wq, meta, sw, 128, torch.bfloat16, "y"))
    b = down(run_gemm(True, xq, sx, 1, wq, meta, sw, 128, torch.bfloat16, "y"))
    assert np.array_equal(a, b)
    z = np.zeros_like(wq)
    y = down(run_gemm(True, xq, sx, 1, z, meta, np.ones_like(sw), 128, torch.float32, "y"))
    assert not y.any()


def test_outputs_outside_the_problem_are_untouched():
    """Partial tiles never store past M or N: a padded output buffer keeps its
    sentinel outside the [M, N] window."""
    m, n, k = 37, 300, 256
    d = workloads.sparse_large(seed=12, m=m, n=n, k=k)
    xq, sx, wq, meta, sw = oracle_operands(d["x"], d["w"], 1, 128, True)
    for mm in (37, 200):     # decode path and large-M path
        xqq = np.concatenate([xq] * (mm // m + 1))[:mm]
        sxx = np.concatenate([sx] * (mm // m + 1))[:mm]
        ybuf = torch.full((mm + 3, n + 8), 7.0, dtype=torch.float32, device=DEV)
        sg.fp8_sparse24_gemm_groupwise(up(xqq), up_scales(sxx), up(wq), up(meta), up_scales(sw), 1, 128,
                                       y=ybuf[:mm, :n])
        yb = down(ybuf)
        assert np.all(yb[mm:, :] == 7.0) and np.all(yb[:, n:] == 7.0)
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xqq, sxx, 1, wq, meta, sw, 128, bound=True)
        assert_within_tolerance(yb[:mm, :n], ref, bound, f"padded M={mm}")


def test_end_to_end_gpu_chain_matches_oracle_chain():
    """GPU prune + GPU quantisers + GPU GEMM on raw fp32 inputs equals the oracle
    chain: the intermediate codes are bit-exact, so the GEMM inputs agree."""
    d = workloads.sparse_large(seed=13, m=256, n=512, k=1024)
    wv, meta = sg.sparse24_prune_compress(up(d["w"]))
    wq, sw = sg.fp8_quant_groupwise(wv, gr=128, gc=64)
    xq, sx = sg.fp8_quant_groupwise(up(d["x"]), gr=1, gc=128)
    y = down(sg.fp8_sparse24_gemm_groupwise(xq, sx, wq, meta, sw, 1, 128))
    oxq, osx, owq, ometa, osw = oracle_operands(d["x"], d["w"], 1, 128, True)
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(oxq, osx, 1, owq, ometa, osw, 128, bound=True)
    assert_within_tolerance(y, ref, bound, "end-to-end")


# --- the packed weight form -------------------------------------------------

@pytest.mark.parametrize("m,n,k", RAGGED)
def test_packed_ragged_shapes(m, n, k):
    check(True, m, n, k, seed=m * 7 + n, packed=True)


@pytest.mark.parametrize("gm,gn", [(1, 1), (128, 1), (128, 128), (1, 128)])
@pytest.mark.parametrize("m", [37, 300])
def test_packed_granularity_modes(gm, gn, m):
    check(True, m, 384, 256, gm=gm, gn=gn, seed=11 + gm + gn, packed=True)


def test_packed_full_size_both_forms():
    check(True, 2048, 4096, 4096, seed=3, packed=True)


@pytest.mark.parametrize("m,n,k", workloads.DECODE_SHAPES)
def test_packed_decode_shapes(m, n, k):
    check(True, m, n, k, seed=4, forms=("y", "yt"), packed=True)


# Decode-sized M with N large enough that a workgroup owns 4 or 2 row blocks
# of 16 and the last workgroup is partly past N (M > 16: X in registers, up to
# four 16-row sub-tiles); K of 384 leaves 5 of the 8 waves without a K block.
@pytest.mark.parametrize("m,n", [(16, 14350), (9, 14400), (37, 7190), (30, 7200), (37, 14350), (64, 14350),
                                 (50, 7200), (17, 14336)])
def test_packed_decode_ragged_row_blocks(m, n):
    check(True, m, n, 384, seed=13 + m, packed=True)


# One GPU's share of an 8-way tensor-parallel decode layer: the column-parallel
# up-projection (N = 14336 / 8 rows of W) and the row-parallel
# down-projection's partial product (K = 14336 / 8), fp32 as an all-reduce
# would sum it before the bf16 rounding.
@pytest.mark.parametrize("m,n,k,out", [(16, 1792, 4096, torch.bfloat16), (16, 4096, 1792, torch.float32),
                                       (37, 1792, 4096, torch.bfloat16)])
def test_packed_tensor_parallel_share_shapes(m, n, k, out):
    check(True, m, n, k, out_dtype=out, seed=5 + m, packed=True)


# Long K: many iterations of the large-M kernel's double-stage loop (odd count
# of K-block pairs) and 32 K blocks per wave in the decode ring.
@pytest.mark.parametrize("m,n,k", [(256, 512, 16384), (200, 300, 16256), (16, 1024, 32768), (37, 600, 24576)])
def test_packed_long_k(m, n, k):
    check(True, m, n, k, out_dtype=torch.float32, forms=("y",), seed=7 + m, packed=True)


def test_packed_fp32_row_major_scales_and_equal_to_unpacked():
    d = workloads.sparse_large(seed=21, m=300, n=700, k=512)
    xq, sx, wq, meta, sw = oracle_operands(d["x"], d["w"], 1, 128, True)
    a = down(run_gemm(True, xq, sx, 1, wq, meta, sw, 128, torch.float32, "y", m_major=False))
    b = down(run_gemm(True, xq, sx, 1, wq, meta, sw, 128, torch.float32, "y", m_major=False, packed=True))
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
    assert_within_tolerance(b, ref, bound, "packed fp32")
    assert_within_tolerance(a, ref, bound, "unpacked fp32")


def test_packed_end_to_end_gpu_prep_chain():
    """GPU prune + quantise + pack, then the packed GEMM, against the oracle chain."""
    d = workloads.sparse_large(seed=22, m=512, n=1024, k=1024)
    wv, meta = sg.sparse24_prune_compress(up(d["w"]))
    wq, sw = sg.fp8_quant_groupwise(wv, gr=128, gc=64)
    wp = sg.sparse24_pack_gfx950(wq, meta)
    xq, sx = sg.fp8_quant_groupwise(up(d["x"]), gr=1, gc=128)
    y = down(sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, wp, 1024, sw, 1, 128))
    oxq, osx, owq, ometa, osw = oracle_operands(d["x"], d["w"], 1, 128, True)
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(oxq, osx, 1, owq, ometa, osw, 128, bound=True)
    assert_within_tolerance(y, ref, bound, "packed end-to-end")


# --- promotion with wide or unusual scale products ---------------------------
# The large-M kernel keeps each wave's accumulators in units of the current K
# block's scale product when every product the wave meets is a positive
# normal number within a factor 2^60 of the others, and otherwise promotes
# each block's partial from zero.  These cases put both forms in one launch.

def scale_case(kind, seed, m=300, n=512, k=2048):
    d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
    xq, _, wq, meta, _ = oracle_operands(d["x"], d["w"], 1, 128, True)
    g = workloads.generators(seed, 2)
    kb = k // 128
    sx = np.exp2(g[0].uniform(-20, 20, size=(m, kb))).astype(np.float32)
    sw = np.exp2(g[1].uniform(-2, 2, size=(-(-n // 128), kb))).astype(np.float32)
    if kind == "extreme_x_rows":       # rows 0..63 and 200..215: products 2^80 apart across K blocks
        sx[0:64, 0::4] = np.float32(2.0 ** -40)
        sx[0:64, 2::4] = np.float32(2.0 ** 40)
        sx[200:216, 3] = np.float32(2.0 ** 70)
    elif kind == "extreme_w_block":    # W rows 128..255: a 2^90 spread
        sw[1, :] = np.float32(2.0 ** -45)
        sw[1, 5] = np.float32(2.0 ** 45)
    elif kind == "zero_and_negative":  # zero, negative and subnormal products in some rows' blocks
        sx[10:20, 4] = 0.0
        sx[70:90, 2] = -sx[70:90, 2]
        sx[150:160, 7] = np.float32(1e-39)
    elif kind == "edge_of_window":     # products exactly 2^60 apart: still the rescaled form
        sx[:, :] = np.float32(1.0)
        sw[:, :] = np.float32(1.0)
        sx[0:64, 0] = np.float32(2.0 ** -30)
        sx[0:64, 2] = np.float32(2.0 ** 30)
    return xq, sx, wq, meta, sw


@pytest.mark.parametrize("kind", ["wide", "extreme_x_rows", "extreme_w_block", "zero_and_negative", "edge_of_window"])
@pytest.mark.parametrize("packed", [False, True])
def test_scale_products_wide_and_unusual(kind, packed):
    say(f"scale case {kind} packed={packed}")
    xq, sx, wq, meta, sw = scale_case(kind, seed=31)
    ref = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128)
    # T with the magnitudes of the scale products (negative scales flip signs only)
    _, bound = oracle.fp8_sparse24_gemm_groupwise(xq, np.abs(sx), 1, wq, meta, np.abs(sw), 128, bound=True)
    for form in ("y", "yt"):
        got = down(run_gemm(True, xq, sx, 1, wq, meta, sw, 128, torch.float32, form, packed=packed))
        assert_within_tolerance((got.T if form == "yt" else got).astype(np.float64), ref, bound, f"{kind} {form}")
