"""Exact GPU parity where the arithmetic is exact.

With integer-valued codes of small magnitude (|v| <= 3: exact e4m3, int8 and
bf16 numbers), power-of-two scales in [1/2, 2] and fp32 output, every product,
every 128-wide K-block sum, every promotion and every partial sum of the GEMM
is an exactly representable fp32 number (sums stay below 2^21 on a grid of
2^-2), whatever the order of accumulation.  The oracle's fp64 value is then
the only correct fp32 result, and the kernels must reproduce it bit for bit:
a dropped term, a wrong sign, a transposed operand or a scale applied to the
wrong K block changes at least one output by at least one grid step, which the
tolerance tests at full K cannot always see.

The inputs are the seeded draws of ``workloads.exact_ints`` (codes made by the
oracle's e4m3 encoder and 2:4 compressor).  Every kernel family is covered:
dense and 2:4 large-M (canonical and packed, both output forms), the decode
kernels, K = 16384, int8 codes, batched and grouped problems, scales constant
along K, the weight-only kernels and the fused int4 + bf16 add, including the
full 2048 x 4096 x 4096 size with every output checked.  The torchao PR
"Introduce new W8A8-FP-CSR quantization API" states one such exact case itself
(jcaip: a sparse tensor is dequantised by multiplying it with an identity);
these tests generalise it.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import down, say, up, up_scales

pytestmark = pytest.mark.gpu


def operands(seed, m, n, k, int8=False, gm=1, gn=128):
    d = workloads.exact_ints(seed, m, n, k, x_scale_rows=-(-m // gm), w_scale_rows=-(-n // gn))
    wv32, meta = oracle.prune_compress24(d["w"])
    if int8:
        xq, wq = d["x"].astype(np.int8), wv32.astype(np.int8)
    else:
        xq, wq = oracle.e4m3_encode(d["x"]), oracle.e4m3_encode(wv32)
    return xq, d["sx"], wq, meta, d["sw"]


def assert_exact(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    bad = np.argwhere(got != ref)
    if len(bad):
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} of {ref.size} outputs differ; first ({i},{j}) got {got[i, j]!r} "
                             f"ref {ref[i, j]!r}")
    say(f"  {what}: all {ref.size} outputs exact")


def gpu_sparse(kind, xq, sx, wq, meta, sw, gm, gn, form, int8=False):
    n = wq.shape[0]
    if kind == "packed":
        wp = up(oracle.pack24_gfx950(wq.view(np.uint8), meta))
        f = sg.int8_sparse24_gemm_groupwise_packed if int8 else sg.fp8_sparse24_gemm_groupwise_packed
        return f(up(xq), up_scales(sx), wp, n, up_scales(sw), gm, gn, out_dtype=torch.float32, form=form)
    f = sg.int8_sparse24_gemm_groupwise if int8 else sg.fp8_sparse24_gemm_groupwise
    return f(up(xq), up_scales(sx), up(wq), up(meta), up_scales(sw), gm, gn, out_dtype=torch.float32, form=form)


def check_sparse(kind, m, n, k, seed, gm=1, gn=128, int8=False, forms=("y", "yt")):
    say(f"exact {kind} {'int8' if int8 else 'e4m3'} M={m} N={n} K={k} gm={gm} gn={gn} seed={seed}")
    xq, sx, wq, meta, sw = operands(seed, m, n, k, int8, gm, gn)
    f = oracle.int8_sparse24_gemm_groupwise if int8 else oracle.fp8_sparse24_gemm_groupwise
    ref = f(xq, sx, gm, wq, meta, sw, gn)
    for form in forms:
        got = down(gpu_sparse(kind, xq, sx, wq, meta, sw, gm, gn, form, int8))
        assert_exact(got.T if form == "yt" else got, ref, f"{kind} form={form}")


@pytest.mark.parametrize("kind", ["canonical", "packed"])
@pytest.mark.parametrize("m,n,k", [(300, 512, 1024), (129, 300, 384), (1, 256, 128), (16, 1024, 2048),
                                   (37, 640, 1152), (64, 256, 512), (65, 384, 256)])
def test_sparse_exact(kind, m, n, k):
    check_sparse(kind, m, n, k, seed=m + n + k)


@pytest.mark.parametrize("gm,gn", [(1, 1), (128, 1), (128, 128)])
@pytest.mark.parametrize("m", [37, 300])
def test_sparse_exact_granularities(gm, gn, m):
    check_sparse("canonical", m, 384, 512, seed=7 + gm + gn, gm=gm, gn=gn)


@pytest.mark.parametrize("m,n,k", [(300, 512, 1024), (16, 1024, 2048), (37, 512, 1024)])
def test_int8_sparse_exact(m, n, k):
    check_sparse("canonical", m, n, k, seed=3 * m, int8=True)
    check_sparse("packed", m, n, k, seed=3 * m, int8=True)


@pytest.mark.parametrize("m", [16, 37, 300])
def test_long_k_exact(m):
    """K = 16384 (128 K blocks): large-M kernel and decode ring."""
    check_sparse("packed", m, 512, 16384, seed=41 + m, forms=("y",))


@pytest.mark.parametrize("m,n,k", [(16, 4096, 14336), (37, 14336, 4096)])
def test_decode_shapes_exact(m, n, k):
    check_sparse("packed", m, n, k, seed=m, forms=("y", "yt"))


def test_sparse_full_size_exact():
    """2048 x 4096 x 4096 2:4, packed weight, every output exact (Y and Y^T)."""
    check_sparse("packed", 2048, 4096, 4096, seed=3)


@pytest.mark.parametrize("m,n,k", [(300, 512, 1024), (37, 384, 512), (2048, 4096, 4096)])
def test_dense_exact(m, n, k):
    say(f"exact dense M={m} N={n} K={k}")
    xq, sx, wq, meta, sw = operands(11, m, n, k)
    wd = oracle.decompress24(wq, meta)
    ref = oracle.fp8_gemm_groupwise(xq, sx, 1, wd, sw, 128)
    for form in ("y", "yt"):
        got = down(sg.fp8_gemm_groupwise(up(xq), up_scales(sx), up(wd), up_scales(sw), 1, 128, out_dtype=torch.float32,
                                         form=form))
        assert_exact(got.T if form == "yt" else got, ref, f"dense form={form}")


@pytest.mark.parametrize("kind", ["dense", "sparse", "packed"])
@pytest.mark.parametrize("m", [16, 300, 2048])
def test_rowwise_exact(kind, m):
    """Scales constant along K (one power of two per row), applied after the K loop."""
    n, k = 1024 if m == 2048 else 512, 4096 if m == 2048 else 1024
    say(f"exact rowwise {kind} M={m} N={n} K={k}")
    xq, sx, wq, meta, sw = operands(23, m, n, k, gn=1)
    sxr, swr = sx[:, 0].copy(), sw[:, 0].copy()
    sxt, swt = sg.k_constant_scales(up(sxr), m, k), sg.k_constant_scales(up(swr), n, k)
    if kind == "dense":
        wd = oracle.decompress24(wq, meta)
        ref = oracle.fp8_gemm_rowwise(xq, sxr, wd, swr)
        got = sg.fp8_gemm_groupwise(up(xq), sxt, up(wd), swt, 1, 1, out_dtype=torch.float32)
    else:
        ref = oracle.fp8_sparse24_gemm_rowwise(xq, sxr, wq, meta, swr)
        if kind == "sparse":
            got = sg.fp8_sparse24_gemm_groupwise(up(xq), sxt, up(wq), up(meta), swt, 1, 1, out_dtype=torch.float32)
        else:
            wp = sg.sparse24_pack_gfx950(up(wq), up(meta))
            got = sg.fp8_sparse24_gemm_groupwise_packed(up(xq), sxt, wp, n, swt, 1, 1, out_dtype=torch.float32)
    assert_exact(down(got), ref, f"rowwise {kind}")


@pytest.mark.parametrize("kind", ["dense", "sparse", "packed"])
def test_batched_exact(kind):
    L, m, n, k = 3, 200, 384, 512
    say(f"exact batched {kind} L={L} M={m} N={n} K={k}")
    ops = [operands(60 + z, m, n, k) for z in range(L)]
    xq = np.stack([o[0] for o in ops])
    sx = np.stack([o[1] for o in ops])
    wq = np.stack([o[2] for o in ops])
    meta = np.stack([o[3] for o in ops])
    sw = np.stack([o[4] for o in ops])

    def sc3(s):   # [L, rows, KB] stored M-major per problem
        return torch.from_numpy(np.ascontiguousarray(s.transpose(0, 2, 1))).cuda().transpose(1, 2)

    if kind == "dense":
        wd = np.stack([oracle.decompress24(wq[z], meta[z]) for z in range(L)])
        got = sg.fp8_gemm_groupwise_batched(up(xq), sc3(sx), up(wd), sc3(sw), 1, 128, out_dtype=torch.float32)
    elif kind == "sparse":
        got = sg.fp8_sparse24_gemm_groupwise_batched(up(xq), sc3(sx), up(wq), up(meta), sc3(sw), 1, 128,
                                                     out_dtype=torch.float32)
    else:
        wp = torch.stack([sg.sparse24_pack_gfx950(up(wq[z]), up(meta[z])) for z in range(L)])
        got = sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), sc3(sx), wp, n, sc3(sw), 1, 128,
                                                            out_dtype=torch.float32)
    got = down(got)
    for z in range(L):
        ref = oracle.fp8_sparse24_gemm_groupwise(xq[z], sx[z], 1, wq[z], meta[z], sw[z], 128)
        assert_exact(got[z], ref, f"batched {kind} z={z}")


@pytest.mark.parametrize("sizes", [[300, 0, 17, 128, 250], [3, 9, 16, 1, 12, 5, 16, 2], [400, 120, 310, 64]])
def test_grouped_exact(sizes):
    """Grouped 2:4 GEMM (one packed weight per group; large tiles, group
    tails on the decode body, or the decode kernel for small groups)."""
    n, k = 512, 1024
    say(f"exact grouped sizes={sizes} N={n} K={k}")
    msum = sum(sizes)
    xq, sx, _, _, _ = operands(70, msum, 8, k)
    ws = [operands(71 + g, 8, n, k) for g in range(len(sizes))]
    wp = torch.stack([sg.sparse24_pack_gfx950(up(w[2]), up(w[3])) for w in ws])
    swg = np.stack([w[4] for w in ws])
    sw3 = torch.from_numpy(np.ascontiguousarray(swg.transpose(0, 2, 1))).cuda().transpose(1, 2)
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_grouped(up(xq), up_scales(sx), sizes, wp, n, sw3, 128,
                                                             out_dtype=torch.float32))
    r0 = 0
    for g, mg in enumerate(sizes):
        if mg:
            ref = oracle.fp8_sparse24_gemm_groupwise(xq[r0:r0 + mg], sx[r0:r0 + mg], 1, ws[g][2], ws[g][3], ws[g][4], 128)
            assert_exact(got[r0:r0 + mg], ref, f"grouped g={g} rows={mg}")
        r0 += mg


@pytest.mark.parametrize("codes", ["e4m3", "int8"])
@pytest.mark.parametrize("m,n,k", [(16, 1024, 2048), (37, 512, 1024), (300, 512, 1024), (2048, 4096, 4096)])
def test_weight_only_exact(codes, m, n, k):
    """Weight-only 2:4: bf16 integer activations times integer codes with
    power-of-two W scales; the large-M tile kernel at full size, every row."""
    say(f"exact w8a16 {codes} M={m} N={n} K={k}")
    xq, _, wq, meta, sw = operands(90 + m, m, n, k, int8=codes == "int8")
    xb = workloads.to_bf16_bits(xq.astype(np.float32) if codes == "int8" else oracle.e4m3_decode(xq).astype(np.float32))
    ref = oracle.w8a16_sparse24_gemm_groupwise(xb, wq, meta, sw, 128, codes=codes)
    got = down(sg.w8a16_sparse24_gemm_groupwise(up(xb), up(wq), up(meta), up_scales(sw), 128, out_dtype=torch.float32))
    assert_exact(got, ref, f"w8a16 {codes}")


def test_mixed_add_exact():
    """Fused int4 + bf16 add: int4 codes equal to integer inputs (every
    (row, 128-group) holds a 7, so the int4 quantiser's scale is exactly 1),
    bf16 integer X2, W2."""
    m, n, k1, k2 = 300, 512, 1024, 64
    gen = workloads.generators(95, 4)
    x1 = workloads.small_ints(gen[0], (m, k1), 7)
    w1 = workloads.small_ints(gen[1], (n, k1), 7)
    x1[:, ::128] = 7.0
    w1[:, ::128] = 7.0
    x1p, sx1 = oracle.int4_quant_groupwise(x1, 128)
    w1p, sw1 = oracle.int4_quant_groupwise(w1, 128)
    assert (sx1 == 1).all() and (sw1 == 1).all()
    x2 = workloads.to_bf16_bits(workloads.small_ints(gen[2], (m, k2), 3))
    w2 = workloads.to_bf16_bits(workloads.small_ints(gen[3], (n, k2), 3))
    ref = oracle.mixed_gemm_add(x1p, sx1, w1p, sw1, x2, w2)
    y = sg.mixed_gemm_add(up(x1p), up_scales(sx1), up(w1p), up_scales(sw1), up(x2), up(w2))
    # bf16 output: the exact sums are integers below 2^17, so compare after the
    # oracle's value is rounded to bf16 the way a correct kernel rounds it
    ref_bf16 = oracle.bf16_decode(workloads.to_bf16_bits(ref.astype(np.float32)))
    assert np.abs(ref).max() < 2 ** 24
    assert_exact(down(y), ref_bf16, "mixed add (bf16 of the exact sum)")
