"""Pins of the oracle's int8 path (the int8 x int8 2:4-sparse GEMM with the
FP8 path's groupwise scales): the quantiser against an independent torch
route, exact power-of-two round trips, the half-step error bound, ties to
even, the all-zero block; the GEMMs against exact rational brute force, an
int64 matmul with unit scales, and the sparse = dense(decompressed) identity."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


@pytest.mark.parametrize("gr,gc,shape", [(1, 128, (5, 384)), (128, 64, (300, 128)), (128, 128, (130, 256)),
                                         (1, 64, (3, 192))])
def test_int8_quant_matches_torch_route(gr, gc, shape):
    rng = np.random.default_rng(41 + gr + gc)
    x = (rng.standard_normal(shape) * np.exp2(rng.uniform(-8, 8, size=(shape[0], 1)))).astype(np.float32)
    codes, s = oracle.int8_quant_groupwise(x, gr, gc)
    rows, cols = shape
    rb = -(-rows // gr)
    t = torch.zeros((rb * gr, cols), dtype=torch.float32)
    t[:rows] = torch.from_numpy(x)
    tb = t.view(rb, gr, cols // gc, gc)
    a = tb.abs().amax(dim=(1, 3), keepdim=True)
    ts = torch.where(a > 0, a / torch.tensor(127.0), torch.ones_like(a))
    q = torch.clamp(torch.round(tb / ts), -127, 127).view(rb * gr, cols)[:rows].to(torch.int8)
    assert np.array_equal(s, ts.view(rb, cols // gc).numpy())
    assert np.array_equal(codes, q.numpy())


def test_int8_power_of_two_roundtrip_is_exact():
    rng = np.random.default_rng(42)
    q = rng.integers(-127, 128, size=(4, 256))
    q[:, 5] = 127
    q[:, 200] = -127
    j = rng.integers(-20, 20, size=(4, 2))
    v = (q * np.repeat(np.exp2(j), 128, axis=1)).astype(np.float32)   # amax = 127 * 2^j, s = 2^j
    codes, s = oracle.int8_quant_groupwise(v, 1, 128)
    assert np.array_equal(s, np.exp2(j).astype(np.float32))
    assert np.array_equal(codes.astype(np.int64), q)


def test_int8_every_nonzero_block_reaches_127_and_error_within_half_step():
    x = workloads.sparse_large(seed=43, m=40, n=8, k=512)["x"]
    x[3, 128:256] = 0.0
    codes, s = oracle.int8_quant_groupwise(x, 1, 128)
    c = codes.astype(np.int64).reshape(40, 4, 128)
    amax = np.abs(c).max(axis=2)
    assert np.all((amax == 127) | ((amax == 0) & (s == 1.0)))
    assert s[3, 1] == 1.0 and not c[3, 1].any()
    deq = c * s[:, :, None].astype(np.float64)
    err = np.abs(deq - x.reshape(40, 4, 128).astype(np.float64))
    # half a step, plus the fp32 rounding of v / s (relative 2^-24 of |v| / s steps)
    assert np.all(err <= s[:, :, None] * (0.5 + 127 * 2.0 ** -23))


def test_int8_ties_round_to_even():
    # amax = 127 gives s = 1 exactly: v = k + 0.5 divides exactly and must go to the even neighbour
    v = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5] + [0.0] * 120], dtype=np.float32)
    codes, s = oracle.int8_quant_groupwise(v, 1, 128)
    assert s[0, 0] == 1.0
    assert codes[0, :8].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def _fraction_gemm(xq, sx, gm, wq, sw, gn):
    """Exact y = sum_kb sx*sw*sum_k x*w and the sum of the blocks' magnitudes."""
    m, k = xq.shape
    n = wq.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    mag = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc, a = Fraction(0), Fraction(0)
            for kb in range(k // 128):
                p = sum(int(xq[i, q]) * int(wq[j, q]) for q in range(kb * 128, kb * 128 + 128))
                t = Fraction(float(sx[i // gm, kb])) * Fraction(float(sw[j // gn, kb])) * p
                acc += t
                a += abs(t)
            out[i][j], mag[i][j] = acc, a
    return out, mag


@pytest.mark.parametrize("m,n,k,gm,gn", [(3, 4, 128, 1, 1), (4, 2, 256, 1, 128), (2, 3, 384, 128, 1)])
def test_int8_exact_rational_brute_force(m, n, k, gm, gn):
    rng = np.random.default_rng(m * 31 + n * 7 + k)
    xq = workloads.random_int8_codes(rng, (m, k))
    wq = workloads.random_int8_codes(rng, (n, k))
    sx = workloads.random_scales(rng, (-(-m // gm), k // 128))
    sw = workloads.random_scales(rng, (-(-n // gn), k // 128))
    y = oracle.int8_gemm_groupwise(xq, sx, gm, wq, sw, gn)
    ref, mag = _fraction_gemm(xq, sx, gm, wq, sw, gn)
    for i in range(m):
        for j in range(n):
            # the partials are exact integers and the scale products exact, so the
            # only error is fp64 accumulation over the K blocks: a few ulps of the
            # magnitudes summed
            assert abs(Fraction(y[i, j]) - ref[i][j]) <= mag[i][j] * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_int8_unit_scales_match_int64_matmul():
    rng = np.random.default_rng(44)
    xq = workloads.random_int8_codes(rng, (7, 512))
    wq = workloads.random_int8_codes(rng, (9, 512))
    one = np.ones((7, 4), np.float32), np.ones((9, 4), np.float32)
    y = oracle.int8_gemm_groupwise(xq, one[0], 1, wq, one[1], 1)
    assert np.array_equal(y, (xq.astype(np.int64) @ wq.astype(np.int64).T).astype(np.float64))


def test_int8_sparse_equals_dense_on_decompressed_weight():
    d = workloads.sparse_large(seed=45, m=20, n=24, k=256)
    wv32, meta = oracle.prune_compress24(d["w"])
    wv, sw = oracle.int8_quant_groupwise(wv32, 128, 64)
    xq, sx = oracle.int8_quant_groupwise(d["x"], 1, 128)
    ys = oracle.int8_sparse24_gemm_groupwise(xq, sx, 1, wv, meta, sw, 128)
    wd = oracle.decompress24(wv.view(np.uint8), meta).view(np.int8)
    yd = oracle.int8_gemm_groupwise(xq, sx, 1, wd, sw, 128)
    assert np.array_equal(ys, yd)
    # the pruned positions are zero codes, the kept ones are the quantised kept values
    assert not wd.reshape(24, 64, 4).astype(bool).sum(axis=2).max() > 2
