"""Pins of the oracle's rowwise / tensorwise-scaled GEMMs (scales constant
along K, applied once after the full K sum): exact rational brute force, an
int64 matmul with unit scales, the groupwise oracle with the same scales
repeated over every K block (the promotion sum it factors), the identity
pin, the sparse = dense(decompressed) identity, and the bound T."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def _codes(rng, shape):
    """Random e4m3 codes over the whole finite range (subnormals, both signs, +-448)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01        # no NaN codes
    return c


def _scales(rng, n):
    return (rng.uniform(0.5, 2.0, size=n) * np.exp2(rng.integers(-30, 30, size=n))).astype(np.float32)


@pytest.mark.parametrize("m,n,k,tensor_x,tensor_w", [(3, 2, 128, False, False), (2, 3, 256, True, False),
                                                      (1, 4, 128, False, True), (2, 2, 256, True, True)])
def test_rowwise_matches_exact_rationals(m, n, k, tensor_x, tensor_w):
    rng = np.random.default_rng(7 + m * 10 + n + k)
    xq, wq = _codes(rng, (m, k)), _codes(rng, (n, k))
    sx = _scales(rng, 1 if tensor_x else m)
    sw = _scales(rng, 1 if tensor_w else n)
    y = oracle.fp8_gemm_rowwise(xq, sx, wq, sw)
    xd, wd = oracle.e4m3_decode(xq), oracle.e4m3_decode(wq)
    for i in range(m):
        for j in range(n):
            acc = sum(Fraction(float(xd[i, kk])) * Fraction(float(wd[j, kk])) for kk in range(k))
            exact = Fraction(float(sx[0 if tensor_x else i])) * Fraction(float(sw[0 if tensor_w else j])) * acc
            # one rounding of the exact value to fp64
            assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 52)


def test_rowwise_unit_scales_integer_codes_match_int64():
    rng = np.random.default_rng(11)
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16, 24, 32], dtype=np.int64)
    xi = rng.choice(ints, size=(6, 384)) * rng.choice([-1, 1], size=(6, 384))
    wi = rng.choice(ints, size=(5, 384)) * rng.choice([-1, 1], size=(5, 384))
    xq = oracle.e4m3_encode(xi.astype(np.float32))
    wq = oracle.e4m3_encode(wi.astype(np.float32))
    y = oracle.fp8_gemm_rowwise(xq, np.ones(6, np.float32), wq, np.ones(1, np.float32))
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))


@pytest.mark.parametrize("tensor", [False, True])
def test_rowwise_equals_groupwise_with_scales_repeated_over_k(tensor):
    d = workloads.sparse_large(seed=12, m=20, n=24, k=768)
    xq, sx_g = oracle.fp8_quant_groupwise(d["x"], 1, 768)
    wq, sw_g = oracle.fp8_quant_groupwise(d["w"], 1, 768)
    sx, sw = sx_g[:, 0], sw_g[:, 0]
    if tensor:
        sx, sw = sx[:1], sw[:1]
    kb = 768 // 128
    y, t = oracle.fp8_gemm_rowwise(xq, sx, wq, sw, bound=True)
    sxe = np.repeat(np.broadcast_to(sx, (20,))[:, None], kb, axis=1)
    swe = np.repeat(np.broadcast_to(sw, (24,))[:, None], kb, axis=1)
    yg, tg = oracle.fp8_gemm_groupwise(xq, sxe, 1, wq, swe, 1, bound=True)
    # same real number; the groupwise route rounds once per K block
    assert np.all(np.abs(y - yg) <= 1e-14 * tg)
    assert np.allclose(t, tg, rtol=1e-14, atol=0)


def test_rowwise_identity_gives_scaled_weight():
    rng = np.random.default_rng(13)
    wq = _codes(rng, (5, 128))
    xq = np.zeros((128, 128), np.uint8)
    xq[np.arange(128), np.arange(128)] = 0x38           # 1.0
    sw = _scales(rng, 5)
    y = oracle.fp8_gemm_rowwise(xq, np.ones(1, np.float32), wq, sw)
    assert np.array_equal(y, (oracle.e4m3_decode(wq) * sw[:, None].astype(np.float64)).T)


def test_sparse_rowwise_equals_dense_on_pruned_weight():
    d = workloads.sparse_large(seed=14, m=9, n=16, k=256)
    keep, pruned = oracle.prune24(d["w"])
    wq = oracle.e4m3_encode(pruned * np.float32(64))
    wv, meta2 = oracle.compress24(wq, keep)
    xq = oracle.e4m3_encode(d["x"])
    sx, sw = _scales(np.random.default_rng(15), 9), _scales(np.random.default_rng(16), 16)
    ys = oracle.fp8_sparse24_gemm_rowwise(xq, sx, wv, meta2, sw)
    yd = oracle.fp8_gemm_rowwise(xq, sx, oracle.decompress24(wv, meta2), sw)
    assert np.array_equal(ys, yd)


def test_int8_sparse_rowwise_matches_int64():
    rng = np.random.default_rng(17)
    x = rng.integers(-127, 128, size=(7, 256)).astype(np.int8)
    w = rng.integers(-127, 128, size=(6, 256)).astype(np.int8)
    keep, _ = oracle.prune24(w.astype(np.float32))
    wv, meta = oracle.compress24(w, keep)
    sx, sw = _scales(rng, 7), _scales(rng, 1)
    y = oracle.int8_sparse24_gemm_rowwise(x, sx, wv, meta, sw)
    wd = np.where(keep, w, 0).astype(np.int64)
    ref = (x.astype(np.int64) @ wd.T).astype(np.float64)   # below 2^53: exact
    assert np.array_equal(y, np.outer(sx.astype(np.float64), np.float64(sw[0]) * np.ones(6)) * ref)


def test_rowwise_bound_dominates_and_is_tight_for_nonnegative_codes():
    rng = np.random.default_rng(18)
    xq, wq = _codes(rng, (8, 256)), _codes(rng, (9, 256))
    sx, sw = _scales(rng, 8), _scales(rng, 9)
    y, t = oracle.fp8_gemm_rowwise(xq, sx, wq, sw, bound=True)
    assert np.all(t >= np.abs(y))
    assert np.any(t > 2 * np.abs(y))                    # mixed signs cancel
    xp, wp = xq & 0x7F, wq & 0x7F
    yp, tp = oracle.fp8_gemm_rowwise(xp, sx, wp, sw, bound=True)
    assert np.array_equal(yp, tp)


def test_bias_on_zero_product_is_the_bias_exactly():
    rng = np.random.default_rng(19)
    xq = np.zeros((5, 128), np.uint8)
    wq = _codes(rng, (7, 128))
    bias = (rng.standard_normal(7) * 10).astype(np.float32)
    y, t = oracle.fp8_gemm_rowwise(xq, _scales(rng, 5), wq, _scales(rng, 7), bound=True)
    yb, tb = oracle.add_bias(y, t, bias)
    assert np.array_equal(yb, np.broadcast_to(bias.astype(np.float64), (5, 7)))
    assert np.array_equal(tb, np.abs(yb))


def test_bias_adds_per_output_column_exactly_on_integers():
    rng = np.random.default_rng(20)
    xi = rng.integers(-8, 9, size=(4, 256))
    wi = rng.integers(-8, 9, size=(6, 256))
    bias = rng.integers(-1000, 1000, size=6).astype(np.float32)
    xq, wq = oracle.e4m3_encode(xi.astype(np.float32)), oracle.e4m3_encode(wi.astype(np.float32))
    y, t = oracle.fp8_gemm_rowwise(xq, np.ones(1, np.float32), wq, np.ones(1, np.float32), bound=True)
    yb, tb = oracle.add_bias(y, t, bias)
    assert np.array_equal(yb, (xi @ wi.T + bias.astype(np.int64)[None, :]).astype(np.float64))
    assert np.array_equal(tb, (np.abs(xi) @ np.abs(wi).T + np.abs(bias).astype(np.int64)[None, :]).astype(np.float64))
