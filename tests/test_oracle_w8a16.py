"""Pins of the oracle's weight-only 2:4 GEMM (bf16 activations x 8-bit 2:4
weight codes, groupwise weight scales): exact rational brute force, an int64
matmul for integer activations and int8 codes with unit scales, and the FP8
2:4 GEMM when the activations are e4m3 values (unit X scales)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def bf16_bits(v):
    """Round-to-nearest-even fp32 -> bf16 bits (the inputs are chosen finite)."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def sparse_codes(rng, n, k, int8):
    w = rng.standard_normal((n, k)).astype(np.float32)
    keep, _ = oracle.prune24(w)
    if int8:
        c = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    else:
        c = rng.integers(0, 256, size=(n, k)).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] ^= 1
    return oracle.compress24(c, keep)


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("gn", [1, 128])
def test_w8a16_matches_exact_rationals(int8, gn):
    rng = np.random.default_rng(5 + int8 + gn)
    m, n, k = 3, 2, 256
    x = bf16_bits(rng.standard_normal((m, k)) * np.exp2(rng.integers(-6, 6, size=(m, 1))))
    wv, meta = sparse_codes(rng, n, k, int8)
    sw = (rng.uniform(0.5, 2, size=(1 if gn == 128 else n, k // 128)) * 2.0 ** -7).astype(np.float32)
    y = oracle.w8a16_sparse24_gemm_groupwise(x, wv, meta, sw, gn, "int8" if int8 else "e4m3")
    xd = oracle.bf16_decode(x)
    wq = oracle.decompress24(wv.view(np.uint8), meta)
    wd = wq.view(np.int8).astype(np.float64) if int8 else oracle.e4m3_decode(wq)
    for i in range(m):
        for j in range(n):
            exact, absum = Fraction(0), Fraction(0)
            for kb in range(k // 128):
                s = Fraction(float(sw[0 if gn == 128 else j, kb]))
                prods = [Fraction(float(xd[i, kk])) * Fraction(float(wd[j, kk])) for kk in range(kb * 128, kb * 128 + 128)]
                exact += s * sum(prods)
                absum += s * sum(abs(p) for p in prods)
            # fp64 rounding of the block sums and of their scaled sum only
            assert abs(Fraction(float(y[i, j])) - exact) <= absum * Fraction(1, 2 ** 46)


def test_w8a16_integer_activations_int8_codes_unit_scales():
    rng = np.random.default_rng(9)
    m, n, k = 5, 6, 384
    xi = rng.integers(-50, 51, size=(m, k))
    wv, meta = sparse_codes(rng, n, k, True)
    y = oracle.w8a16_sparse24_gemm_groupwise(bf16_bits(xi.astype(np.float32)), wv, meta,
                                             np.ones((n, k // 128), np.float32), 1, "int8")
    wd = oracle.decompress24(wv.view(np.uint8), meta).view(np.int8).astype(np.int64)
    assert np.array_equal(y, (xi @ wd.T).astype(np.float64))


def test_w8a16_equals_fp8_gemm_on_e4m3_activations():
    d = workloads.sparse_large(seed=11, m=7, n=256, k=512)
    xq = oracle.e4m3_encode(d["x"])
    wv32, meta = oracle.prune_compress24(d["w"])
    wq, sw = oracle.fp8_quant_groupwise(wv32, 128, 64)
    x_bits = bf16_bits(oracle.e4m3_decode(xq).astype(np.float32))     # e4m3 values are exact in bf16
    y, t = oracle.w8a16_sparse24_gemm_groupwise(x_bits, wq, meta, sw, 128, "e4m3", bound=True)
    ones = np.ones((7, 512 // 128), np.float32)
    yf, tf = oracle.fp8_sparse24_gemm_groupwise(xq, ones, 1, wq, meta, sw, 128, bound=True)
    assert np.array_equal(y, yf) and np.array_equal(t, tf)


def test_w4a16_matches_exact_rationals():
    """The int4 path from its packed bytes: nibble order, sign, decompression
    and per-row scales against exact rationals written out here."""
    rng = np.random.default_rng(31)
    m, n, k = 2, 3, 256
    x = bf16_bits(rng.standard_normal((m, k)))
    q = rng.integers(-7, 8, size=(n, k))
    keep, _ = oracle.prune24(rng.standard_normal((n, k)).astype(np.float32))
    qv, meta = oracle.compress24(q.astype(np.int8), keep)             # [n, k/2] values
    nib = (qv.astype(np.int64) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)   # element 2j low nibble
    sw = (rng.uniform(0.5, 2, size=(n, k // 128)) * 2.0 ** -3).astype(np.float32)
    y = oracle.w4a16_sparse24_gemm_groupwise(x, packed, meta, sw)
    xd = oracle.bf16_decode(x)
    qd = np.where(keep, q, 0)
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            for kb in range(k // 128):
                part = sum(Fraction(float(xd[i, kk])) * int(qd[j, kk]) for kk in range(kb * 128, kb * 128 + 128))
                exact += Fraction(float(sw[j, kb])) * part
            absum = sum(Fraction(float(sw[j, kk // 128])) * abs(Fraction(float(xd[i, kk]))) * abs(int(qd[j, kk]))
                        for kk in range(k))
            assert abs(Fraction(float(y[i, j])) - exact) <= absum * Fraction(1, 2 ** 46)
