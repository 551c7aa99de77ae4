"""Groupwise-scaled FP8 GEMM (dense and 2:4-sparse weight) and the fused
int4 + bf16 add, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Dense FP8 GEMM with groupwise scales, Y = X . W^T, following CUTLASS PR #2095
"Improvements for: Groupwise scaling along M for FP8 gemm":
* hwu36's comment: ScaleGranularityM and ScaleGranularityN are each 1 or 128;
  each 128-wide K block carries its own scale for X (per gM rows) and for W
  (per gN rows);
* hwu36's / manishucsd's review of the promotion interval: the FP8 products of
  one K tile are accumulated from zero (ScaleOut::Zero) and then promoted,
  scaled, into the fp32 accumulators; here once per 128-wide K block.

So, for K block kb covering k in [128 kb, 128 kb + 128):
    P[m, n, kb] = sum_k dec(xq[m, k]) * dec(wq[n, k])            (exact in fp64:
                  every product is an integer multiple of 2^-18 below 2^17.6,
                  and 128 of them sum below 2^24.6, i.e. < 2^43 quanta)
    y[m, n]     = sum_kb (sx[m // gM, kb] * sw[n // gN, kb]) * P[m, n, kb]
The scale product of two fp32 values is exact in fp64.

The 2:4-sparse GEMM is the same GEMM on the decompressed weight: the
compressed values and metadata stand for the dense pruned weight (torchao PR
#3258 "Introduce new W8A8-FP-CSR quantization API", jcaip's comment that a
sparse tensor is dequantised by multiplying it with an identity matrix, i.e.
it *is* the dense matrix it encodes).

The swapped form of CUTLASS issue #2029 ("[QST] CUTLASS support for fp8 sparse
matrix (for W) ...", klevzoff's swap+transpose answer) is C^T = B^T . A^T:
Y^T[n, m] = y[m, n].  It needs no function of its own: calling the dense GEMM
with the operands exchanged gives the transpose bit for bit (pinned by a test).

Fused add (CUTLASS issue #2058, "[QST] How to implement a fused mixed
precision matrix multiplication such as w4a4 + w16a16?", hyx1999's statement:
Y = X1 W1^T + X2 W2^T with X1, W1 quantised to 4 bit):
    y = sum_kb sx1[m, kb] * sw1[n, kb] * sum_{k in kb} int4(x1) int4(w1)
        + sum_{k < K2} bf16(x2[m, k]) * bf16(w2[n, k])

int8 x int8 with the same groupwise scales (the other 2:4 kernel torchao PR
#3258 names, jcaip's comment): the same sum with int8 codes; every 128-term
partial is an integer below 2^21, exact in fp64.

Scales constant along K (rowwise: one scale per X row and per W row;
tensorwise: one per tensor).  The weight quantisation code quoted in torchao
PR #3258 expands one scale per weight row across all of that row's columns,
and jcaip's review asks for the kernels that fuse the scale multiplication
into the GEMM.  With s independent of kb the promotion sum factors,
    y[m, n] = sx[m] * sw[n] * sum_k dec(xq[m, k]) * dec(wq[n, k]),
so the scale can be applied once, after the whole K sum.  The full-K sum is
still exact in fp64 (integer multiples of 2^-18 below 2^(17.6 + log2 K) <
2^53 quanta for K < 2^17).

Weight-only 2:4 GEMM (W8A16): bf16 activations, unquantised, times a 2:4
weight of 8-bit codes (e4m3 or int8) with groupwise scales.  torchao PR
#3258's review (jcaip) says weight-only sparsity configs for int8 and float8
have no mixed-dtype kernel to run on; this is that operation:
    y[m, n] = sum_kb sw[n // gN, kb] * sum_{k in kb} bf16(x[m, k]) * dec(wq[n, k])
Every product is exact in fp64 (8 x 8 significant bits); the K-block sums are
exact up to fp64 rounding (relative 2^-53 of the block's abs-sum).

W4A16 is the same with 4-bit codes: the 2:4-compressed values quantised to
int4 (one scale per row and 128-wide K block, i.e. per 64 compressed values),
packed two per byte, element 2j in the low nibble of byte j.

Bias epilogue: the sparse FP8 linear implementation torchao PR #3258's review
points to takes a bias argument; a linear layer adds it to every row of the
output, y[m, n] + bias[n], after the scales.  In the tolerance the bias is one
more term of the abs-sum with scale 1 (like the bf16 part of the fused add).

Tolerance (the accepted error of a GPU result g against the oracle y):
    |g - y| <= 1e-2 |y| + 1e-3 T,
    T[m, n] = sum_kb s(m, n, kb) * sum_{k in kb} |dec x * dec w|  (+ sum |x2 w2|).
"""

import numpy as np

from .bf16 import bf16_decode
from .e4m3 import e4m3_decode
from .quant import int4_decode
from .sparse24 import decompress24

KBLK = 128


def expand_scales(s, g: int, rows: int) -> np.ndarray:
    """Scale array [ceil(rows/g), KB] -> one row per matrix row, fp64 [rows, KB]."""
    s = np.asarray(s, dtype=np.float32)
    return np.repeat(s, g, axis=0)[:rows].astype(np.float64)


def _scaled_kblock_sum(xd, sxe, wd, swe, absolute: bool):
    m, k = xd.shape
    n = wd.shape[0]
    assert k % KBLK == 0 and wd.shape[1] == k
    y = np.zeros((m, n), dtype=np.float64)
    for kb in range(k // KBLK):
        ks = slice(kb * KBLK, (kb + 1) * KBLK)
        xs, ws = xd[:, ks], wd[:, ks]
        if absolute:
            xs, ws = np.abs(xs), np.abs(ws)
        p = xs @ ws.T                                   # exact partial of this K block
        y += np.outer(sxe[:, kb], swe[:, kb]) * p       # promote with the block's scales
    return y


def fp8_gemm_groupwise(xq, sx, gm: int, wq, sw, gn: int, bound: bool = False):
    """xq [M, K] e4m3 codes, sx fp32 [ceil(M/gm), K/128]; wq [N, K] codes,
    sw fp32 [ceil(N/gn), K/128].  Returns y fp64 [M, N] (and T if bound)."""
    xq = np.asarray(xq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    m, k = xq.shape
    n = wq.shape[0]
    assert gm in (1, 128) and gn in (1, 128)
    xd, wd = e4m3_decode(xq), e4m3_decode(wq)
    sxe, swe = expand_scales(sx, gm, m), expand_scales(sw, gn, n)
    assert sxe.shape == (m, k // KBLK) and swe.shape == (n, k // KBLK)
    y = _scaled_kblock_sum(xd, sxe, wd, swe, absolute=False)
    if not bound:
        return y
    return y, _scaled_kblock_sum(xd, sxe, wd, swe, absolute=True)


def fp8_sparse24_gemm_groupwise(xq, sx, gm: int, wv, wmeta, sw, gn: int, bound: bool = False):
    """Same as ``fp8_gemm_groupwise`` with W given as 2:4 compressed codes
    wv [N, K/2] and metadata wmeta [N, K/8]."""
    wq = decompress24(np.asarray(wv, dtype=np.uint8), wmeta)
    return fp8_gemm_groupwise(xq, sx, gm, wq, sw, gn, bound=bound)


def int8_gemm_groupwise(xq, sx, gm: int, wq, sw, gn: int, bound: bool = False):
    """xq [M, K] int8 codes, sx fp32 [ceil(M/gm), K/128]; wq [N, K] int8 codes,
    sw fp32 [ceil(N/gn), K/128].  Returns y fp64 [M, N] (and T if bound)."""
    xd = np.asarray(xq, dtype=np.int8).astype(np.float64)
    wd = np.asarray(wq, dtype=np.int8).astype(np.float64)
    m, k = xd.shape
    n = wd.shape[0]
    assert gm in (1, 128) and gn in (1, 128)
    sxe, swe = expand_scales(sx, gm, m), expand_scales(sw, gn, n)
    assert sxe.shape == (m, k // KBLK) and swe.shape == (n, k // KBLK)
    y = _scaled_kblock_sum(xd, sxe, wd, swe, absolute=False)
    if not bound:
        return y
    return y, _scaled_kblock_sum(xd, sxe, wd, swe, absolute=True)


def int8_sparse24_gemm_groupwise(xq, sx, gm: int, wv, wmeta, sw, gn: int, bound: bool = False):
    """``int8_gemm_groupwise`` with W given as 2:4 compressed int8 codes
    wv [N, K/2] and metadata wmeta [N, K/8]."""
    wq = decompress24(np.asarray(wv, dtype=np.int8).view(np.uint8), wmeta).view(np.int8)
    return int8_gemm_groupwise(xq, sx, gm, wq, sw, gn, bound=bound)


def _row_scales(s, rows: int) -> np.ndarray:
    """One fp32 scale per row ([rows]) or one for the tensor ([1]) -> fp64 [rows]."""
    s = np.asarray(s, dtype=np.float32).reshape(-1)
    assert s.shape[0] in (1, rows)
    return np.broadcast_to(s, (rows,)).astype(np.float64)


def _rowwise(xd, sx, wd, sw, bound: bool):
    m, k = xd.shape
    n = wd.shape[0]
    assert wd.shape[1] == k and k % KBLK == 0 and k < (1 << 17)
    s = np.outer(_row_scales(sx, m), _row_scales(sw, n))   # exact fp32 x fp32 products
    y = s * (xd @ wd.T)                                     # exact full-K sum, one rounding
    if not bound:
        return y
    return y, s * (np.abs(xd) @ np.abs(wd).T)


def fp8_gemm_rowwise(xq, sx, wq, sw, bound: bool = False):
    """xq [M, K] e4m3 codes with sx fp32 [M] (rowwise) or [1] (tensorwise);
    wq [N, K] codes with sw fp32 [N] or [1].  y = sx[m] sw[n] sum_k x w, fp64."""
    xd = e4m3_decode(np.asarray(xq, dtype=np.uint8))
    wd = e4m3_decode(np.asarray(wq, dtype=np.uint8))
    return _rowwise(xd, sx, wd, sw, bound)


def fp8_sparse24_gemm_rowwise(xq, sx, wv, wmeta, sw, bound: bool = False):
    """``fp8_gemm_rowwise`` with W as 2:4 compressed codes wv [N, K/2] + wmeta [N, K/8]."""
    wq = decompress24(np.asarray(wv, dtype=np.uint8), wmeta)
    return fp8_gemm_rowwise(xq, sx, wq, sw, bound=bound)


def int8_sparse24_gemm_rowwise(xq, sx, wv, wmeta, sw, bound: bool = False):
    """Rowwise / tensorwise scales with int8 codes and a 2:4 compressed int8 W."""
    wq = decompress24(np.asarray(wv, dtype=np.int8).view(np.uint8), wmeta).view(np.int8)
    xd = np.asarray(xq, dtype=np.int8).astype(np.float64)
    return _rowwise(xd, sx, wq.astype(np.float64), sw, bound)


def w8a16_sparse24_gemm_groupwise(x_bits, wv, wmeta, sw, gn: int, codes: str = "e4m3", bound: bool = False):
    """x_bits bf16 bits [M, K]; wv [N, K/2] 2:4 compressed codes (e4m3 bytes, or
    int8) with metadata wmeta [N, K/8] and scales sw [ceil(N/gn), K/128]."""
    assert codes in ("e4m3", "int8") and gn in (1, 128)
    xd = bf16_decode(x_bits)
    wq = decompress24(np.asarray(wv).view(np.uint8), wmeta)
    wd = e4m3_decode(wq) if codes == "e4m3" else wq.view(np.int8).astype(np.float64)
    m, k = xd.shape
    n = wd.shape[0]
    swe = expand_scales(sw, gn, n)
    assert swe.shape == (n, k // KBLK) and wd.shape[1] == k
    ones = np.ones((m, k // KBLK), dtype=np.float64)
    y = _scaled_kblock_sum(xd, ones, wd, swe, absolute=False)
    if not bound:
        return y
    return y, _scaled_kblock_sum(xd, ones, wd, swe, absolute=True)


def w4a16_sparse24_gemm_groupwise(x_bits, wv4, wmeta, sw, bound: bool = False):
    """x_bits bf16 bits [M, K]; wv4 packed int4 [N, K/4] (the 2:4-compressed
    values, two per byte); wmeta [N, K/8]; sw fp32 [N, K/128] (one per row and K block)."""
    codes = int4_decode(wv4).astype(np.int8)                       # [N, K/2]
    return w8a16_sparse24_gemm_groupwise(x_bits, codes, wmeta, sw, 1, "int8", bound=bound)


def add_bias(y, bound, bias):
    """The bias epilogue: y [M, N] fp64 (and its bound T) plus bias fp32 [N]
    on every row; returns (y + bias, T + |bias|)."""
    b = np.asarray(bias, dtype=np.float32).astype(np.float64).reshape(1, -1)
    assert b.shape[1] == y.shape[1]
    return y + b, bound + np.abs(b)


def mixed_gemm_add(x1p, sx1, w1p, sw1, x2, w2, bound: bool = False):
    """x1p int4 [M, K1/2], sx1 fp32 [M, K1/128]; w1p int4 [N, K1/2],
    sw1 fp32 [N, K1/128]; x2 bf16 bits [M, K2]; w2 bf16 bits [N, K2]."""
    x1 = int4_decode(x1p).astype(np.float64)
    w1 = int4_decode(w1p).astype(np.float64)
    m, n = x1.shape[0], w1.shape[0]
    sxe, swe = expand_scales(sx1, 1, m), expand_scales(sw1, 1, n)
    x2d, w2d = bf16_decode(x2), bf16_decode(w2)
    y = _scaled_kblock_sum(x1, sxe, w1, swe, absolute=False) + x2d @ w2d.T
    if not bound:
        return y
    t = _scaled_kblock_sum(x1, sxe, w1, swe, absolute=True) + np.abs(x2d) @ np.abs(w2d).T
    return y, t


def within_tolerance(got, ref, bound, rel: float = 1e-2, absf: float = 1e-3) -> np.ndarray:
    """Elementwise |got - ref| <= rel |ref| + absf T."""
    got = np.asarray(got, dtype=np.float64)
    return np.abs(got - ref) <= rel * np.abs(ref) + absf * bound
