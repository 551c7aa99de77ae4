"""Groupwise quantisers: FP8 e4m3 with one scale per (gr x gc) block, and the
symmetric int4 input quantiser of the fused add.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

FP8 (``fp8_quant_groupwise``), following
* CUTLASS PR #2095 "Improvements for: Groupwise scaling along M for FP8 gemm",
  hwu36's comment listing the ScaleGranularityM/N modes: one scale per
  (granularity x 128-wide K block); 1 or 128 rows per scale;
* the same PR's PR description: the scale tensor has M / ScaleGranularityM
  rows per K tile (an edge block that is partial still owns one scale);
* torchao PR #3258 "Introduce new W8A8-FP-CSR quantization API", jcaip's review
  comments: the scale must be positive, an all-zero tensor must be supported,
  and the activation is scaled and cast to float8_e4m3fn.

Per block:  amax = max |v|;  s = fl32(amax / 448)  (or s = 1 when amax == 0);
code = e4m3_encode(fl32(v / s)) with IEEE fp32 correctly rounded divides.

Non-finite inputs (the pages say nothing of them; the reading here lets IEEE
arithmetic run through the same formulas): amax is NaN when the block holds a
NaN (a maximum that ignored NaN would hide it) and +inf when it holds an
infinity, so s is NaN or +inf; codes are still the encoder applied to v / s,
where e4m3 gives 0x7F for NaN and the integer grids give 0.

int4 (``int4_quant_groupwise``), for CUTLASS issue #2058 "[QST] How to
implement a fused mixed precision matrix multiplication such as w4a4 +
w16a16?" (hyx1999: X1 and W1 are quantised to 4 bit).  The page fixes no
scheme; the reading used here is symmetric per (row, 128-column group):
s = fl32(amax / 7) (1 when amax == 0), q = clamp(rint_even(fl32(v / s)), -7, 7),
two's-complement nibbles packed two per byte, element 2j in the low nibble
of byte j.

int8 (``int8_quant_groupwise``), for the int8 x int8 2:4-sparse GEMM that
torchao PR #3258 "Introduce new W8A8-FP-CSR quantization API" names beside the
fp8 one (jcaip: the only kernels are int8 x int8 2:4 sparse and fp8 x fp8 2:4
sparse).  The page fixes no int8 scheme; the reading used here keeps the FP8
path's groupwise blocks (1 or 128 rows x 64 or 128 columns) and uses the
symmetric int8 grid: s = fl32(amax / 127) (1 when amax == 0),
q = clamp(rint_even(fl32(v / s)), -127, 127), stored as int8.
"""

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode


def _block_amax(x32: np.ndarray, gr: int, gc: int) -> np.ndarray:
    """max |v| over each gr x gc block, NaN if the block holds one (numpy's max
    propagates NaN); edge blocks are partial (padding with zeros does not
    change a maximum of absolute values)."""
    rows, cols = x32.shape
    rb, cb = -(-rows // gr), -(-cols // gc)
    a = np.zeros((rb * gr, cb * gc), dtype=np.float32)
    a[:rows, :cols] = np.abs(x32)
    return a.reshape(rb, gr, cb, gc).max(axis=(1, 3))


def _int_codes(q: np.ndarray, qmax: int) -> np.ndarray:
    """clamp(rint_even(q), -qmax, qmax) as int64 (an infinite q clamps); NaN -> 0."""
    nan = np.isnan(q)
    return np.where(nan, 0, np.clip(np.rint(np.where(nan, 0, q)), -qmax, qmax)).astype(np.int64)


def _expand(s: np.ndarray, gr: int, gc: int, rows: int, cols: int) -> np.ndarray:
    return np.repeat(np.repeat(s, gr, axis=0), gc, axis=1)[:rows, :cols]


def fp8_quant_groupwise(x, gr: int, gc: int):
    """x: fp32 [rows, cols].  Returns (codes uint8 [rows, cols],
    scales fp32 [ceil(rows/gr), ceil(cols/gc)], row-major)."""
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    amax = _block_amax(x32, gr, gc)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(invalid="ignore"):                              # inf / inf -> NaN
        q = (x32 / _expand(s, gr, gc, rows, cols)).astype(np.float32)   # fp32 IEEE divide
    codes = e4m3_encode(q)
    return codes, s


def int4_quant_groupwise(x, gc: int = 128):
    """x: fp32 [rows, cols] (cols even).  Returns (packed uint8 [rows, cols/2],
    scales fp32 [rows, ceil(cols/gc)])."""
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    assert cols % 2 == 0
    amax = _block_amax(x32, 1, gc)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(7.0)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        q = (x32 / _expand(s, 1, gc, rows, cols)).astype(np.float32)
    qi = _int_codes(q, 7)
    nib = (qi & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, s


def int8_quant_groupwise(x, gr: int, gc: int):
    """x: fp32 [rows, cols].  Returns (codes int8 [rows, cols],
    scales fp32 [ceil(rows/gr), ceil(cols/gc)], row-major)."""
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    amax = _block_amax(x32, gr, gc)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        q = (x32 / _expand(s, gr, gc, rows, cols)).astype(np.float32)   # fp32 IEEE divide
    codes = _int_codes(q, 127).astype(np.int8)
    return codes, s


def int4_decode(packed) -> np.ndarray:
    """Packed int4 [rows, cols/2] -> int64 [rows, cols]; nibble n means n - 16*(n >= 8)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = lo - 16 * (lo >= 8)
    out[:, 1::2] = hi - 16 * (hi >= 8)
    return out
