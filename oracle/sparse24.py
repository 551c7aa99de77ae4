"""2:4 magnitude pruning along K and its compressed storage (values + metadata).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pruning follows torchao PR #3258 "Introduce new W8A8-FP-CSR quantization API",
jcaip's review comments on the pruning code: the weight is viewed in groups of
4 consecutive elements of a row, the two smallest magnitudes (by an argsort of
|w|) are set to zero and the other two survive.  The pages do not say how equal
magnitudes are ordered; the reading here is that the larger magnitude wins
and, between equal magnitudes, the lower index wins (+0 and -0 are equal).
Nor do they say where NaN goes; the reading here ranks NaN above every number
(a NaN weight is never silently dropped) with all NaNs equal.  Pruned entries
become zero (+0.0, or code 0x00); survivors keep their bits.

Weights may be fp32, bf16 bit patterns (uint16) or e4m3 codes (uint8, a weight
quantised before pruning, as the FP8 path of that PR can take it): the codes
are decoded to their values and ranked by magnitude like any other weight.

Storage follows the same review ("store the specified values and the sparse
metadata", not a dense copy) and the operand triple of CUTLASS issue #2029
(klevzoff's mainloop arguments: values pointer + metadata pointer E).  The
pages fix no metadata bit layout; the layout used here is:
    vals[r, 2g + j] = w[r, 4g + i_j], with i_0 < i_1 the two kept positions,
    nibble(g)       = i_0 | (i_1 << 2),
    meta[r, b]      = nibble(2b) | (nibble(2b + 1) << 4)      (shape [R, K/8]).
"""

import numpy as np

from .e4m3 import e4m3_decode


def _values(w) -> np.ndarray:
    """The weights' values in fp64 (exact for all three formats)."""
    w = np.asarray(w)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        if w.dtype == np.uint16:         # bf16 bits
            return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if w.dtype == np.uint8:          # e4m3 codes
            return e4m3_decode(w)
        return np.asarray(w, dtype=np.float32).astype(np.float64)


def prune24(w):
    """w: fp32 [R, K] (or bf16 bits as uint16), K % 4 == 0.
    Returns (kept mask bool [R, K], pruned copy of w with +0 in dropped slots)."""
    w = np.asarray(w)
    rows, k = w.shape
    assert k % 4 == 0
    v = _values(w).reshape(rows, k // 4, 4)
    nan = np.isnan(v)
    mag = np.where(nan, 0.0, np.abs(v))
    # Rank each group by (NaN first, then -|w|, then index): lexsort is stable,
    # so equal keys keep index order; the first two of that order survive.
    order = np.lexsort((-mag, ~nan), axis=-1)
    keep = np.zeros((rows, k // 4, 4), dtype=bool)
    np.put_along_axis(keep, order[..., :2], True, axis=-1)
    keep = keep.reshape(rows, k)
    pruned = np.where(keep, w, np.zeros((), dtype=w.dtype)).astype(w.dtype)
    return keep, pruned


def compress24(w, keep):
    """Gather the kept values (ascending index within each group) and pack metadata."""
    w = np.asarray(w)
    rows, k = w.shape
    kg = np.asarray(keep, dtype=bool).reshape(rows, k // 4, 4)
    assert np.all(kg.sum(axis=-1) == 2), "every group of 4 must keep exactly 2"
    # Positions 0..3 of the kept entries, in ascending order: i0 < i1.
    pos = np.sort(np.where(kg, np.arange(4), 99), axis=-1)[..., :2]
    i0, i1 = pos[..., 0], pos[..., 1]
    wg = w.reshape(rows, k // 4, 4)
    vals = np.stack([np.take_along_axis(wg, i0[..., None], -1)[..., 0],
                     np.take_along_axis(wg, i1[..., None], -1)[..., 0]], axis=-1)
    vals = vals.reshape(rows, k // 2).astype(w.dtype)
    nib = (i0 | (i1 << 2)).astype(np.uint8)                      # [R, K/4]
    meta = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)   # [R, K/8]
    return vals, meta


def decompress24(vals, meta):
    """Scatter compressed values back to a dense [R, K] array, zeros elsewhere."""
    vals = np.asarray(vals)
    meta = np.asarray(meta, dtype=np.uint8)
    rows, half = vals.shape
    k = half * 2
    assert meta.shape == (rows, k // 8)
    nib = np.empty((rows, k // 4), dtype=np.int64)
    nib[:, 0::2] = meta & 0xF
    nib[:, 1::2] = meta >> 4
    i0, i1 = nib & 3, (nib >> 2) & 3
    vg = vals.reshape(rows, k // 4, 2)
    dense = np.zeros((rows, k // 4, 4), dtype=vals.dtype)
    np.put_along_axis(dense, i0[..., None], vg[..., 0:1], axis=-1)
    np.put_along_axis(dense, i1[..., None], vg[..., 1:2], axis=-1)
    return dense.reshape(rows, k)


def prune_compress24(w):
    """Prune then compress: the weight-preparation step (values, metadata)."""
    keep, pruned = prune24(w)
    return compress24(pruned, keep)
