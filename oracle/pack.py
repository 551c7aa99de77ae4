"""The gfx950 packed layout of a 2:4-compressed FP8 weight, and its inverse.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages keep the sparse operand in a hardware-specific arrangement produced
by a packing kernel: torchao PR #3258 "Introduce new W8A8-FP-CSR quantization
API" (jcaip: use the CUTLASS packing kernel for FP8 semi-structured weights
rather than the generic conversion) and CUTLASS issue #2029 (klevzoff: the
mainloop takes the values together with the metadata tensor E in its own
layout).  This module defines that arrangement for gfx950's SMFMAC and the
LDS image the GEMM kernels read; it is a pure byte permutation of the
canonical values [N, K/2] and metadata [N, K/8] (``sparse24.py``), with rows
padded to a multiple of 16 with zeros.

The weight is cut into 16-row blocks R (rows 16 R .. 16 R + 15); for block R
and 128-wide K block kb a 1280-byte chunk starts at byte (R * KB + kb) * 1280
(KB = K / 128), so that the chunks of one row block follow each other along K.
For local row lr = 0..15 and lane group g = 0..3 (b = 32 (g & 1) + 8 (g >> 1))
the chunk holds
  * values, 16 bytes at lr * 64 + 16 * (g ^ ((lr >> 1) & 3)):
        compressed bytes [b, b + 8) and [b + 16, b + 24) of the row's 64
        compressed bytes of block kb (the SMFMAC A operand of lane group g);
  * metadata, 4 bytes at 1024 + lr * 16 + 4 * ((g + 2 * ((lr >> 3) & 1)) & 3):
        metadata bytes b/4, b/4 + 1, b/4 + 4, b/4 + 5 of the row's 16 metadata
        bytes of block kb (the SMFMAC index word of lane group g).
"""

import numpy as np

ROWS = 16
CHUNK_BYTES = 1280
META_OFF = 1024


def packed_bytes(n: int, k: int) -> int:
    return -(-n // ROWS) * (k // 128) * CHUNK_BYTES


def _positions(n: int, kb_count: int):
    """Byte positions in the packed buffer, per (row, kb, g): values start and
    metadata word start."""
    rows = np.arange(n)
    t, r = rows // ROWS, rows % ROWS
    kb = np.arange(kb_count)
    g = np.arange(4)
    base = (t[:, None] * kb_count + kb[None, :]) * CHUNK_BYTES                     # [n, KB]
    vpos = base[:, :, None] + (r * 64)[:, None, None] + 16 * (g[None, None, :] ^ ((r[:, None, None] >> 1) & 3))
    mslot = (g[None, None, :] + 2 * ((r[:, None, None] >> 3) & 1)) & 3
    mpos = base[:, :, None] + META_OFF + (r * 16)[:, None, None] + 4 * mslot
    return vpos, mpos                                                                # [n, KB, 4]


def _lane_group_bytes():
    """For each lane group g: the 16 value-byte indices and the 4 metadata-byte
    indices it takes from a row's K block."""
    vidx, midx = [], []
    for g in range(4):
        b = 32 * (g & 1) + 8 * (g >> 1)
        vidx.append(list(range(b, b + 8)) + list(range(b + 16, b + 24)))
        midx.append([b // 4, b // 4 + 1, b // 4 + 4, b // 4 + 5])
    return np.array(vidx), np.array(midx)


def pack24_gfx950(vals, meta) -> np.ndarray:
    """vals uint8 [N, K/2] (e4m3 codes), meta uint8 [N, K/8] -> packed uint8."""
    vals = np.asarray(vals, dtype=np.uint8)
    meta = np.asarray(meta, dtype=np.uint8)
    n, half = vals.shape
    k = 2 * half
    assert k % 128 == 0 and meta.shape == (n, k // 8)
    kbc = k // 128
    out = np.zeros(packed_bytes(n, k), dtype=np.uint8)
    vpos, mpos = _positions(n, kbc)
    vidx, midx = _lane_group_bytes()
    vb = vals.reshape(n, kbc, 64)
    mb = meta.reshape(n, kbc, 16)
    for g in range(4):
        for j in range(16):
            out[vpos[:, :, g] + j] = vb[:, :, vidx[g, j]]
        for j in range(4):
            out[mpos[:, :, g] + j] = mb[:, :, midx[g, j]]
    return out


def unpack24_gfx950(packed, n: int, k: int):
    """Inverse of ``pack24_gfx950``: -> (vals [N, K/2], meta [N, K/8])."""
    packed = np.asarray(packed, dtype=np.uint8)
    kbc = k // 128
    vpos, mpos = _positions(n, kbc)
    vidx, midx = _lane_group_bytes()
    vb = np.zeros((n, kbc, 64), dtype=np.uint8)
    mb = np.zeros((n, kbc, 16), dtype=np.uint8)
    for g in range(4):
        for j in range(16):
            vb[:, :, vidx[g, j]] = packed[vpos[:, :, g] + j]
        for j in range(4):
            mb[:, :, midx[g, j]] = packed[mpos[:, :, g] + j]
    return vb.reshape(n, k // 2), mb.reshape(n, k // 8)


# ------------------------------------------------------------------ int4
# The blocked form of a 2:4-compressed int4 weight (codes [N, K/4], two per
# byte as ``quant.int4_quant_groupwise`` stores them, metadata [N, K/8]): the
# same row-block / K-block chunking as above, without any permutation inside a
# chunk.  For 16-row block R and 128-wide K block kb the 768-byte chunk at
# (R * KB + kb) * 768 holds the 16 rows' 32 code bytes of block kb, row after
# row (local row lr at lr * 32), then their 16 metadata bytes (lr at
# 512 + lr * 16); rows past N are zero.  This too is the library's own layout
# (what its weight-only kernels stream), a byte permutation of the canonical
# arrays in the spirit of the packing kernels the pages describe.

W4_CHUNK_BYTES = 768
W4_META_OFF = 512


def w4_packed_bytes(n: int, k: int) -> int:
    return -(-n // ROWS) * (k // 128) * W4_CHUNK_BYTES


def pack24_w4_blocked(codes4, meta) -> np.ndarray:
    """codes4 uint8 [N, K/4] (int4 pairs), meta uint8 [N, K/8] -> blocked uint8."""
    codes4 = np.asarray(codes4, dtype=np.uint8)
    meta = np.asarray(meta, dtype=np.uint8)
    n, quarter = codes4.shape
    k = 4 * quarter
    assert k % 128 == 0 and meta.shape == (n, k // 8)
    kbc, t = k // 128, -(-n // ROWS)
    c = np.zeros((t * ROWS, quarter), np.uint8)
    m = np.zeros((t * ROWS, k // 8), np.uint8)
    c[:n], m[:n] = codes4, meta
    # [T, 16, KB, 32] -> [T, KB, 16, 32]: one row block's K block is 16 rows of 32 bytes
    cb = c.reshape(t, ROWS, kbc, 32).transpose(0, 2, 1, 3).reshape(t, kbc, 512)
    mb = m.reshape(t, ROWS, kbc, 16).transpose(0, 2, 1, 3).reshape(t, kbc, 256)
    return np.concatenate([cb, mb], axis=2).reshape(-1)


def unpack24_w4_blocked(packed, n: int, k: int):
    """Inverse of ``pack24_w4_blocked``: -> (codes4 [N, K/4], meta [N, K/8])."""
    packed = np.asarray(packed, dtype=np.uint8)
    kbc, t = k // 128, -(-n // ROWS)
    ch = packed.reshape(t, kbc, W4_CHUNK_BYTES)
    c = ch[:, :, :W4_META_OFF].reshape(t, kbc, ROWS, 32).transpose(0, 2, 1, 3).reshape(t * ROWS, k // 4)
    m = ch[:, :, W4_META_OFF:].reshape(t, kbc, ROWS, 16).transpose(0, 2, 1, 3).reshape(t * ROWS, k // 8)
    return c[:n].copy(), m[:n].copy()
