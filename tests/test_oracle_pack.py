"""Pins of the oracle's gfx950 packed weight layout: hand-derived bytes, a
bijective round trip with zero padding, and the per-block sizes."""
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_row0():
    vals = np.zeros((1, 64), np.uint8)
    vals[0] = np.arange(64)
    meta = np.zeros((1, 16), np.uint8)
    meta[0] = np.arange(200, 216)
    p = oracle.pack24_gfx950(vals, meta)
    assert p.size == 1280
    seen = 0
    for line in open(os.path.join(GOLDEN, "pack_gfx950_row0.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        off, *bs = [int(v) for v in line.split()]
        assert list(p[off:off + len(bs)]) == bs, off
        seen += len(bs)
    assert seen == 80 and np.count_nonzero(p) == 79      # one value byte is 0


def test_roundtrip_and_zero_padding():
    rng = np.random.default_rng(41)
    n, k = 300, 384
    vals = workloads.random_e4m3_codes(rng, (n, k // 2))
    meta = rng.integers(0, 256, size=(n, k // 8)).astype(np.uint8)
    p = oracle.pack24_gfx950(vals, meta)
    assert p.size == oracle.packed_bytes(n, k) == 19 * 3 * 1280
    v2, m2 = oracle.unpack24_gfx950(p, n, k)
    assert np.array_equal(v2, vals) and np.array_equal(m2, meta)
    # padded rows 300..303 of row block 18 hold zeros only
    pv, pm = oracle.unpack24_gfx950(p, 304, k)
    assert not pv[300:].any() and not pm[300:].any()
    # every byte of the 16-row blocks is used exactly once by the first 304 rows
    assert np.count_nonzero(oracle.pack24_gfx950(np.full((304, k // 2), 7, np.uint8),
                                                 np.full((304, k // 8), 9, np.uint8))) == p.size


def test_row_block_chunks_are_contiguous_along_k():
    """The chunk of (row block R, K block kb) starts at (R * KB + kb) * 1280, so
    one row block's chunks follow each other: packing a row block alone gives
    exactly its bytes of the full buffer."""
    rng = np.random.default_rng(43)
    n, k = 48, 512
    vals = workloads.random_e4m3_codes(rng, (n, k // 2))
    meta = rng.integers(0, 256, size=(n, k // 8)).astype(np.uint8)
    p = oracle.pack24_gfx950(vals, meta)
    per_block = (k // 128) * 1280
    for rb in range(3):
        sub = oracle.pack24_gfx950(vals[16 * rb:16 * rb + 16], meta[16 * rb:16 * rb + 16])
        assert np.array_equal(p[rb * per_block:(rb + 1) * per_block], sub)


def test_each_lane_group_word_is_its_smfmac_index():
    """The metadata word of lane group g covers the groups of 4 at dense k =
    b + 4 j (j < 4) and b + 32 + 4 j, b = 64 (g & 1) + 16 (g >> 1): nibble j of
    the word is the canonical nibble of group (b / 4 + j), then (b / 4 + 8 + j)."""
    rng = np.random.default_rng(42)
    meta = rng.integers(0, 256, size=(16, 16)).astype(np.uint8)
    vals = np.zeros((16, 64), np.uint8)
    p = oracle.pack24_gfx950(vals, meta)
    nib = np.empty((16, 32), np.int64)
    nib[:, 0::2] = meta & 15
    nib[:, 1::2] = meta >> 4
    for r in range(16):
        for g in range(4):
            slot = (g + 2 * ((r >> 3) & 1)) & 3
            w = int.from_bytes(bytes(p[1024 + r * 16 + 4 * slot:1024 + r * 16 + 4 * slot + 4]), "little")
            base = 64 * (g & 1) + 16 * (g >> 1)
            groups = [base // 4 + j for j in range(4)] + [base // 4 + 8 + j for j in range(4)]
            assert [(w >> (4 * j)) & 15 for j in range(8)] == [nib[r, q] for q in groups]


# ------------------------------------------------------------- int4 blocked

def test_w4_blocked_bytes_one_by_one():
    """Every byte of a small blocked weight placed by the position formula,
    element by element (the oracle reshapes and transposes)."""
    rng = np.random.default_rng(43)
    n, k = 37, 384                       # three row blocks, the last one 5 rows long
    codes = rng.integers(0, 256, size=(n, k // 4)).astype(np.uint8)
    meta = rng.integers(0, 256, size=(n, k // 8)).astype(np.uint8)
    p = oracle.pack24_w4_blocked(codes, meta)
    kbc = k // 128
    assert p.size == oracle.w4_packed_bytes(n, k) == 3 * kbc * 768
    want = np.zeros(p.size, np.uint8)
    for row in range(n):
        rb, lr = divmod(row, 16)
        for kb in range(kbc):
            base = (rb * kbc + kb) * 768
            for j in range(32):
                want[base + lr * 32 + j] = codes[row, kb * 32 + j]
            for j in range(16):
                want[base + 512 + lr * 16 + j] = meta[row, kb * 16 + j]
    assert np.array_equal(p, want)


def test_w4_blocked_roundtrip_and_zero_rows():
    rng = np.random.default_rng(44)
    n, k = 300, 512
    codes = rng.integers(0, 256, size=(n, k // 4)).astype(np.uint8)
    meta = rng.integers(0, 256, size=(n, k // 8)).astype(np.uint8)
    p = oracle.pack24_w4_blocked(codes, meta)
    c2, m2 = oracle.unpack24_w4_blocked(p, n, k)
    assert np.array_equal(c2, codes) and np.array_equal(m2, meta)
    # rows 300..303 (row block 18, local rows 12..15) are zero in every chunk
    ch = p.reshape(19, k // 128, 768)[18]
    assert not ch[:, 12 * 32:512].any() and not ch[:, 512 + 12 * 16:].any()
    # a one-row weight: each chunk holds its 32 + 16 bytes and zeros
    p1 = oracle.pack24_w4_blocked(codes[:1], meta[:1]).reshape(k // 128, 768)
    assert np.array_equal(p1[:, :32], codes[0].reshape(k // 128, 32))
    assert np.array_equal(p1[:, 512:528], meta[0].reshape(k // 128, 16))
    assert np.count_nonzero(p1[:, 32:512]) == 0 and np.count_nonzero(p1[:, 528:]) == 0
