"""Pins of the oracle's 2:4 pruning and packing: exhaustive brute force against
a rule written independently, hand-worked golden rows, round trips."""
import itertools
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LEGAL_NIBBLES = {0x4, 0x8, 0x9, 0xC, 0xD, 0xE}


def _kept_by_counting(group):
    """Entry i survives iff fewer than two entries beat it, where j beats i when
    |w_j| > |w_i|, or |w_j| == |w_i| and j < i."""
    a = [abs(float(v)) for v in group]
    kept = []
    for i in range(4):
        beaten_by = sum(1 for j in range(4) if a[j] > a[i] or (a[j] == a[i] and j < i))
        if beaten_by < 2:
            kept.append(i)
    return kept


def test_prune_brute_force_all_groups():
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0], dtype=np.float32)
    groups = np.array(list(itertools.product(range(8), repeat=4)))
    w = alphabet[groups]                                   # [4096, 4]
    keep, pruned = oracle.prune24(w)
    for r in range(w.shape[0]):
        want = _kept_by_counting(w[r])
        assert len(want) == 2
        assert list(np.nonzero(keep[r])[0]) == want, w[r]
    # pruned slots are +0.0, kept slots keep their bits
    assert np.array_equal(pruned.view(np.uint32)[~keep], np.zeros((~keep).sum(), np.uint32))
    assert np.array_equal(pruned.view(np.uint32)[keep], w.view(np.uint32)[keep])
    # the group maximum magnitude always survives
    assert np.array_equal(np.abs(pruned).max(axis=1), np.abs(w).max(axis=1))
    # idempotent
    keep2, pruned2 = oracle.prune24(pruned)
    assert np.array_equal(pruned2.view(np.uint32), pruned.view(np.uint32))


def _golden_rows():
    rows = []
    cur = {}
    for line in open(os.path.join(GOLDEN, "sparse24_hand_examples.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, val = line.split(":", 1)
        cur[key] = val.split()
        if key == "meta":
            rows.append(cur)
            cur = {}
    return rows


def test_golden_hand_examples():
    rows = _golden_rows()
    assert len(rows) == 6
    seen = set()
    for ex in rows:
        w = np.array([[float(v) for v in ex["w"]]], dtype=np.float32)
        keep, _ = oracle.prune24(w)
        want_keep = [tuple(int(i) for i in g.split(",")) for g in ex["keep"]]
        for g, pair in enumerate(want_keep):
            assert tuple(np.nonzero(keep[0, 4 * g:4 * g + 4])[0]) == pair
        vals, meta = oracle.prune_compress24(w)
        assert list(vals[0]) == [float(v) for v in ex["vals"]]
        assert meta[0, 0] == int(ex["meta"][0], 16)
        seen |= {int(meta[0, 0]) & 15, int(meta[0, 0]) >> 4}
    assert seen == LEGAL_NIBBLES


def test_roundtrip_and_legal_nibbles():
    w = workloads.sparse_large(seed=21, m=4, n=96, k=512)["w"]
    keep, pruned = oracle.prune24(w)
    vals, meta = oracle.compress24(pruned, keep)
    assert vals.shape == (96, 256) and meta.shape == (96, 64)
    nibs = np.concatenate([meta & 15, meta >> 4]).ravel()
    assert set(np.unique(nibs)) <= LEGAL_NIBBLES
    dense = oracle.decompress24(vals, meta)
    assert np.array_equal(dense.view(np.uint32), pruned.view(np.uint32))
    vals2, meta2 = oracle.compress24(dense, keep)
    assert np.array_equal(vals2.view(np.uint32), vals.view(np.uint32))
    assert np.array_equal(meta2, meta)


def test_compress_of_decompress_is_identity_on_codes():
    rng = np.random.default_rng(22)
    pairs = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    sel = rng.integers(0, 6, size=(8, 64))
    nib = np.array([[p[0] | (p[1] << 2) for p in (pairs[i] for i in row)] for row in sel], np.uint8)
    meta = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    vals = workloads.random_e4m3_codes(rng, (8, 128))
    vals[vals == 0] = 0x38          # non-zero codes so positions are recoverable
    vals[vals == 0x80] = 0x38
    dense = oracle.decompress24(vals, meta)
    keep = dense != 0
    v2, m2 = oracle.compress24(dense, keep)
    assert np.array_equal(v2, vals) and np.array_equal(m2, meta)


def test_bf16_prune_matches_f32_of_same_values():
    w = workloads.sparse_large(seed=23, m=4, n=16, k=64)["w"]
    bits = workloads.to_bf16_bits(w)
    wf = (bits.astype(np.uint32) << 16).view(np.float32)
    k1, _ = oracle.prune24(bits)
    k2, _ = oracle.prune24(wf)
    assert np.array_equal(k1, k2)
    vals, meta = oracle.prune_compress24(bits)
    assert vals.dtype == np.uint16
    assert np.array_equal(oracle.decompress24(vals, meta), np.where(k1, bits, 0))


def test_all_zero_weight_is_supported():
    vals, meta = oracle.prune_compress24(np.zeros((3, 16), np.float32))
    assert np.all(vals == 0) and np.all(meta == 0x44)


def _rank_key(v):
    """(is NaN, |v|): NaN above every number, NaNs equal among themselves."""
    v = float(v)
    return (1, 0.0) if v != v else (0, abs(v))


def test_prune_brute_force_nonfinite():
    """Every group over {+-0, +-1, +-inf, +-NaN}: the survivors are the entries
    beaten by fewer than two others, with NaN ranked above infinity."""
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, -np.nan], dtype=np.float32)
    groups = np.array(list(itertools.product(range(8), repeat=4)))
    w = alphabet[groups]
    keep, pruned = oracle.prune24(w)
    for r in range(w.shape[0]):
        k = [_rank_key(v) for v in w[r]]
        want = [i for i in range(4) if sum(1 for j in range(4) if k[j] > k[i] or (k[j] == k[i] and j < i)) < 2]
        assert list(np.nonzero(keep[r])[0]) == want, w[r]
    assert np.array_equal(pruned.view(np.uint32)[keep], w.view(np.uint32)[keep])


def test_prune_e4m3_codes_rank_like_their_magnitude_bits():
    """e4m3 codes: with the sign bit cleared a code orders like its magnitude
    (0x7F, the NaN, above 0x7E = 448), so the survivors follow the counting rule
    on code & 0x7F -- written on the codes alone, without decoding them."""
    rng = np.random.default_rng(5)
    c = rng.integers(0, 256, size=(20000, 4)).astype(np.uint8)
    c[:2000, :] = rng.choice(np.array([0x00, 0x80, 0x7F, 0xFF, 0x7E, 0xFE], np.uint8), size=(2000, 4))
    keep, pruned = oracle.prune24(c)
    for r in range(c.shape[0]):
        key = [int(v) & 0x7F for v in c[r]]
        want = [i for i in range(4) if sum(1 for j in range(4) if key[j] > key[i] or (key[j] == key[i] and j < i)) < 2]
        assert list(np.nonzero(keep[r])[0]) == want, c[r]
    assert np.all(pruned[~keep] == 0) and np.array_equal(pruned[keep], c[keep])
    vals, meta = oracle.prune_compress24(c.reshape(-1, 8))
    assert vals.dtype == np.uint8 and meta.shape == (c.shape[0] // 2, 1)


def _golden_nonfinite_rows():
    rows, cur = [], {}
    for line in open(os.path.join(GOLDEN, "sparse24_nonfinite_e4m3.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, val = line.split(":", 1)
        cur[key] = val.split()
        if key == "meta":
            rows.append(cur)
            cur = {}
    return rows


def test_golden_nonfinite_and_e4m3_examples():
    rows = _golden_nonfinite_rows()
    assert [r["kind"][0] for r in rows] == ["f32", "f32", "e4m3", "e4m3"]
    for ex in rows:
        if ex["kind"][0] == "f32":
            w = np.array([[float(v) for v in ex["w"]]], dtype=np.float32)
            want_vals = np.array([float(v) for v in ex["vals"]], dtype=np.float32)
        else:
            w = np.array([[int(v, 16) for v in ex["w"]]], dtype=np.uint8)
            want_vals = np.array([int(v, 16) for v in ex["vals"]], dtype=np.uint8)
        keep, _ = oracle.prune24(w)
        for g, pair in enumerate(ex["keep"]):
            assert tuple(np.nonzero(keep[0, 4 * g:4 * g + 4])[0]) == tuple(int(i) for i in pair.split(","))
        vals, meta = oracle.prune_compress24(w)
        if w.dtype == np.uint8:
            assert np.array_equal(vals[0], want_vals)
        else:   # NaN != NaN: compare NaN positions, then the rest by value
            assert np.array_equal(np.isnan(vals[0]), np.isnan(want_vals))
            ok = ~np.isnan(want_vals)
            assert np.array_equal(vals[0][ok], want_vals[ok])
        assert meta[0, 0] == int(ex["meta"][0], 16)
