"""Pins of the oracle's groupwise quantisers: an independent PyTorch route,
closed-form invariants and exact power-of-two round trips."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _torch_quant(x: np.ndarray, gr: int, gc: int):
    """Same definition through PyTorch ops: amax per block, fp32 divide, cast."""
    t = torch.from_numpy(x)
    rows, cols = t.shape
    rb, cb = -(-rows // gr), -(-cols // gc)
    s = torch.ones(rb, cb, dtype=torch.float32)
    codes = torch.empty(rows, cols, dtype=torch.uint8)
    for i in range(rb):
        for j in range(cb):
            blk = t[i * gr:(i + 1) * gr, j * gc:(j + 1) * gc]
            a = blk.abs().max()
            if a > 0:
                s[i, j] = a / torch.tensor(448.0, dtype=torch.float32)
            q = (blk / s[i, j]).to(torch.float8_e4m3fn).view(torch.uint8)
            codes[i * gr:(i + 1) * gr, j * gc:(j + 1) * gc] = q
    return codes.numpy(), s.numpy()


@pytest.mark.parametrize("gr,gc,shape", [(1, 128, (37, 256)), (128, 128, (200, 300)),
                                         (128, 64, (130, 192)), (1, 128, (5, 129))])
def test_quant_matches_torch_route(gr, gc, shape):
    d = workloads.dense_outliers(seed=11, m=shape[0], n=8, k=shape[1])
    codes, s = oracle.fp8_quant_groupwise(d["x"], gr, gc)
    tc, ts = _torch_quant(d["x"], gr, gc)
    assert s.shape == (-(-shape[0] // gr), -(-shape[1] // gc))
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(codes, tc)


def test_every_nonzero_block_reaches_448():
    x = workloads.dense_outliers(seed=12, m=256, n=8, k=512)["x"]
    codes, s = oracle.fp8_quant_groupwise(x, 128, 128)
    mag = codes & 0x7F
    blocks = mag.reshape(2, 128, 4, 128).max(axis=(1, 3))
    assert np.all(blocks == 0x7E)
    assert np.all(s > 0)


def test_dequant_error_within_half_ulp():
    x = workloads.sparse_large(seed=13, m=64, n=8, k=256)["x"]
    codes, s = oracle.fp8_quant_groupwise(x, 1, 128)
    se = np.repeat(s, 128, axis=1).astype(np.float64)
    q = x.astype(np.float64) / se
    dec = oracle.e4m3_decode(codes)
    # ulp of e4m3 at |q|: 2^(floor(log2|q|) - 3) for normals, 2^-9 for subnormals
    e = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    assert np.all(np.abs(dec - q) <= ulp / 2 + 2.0 ** -23 * np.abs(q))


def test_power_of_two_roundtrip_is_exact():
    """If v = dec(c) * 2^j and the block holds a +-448 code, then s = 2^j and the
    codes come back unchanged."""
    rng = np.random.default_rng(14)
    c = workloads.random_e4m3_codes(rng, (128, 256))
    c[rng.integers(0, 128), 5] = 0x7E
    c[rng.integers(0, 128), 200] = 0xFE
    js = rng.integers(-20, 20, size=(1, 2))
    v = (oracle.e4m3_decode(c) * np.repeat(np.exp2(js), 128, axis=1)).astype(np.float32)
    codes, s = oracle.fp8_quant_groupwise(v, 128, 128)
    assert np.array_equal(s, np.exp2(js).astype(np.float32))
    assert np.array_equal(codes, c)


def test_all_zero_block_scale_one_codes_zero():
    x = np.zeros((3, 256), dtype=np.float32)
    x[1, 200] = 5.0                     # second block of row 1 is non-zero
    codes, s = oracle.fp8_quant_groupwise(x, 1, 128)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[2, 1] == 1.0
    assert s[1, 1] == np.float32(5.0) / np.float32(448.0)
    assert codes[1, 200] == 0x7E
    assert np.count_nonzero(codes) == 1


def test_partial_edge_block_uses_only_its_rows():
    x = np.ones((130, 128), dtype=np.float32)
    x[129, 0] = 64.0                    # only in the second (2-row) block
    _, s = oracle.fp8_quant_groupwise(x, 128, 128)
    assert s.shape == (2, 1)
    assert s[0, 0] == np.float32(1.0) / np.float32(448.0)
    assert s[1, 0] == np.float32(64.0) / np.float32(448.0)


# --- int4 ---------------------------------------------------------------

def test_int4_decode_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    d = oracle.int4_decode(b)
    lo, hi = d[0, 0::2], d[0, 1::2]
    for byte in range(256):
        n0, n1 = byte & 15, byte >> 4
        assert lo[byte] == (n0 if n0 < 8 else n0 - 16)
        assert hi[byte] == (n1 if n1 < 8 else n1 - 16)


def test_int4_quant_matches_torch_route():
    x = workloads.mixed_add(seed=15, m=9, n=4, k1=384, k2=32)["x1"]
    packed, s = oracle.int4_quant_groupwise(x, 128)
    t = torch.from_numpy(x).view(9, 3, 128)
    a = t.abs().amax(dim=2, keepdim=True)
    ts = torch.where(a > 0, a / torch.tensor(7.0), torch.ones_like(a))
    q = torch.clamp(torch.round(t / ts), -7, 7).to(torch.int64).view(9, 384)
    assert np.array_equal(s, ts.view(9, 3).numpy())
    assert np.array_equal(oracle.int4_decode(packed), q.numpy())


def test_int4_power_of_two_roundtrip():
    rng = np.random.default_rng(16)
    q = rng.integers(-7, 8, size=(4, 256))
    q[:, 3] = 7
    q[:, 130] = -7
    j = rng.integers(-10, 10, size=(4, 2))
    # v = q * 7 * 2^j / 7 ... choose v = q * 2^j so amax = 7 * 2^j and s = 2^j exactly
    v = (q * np.repeat(np.exp2(j), 128, axis=1)).astype(np.float32)
    packed, s = oracle.int4_quant_groupwise(v, 128)
    assert np.array_equal(s, np.exp2(j).astype(np.float32))
    assert np.array_equal(oracle.int4_decode(packed), q)


def test_divide_not_reciprocal_on_a_tie():
    """amax = 449 gives s = fl32(449/448).  v = fl32(1.6875 s) divides back to
    exactly 1.6875, a tie between 1.625 (0x3D) and 1.75 (0x3E) that goes to the
    even code 0x3E; v * fl32(1/s) lands just below the tie and would give 0x3D."""
    s_exp = np.float32(449.0) / np.float32(448.0)
    v = np.float32(1.6875) * s_exp
    assert np.float32(v / s_exp) == np.float32(1.6875)
    assert np.float32(v * (np.float32(1) / s_exp)) < np.float32(1.6875)
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 1] = 449.0, v
    codes, s = oracle.fp8_quant_groupwise(x, 1, 128)
    assert s[0, 0] == s_exp
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0x3E
    tc, _ = _torch_quant(x, 1, 128)
    assert tc[0, 1] == 0x3E


@pytest.mark.parametrize("whole", ["rows", "tensor"])
def test_whole_row_and_tensor_groups_roundtrip_and_reach_448(whole):
    """One group per row (gr = 1, gc = cols) or per tensor (gr = rows): a power-
    of-two multiple of e4m3 values whose group maximum is 448 * 2^j comes back
    code for code with scale 2^j, and the group maximum's code is +-448."""
    rng = np.random.default_rng(77)
    rows, cols = 6, 384
    codes = rng.integers(0, 0x7F, size=(rows, cols)).astype(np.uint8) | (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    codes[np.arange(rows), rng.integers(0, cols, rows)] = 0x7E          # 448 in every row
    j = rng.integers(-12, 12, size=(rows, 1)) if whole == "rows" else np.full((rows, 1), 5)
    v = (oracle.e4m3_decode(codes) * np.exp2(j)).astype(np.float32)
    gr = 1 if whole == "rows" else rows
    q, s = oracle.fp8_quant_groupwise(v, gr, cols)
    assert s.shape == ((rows, 1) if whole == "rows" else (1, 1))
    assert np.array_equal(s.reshape(-1), np.exp2(j[:, 0] if whole == "rows" else j[:1, 0]).astype(np.float32))
    assert np.array_equal(q, codes)


def test_nonfinite_blocks_follow_ieee_through_the_formulas():
    """A block holding a NaN: amax NaN, scale NaN, every quotient NaN, so every
    e4m3 code is 0x7F and every integer code 0.  A block holding +-inf (no NaN):
    amax and scale +inf; a finite v gives v / inf = +-0 (codes 0x00 / 0x80, or
    integer 0) and the infinity gives inf / inf = NaN (0x7F, or 0).  Other
    blocks are untouched."""
    x = np.zeros((3, 256), np.float32)
    x[0, :128] = np.linspace(-3, 3, 128, dtype=np.float32)
    x[0, 7] = np.nan
    x[1, :128] = 2.0
    x[1, 5] = -1.0
    x[1, 9] = -np.inf
    x[:, 128:] = 4.0
    q, s = oracle.fp8_quant_groupwise(x, 1, 128)
    assert np.isnan(s[0, 0]) and s[1, 0] == np.inf and np.all(s[:, 1] == np.float32(4.0 / 448.0))
    assert np.all(q[0, :128] == 0x7F)
    want = np.zeros(128, np.uint8)
    want[5] = 0x80
    want[9] = 0x7F
    assert np.array_equal(q[1, :128], want)
    assert np.all(q[:, 128:] == 0x7E)
    q8, s8 = oracle.int8_quant_groupwise(x, 1, 128)
    assert np.isnan(s8[0, 0]) and s8[1, 0] == np.inf
    assert np.all(q8[:2, :128] == 0) and np.all(q8[:, 128:] == 127)
    q4, s4 = oracle.int4_quant_groupwise(x, 128)
    assert np.isnan(s4[0, 0]) and s4[1, 0] == np.inf
    assert np.all(q4[:2, :64] == 0) and np.all(q4[:, 64:] == 0x77)


def test_nan_scale_comes_from_amax_not_from_the_zero_rule():
    """The all-zero rule (s = 1) applies to amax == 0 only: a NaN block must not
    fall into it (a comparison amax > 0 is false for NaN)."""
    x = np.zeros((1, 128), np.float32)
    x[0, 3] = np.nan
    _, s = oracle.fp8_quant_groupwise(x, 1, 128)
    assert np.isnan(s[0, 0])
    x[0, 3] = 0.0
    _, s = oracle.fp8_quant_groupwise(x, 1, 128)
    assert s[0, 0] == 1.0
