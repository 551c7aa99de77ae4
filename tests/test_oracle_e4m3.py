"""Pins of the oracle's e4m3 codec against PyTorch's CPU float8_e4m3fn cast
(an independent implementation of the cast the torchao page uses) and the
format's closed-form spot values."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.float().numpy().astype(np.float64)


def _torch_encode(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_256_codes_match_torch():
    c = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_decode(c), _torch_decode(c)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.isnan(ours).sum() == 2          # 0x7F and 0xFF only


def test_decode_golden_spot_values():
    rows = 0
    for line in open(os.path.join(GOLDEN, "e4m3_spot_values.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()[:2]
        got = oracle.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        want = float(val)
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), code
        rows += 1
    assert rows == 13


def test_encode_roundtrips_every_finite_code():
    c = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], dtype=np.uint8)
    v = oracle.e4m3_decode(c).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(v), c)


def _midpoints_and_neighbours():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    vals = np.concatenate([mid, up, dn, pos.astype(np.float32)])
    return np.concatenate([vals, -vals])


def test_encode_midpoints_match_torch():
    v = _midpoints_and_neighbours()
    assert np.array_equal(oracle.e4m3_encode(v), _torch_encode(v))


def test_encode_random_match_torch():
    rng = np.random.default_rng(1234)
    n = 1_000_000
    mag = np.exp2(rng.uniform(-14.0, np.log2(463.9), size=n)).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    v = mag * sign
    assert np.array_equal(oracle.e4m3_encode(v), _torch_encode(v))


def test_encode_ties_go_to_even_code():
    # 1.0625 sits halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38.
    # 1.1875 sits halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A.
    # 2^-10 is halfway between 0 and the smallest subnormal: 0x00.
    v = np.array([1.0625, 1.1875, 2.0 ** -10, -1.0625], dtype=np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x38, 0x3A, 0x00, 0xB8]


def test_encode_saturates_and_keeps_sign_of_zero():
    v = np.array([448.0, 449.0, 464.0, 1e6, 3e38, -500.0, -1e-30, -0.0, 0.0], dtype=np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]


@pytest.mark.parametrize("v", [np.nan, -np.nan])
def test_encode_nan(v):
    """Every NaN, whatever its sign, gets the one code 0x7F."""
    code = oracle.e4m3_encode(np.array([v], dtype=np.float32))[0]
    assert code == 0x7F


def test_encode_infinities_saturate():
    v = np.array([np.inf, -np.inf], dtype=np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E, 0xFE]
