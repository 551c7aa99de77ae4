"""OCP FP8 E4M3 ("e4m3fn") decode and encode, written from the format's definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The torchao PR "Introduce new W8A8-FP-CSR quantization API" (the reviewed
linear path, jcaip's comments on the activation cast) quantises by scaling and
casting to ``torch.float8_e4m3fn``: the OCP E4M3 variant with no infinities,
one NaN pattern per sign (S.1111.111) and largest finite magnitude 448.  The
per-block scale of the workloads is amax/448, which is that format's maximum.

Decode (exact, closed form), for code c with sign s = c>>7, exponent
e = (c>>3)&15, mantissa m = c&7:
    e == 15 and m == 7 -> NaN
    e == 0             -> (-1)^s * m * 2^-9           (subnormal)
    otherwise          -> (-1)^s * (1 + m/8) * 2^(e-7)

Encode: round |v| to the nearest finite E4M3 magnitude, ties to the code with
an even mantissa LSB, saturate magnitudes above 448 to 448 (infinities
included), and keep the sign bit of v (so a negative value that rounds to zero
gives 0x80, -0).  Every NaN input gives 0x7F: the format has a NaN code for each
sign, the pages fix no NaN handling, and the reading here is one canonical code.
"""

import numpy as np

E4M3_MAX = 448.0


def _decode_one(c: int) -> float:
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# All 256 code values, built one at a time from the closed form above.
_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
# The 127 finite non-negative magnitudes, codes 0x00..0x7E, strictly ascending.
_POS = _TABLE[:0x7F].copy()
# Midpoints between neighbours: v lies between codes i and i+1 when
# _MID[i-1] <= v <= _MID[i].  Sums of two E4M3 values are exact in fp64.
_MID = (_POS[:-1] + _POS[1:]) / 2.0


def e4m3_decode(codes) -> np.ndarray:
    """Decode e4m3 codes (uint8 array) to fp64 values, exactly."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def e4m3_encode(v) -> np.ndarray:
    """Encode fp32 values to e4m3 codes: nearest, ties to even code, saturating."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    sign = np.signbit(v).astype(np.uint8) << 7
    # Lower neighbour index lo = number of midpoints strictly below a; the
    # candidate codes are lo (below or at a) ... decided against the midpoints.
    lo = np.searchsorted(_MID, a, side="left")          # first midpoint >= a
    code = lo.astype(np.int64)                           # a <= _MID[lo]: nearest is lo, except ties
    lo_c = np.minimum(lo, len(_MID) - 1)
    tie = (lo < len(_MID)) & (a == _MID[lo_c])
    # On a tie between codes lo and lo+1 pick the even one.
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    code = np.minimum(code, 0x7E)                        # saturate to 448
    code = (code.astype(np.uint8) | sign).astype(np.uint8)
    return np.where(np.isnan(a), np.uint8(0x7F), code).astype(np.uint8)
