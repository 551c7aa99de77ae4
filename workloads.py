"""Seeded synthetic inputs for the five workloads of the FP8 / 2:4 GEMM layers.

This module only draws numbers.  It holds no quantisation, pruning, packing or
GEMM arithmetic, so both the HIP path and the CPU oracle can take their inputs
from it without sharing any of the method's code.

Recipe (the same bytes go to the GPU and to the oracle):
* one NumPy ``Generator(PCG64)`` per tensor, spawned in a fixed order from
  ``SeedSequence(seed)``; the default seed of each workload is its number;
* activations are N(0, 1) and weights N(0, 0.02), drawn as fp32
  (``standard_normal(dtype=float32)``; the weight is scaled by float32(0.02));
* the dense workload's activations carry 1% outliers: an i.i.d.
  Bernoulli(0.01) mask, drawn from its own stream, multiplies entries by 20;
* bf16 operands are the fp32 draws rounded to nearest-even bf16.

Shapes (rows x K, row-major):
1. tiny 2:4:     X [64, 256],   W [128, 256]
2. dense:        X [2048, 4096] (with outliers), W [4096, 4096]
3. 2:4 large:    X [2048, 4096], W [4096, 4096]
4. decode 2:4:   X [M, K], W [N, K]; M in {16, 37}; (N, K) in {(14336, 4096), (4096, 14336)}
5. fused add:    X1 [2048, 4096], W1 [4096, 4096] (fp32, to be int4-quantised),
                 X2 [2048, 64], W2 [4096, 64] (bf16 bits)
"""

import numpy as np

ACT_STD = 1.0
W_STD = 0.02
OUTLIER_P = 0.01
OUTLIER_MUL = 20.0


def generators(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def normal(gen, shape, std: float = 1.0) -> np.ndarray:
    a = gen.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def tiny_sparse(seed: int = 1, m: int = 64, n: int = 128, k: int = 256):
    gx, gw = generators(seed, 2)
    return {"x": normal(gx, (m, k), ACT_STD), "w": normal(gw, (n, k), W_STD)}


def dense_outliers(seed: int = 2, m: int = 2048, n: int = 4096, k: int = 4096):
    gx, gm, gw = generators(seed, 3)
    x = normal(gx, (m, k), ACT_STD)
    mask = gm.random((m, k), dtype=np.float32) < np.float32(OUTLIER_P)
    x[mask] *= np.float32(OUTLIER_MUL)
    return {"x": x, "w": normal(gw, (n, k), W_STD)}


def sparse_large(seed: int = 3, m: int = 2048, n: int = 4096, k: int = 4096):
    gx, gw = generators(seed, 2)
    return {"x": normal(gx, (m, k), ACT_STD), "w": normal(gw, (n, k), W_STD)}


DECODE_SHAPES = [(16, 14336, 4096), (16, 4096, 14336), (37, 14336, 4096), (37, 4096, 14336)]


def decode(seed: int = 4, m: int = 16, n: int = 14336, k: int = 4096):
    gx, gw = generators(seed, 2)
    return {"x": normal(gx, (m, k), ACT_STD), "w": normal(gw, (n, k), W_STD)}


def mixed_add(seed: int = 5, m: int = 2048, n: int = 4096, k1: int = 4096, k2: int = 64):
    g1, g2, g3, g4 = generators(seed, 4)
    return {
        "x1": normal(g1, (m, k1), ACT_STD),
        "w1": normal(g2, (n, k1), W_STD),
        "x2": to_bf16_bits(normal(g3, (m, k2), ACT_STD)),
        "w2": to_bf16_bits(normal(g4, (n, k2), W_STD)),
    }


def random_e4m3_codes(gen, shape) -> np.ndarray:
    """Uniform random finite e4m3 codes (NaN patterns 0x7F / 0xFF excluded)."""
    c = gen.integers(0, 254, size=shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)                  # skip 0x7F
    return c.astype(np.uint8)


def random_int8_codes(gen, shape) -> np.ndarray:
    """Uniform random symmetric int8 codes in [-127, 127]."""
    return gen.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)


def random_scales(gen, shape) -> np.ndarray:
    """Positive fp32 scales spread over a few binades."""
    return np.exp2(gen.uniform(-12.0, 2.0, size=shape)).astype(np.float32)


def small_ints(gen, shape, vmax: int) -> np.ndarray:
    """Integer-valued fp32 in [-vmax, vmax] (every such value is an exact e4m3,
    int8 and bf16 number for vmax <= 16)."""
    return gen.integers(-vmax, vmax + 1, size=shape).astype(np.float32)


def two_of_four_ints(gen, shape, vmax: int) -> np.ndarray:
    """Integer-valued fp32 [rows, k] with exactly two nonzero entries, each in
    +-[1, vmax], at random positions of every aligned group of four along k."""
    rows, k = shape
    g = k // 4
    # positions: a random pair out of the 6 pairs of a group of four
    pairs = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])
    pick = pairs[gen.integers(0, 6, size=(rows, g))]                       # [rows, g, 2]
    mag = gen.integers(1, vmax + 1, size=(rows, g, 2))
    sign = np.where(gen.random((rows, g, 2)) < 0.5, -1, 1)
    out = np.zeros((rows, g, 4), dtype=np.float32)
    r_idx = np.arange(rows)[:, None, None]
    g_idx = np.arange(g)[None, :, None]
    out[r_idx, g_idx, pick] = (mag * sign).astype(np.float32)
    return out.reshape(rows, k)


def pow2_scales(gen, shape, emin: int, emax: int) -> np.ndarray:
    """fp32 powers of two 2^e, e uniform in [emin, emax]."""
    return np.exp2(gen.integers(emin, emax + 1, size=shape)).astype(np.float32)


def exact_ints(seed: int, m: int, n: int, k: int, vmax: int = 3, emin: int = -1, emax: int = 1,
               x_scale_rows: int = None, w_scale_rows: int = None):
    """Operands whose GEMM is exact in fp32: integer-valued X [m, k] in
    [-vmax, vmax], W [n, k] with two integer nonzeros per group of four, and
    power-of-two scales for X [x_scale_rows, k/128] and W [w_scale_rows, k/128]
    (defaults: one per X row, one per 128 W rows)."""
    gx, gw, gsx, gsw = generators(seed, 4)
    xs = m if x_scale_rows is None else x_scale_rows
    ws = -(-n // 128) if w_scale_rows is None else w_scale_rows
    return {"x": small_ints(gx, (m, k), vmax), "w": two_of_four_ints(gw, (n, k), vmax),
            "sx": pow2_scales(gsx, (xs, k // 128), emin, emax), "sw": pow2_scales(gsw, (ws, k // 128), emin, emax)}
