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
