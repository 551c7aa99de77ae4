"""Seeded sweeps of random ragged shapes through every GEMM entry point,
against the oracle: sparse and dense FP8 (canonical and packed weights, both
output forms, every scale-granularity mode, bf16 and fp32 outputs), int8 x
int8 2:4, and the weight-only GEMM with e4m3, int8 and int4 codes (including
shapes wide enough for its large-M tile kernel).  Shapes are drawn once, from
a fixed seed, so the cases are the same on every run; each names its draw."""
import numpy as np
import pytest
import torch

from test_gpu_gemm import check as check_fp8
from test_gpu_int8 import check as check_int8
from test_gpu_w8a16 import check as check_w8, check_w4

pytestmark = pytest.mark.gpu


def _draws(seed, count, wide=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 400))]))
        n = int(rng.integers(2000, 9000)) if wide and i % 2 else int(rng.integers(1, 900))
        k = 128 * int(rng.integers(1, 5))
        out.append((i, m, n, k, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("case", _draws(901, 16), ids=lambda c: f"d{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_sweep_fp8(case):
    i, m, n, k, s = case
    rng = np.random.default_rng(s)
    sparse = bool(rng.integers(0, 2)) or i % 4 == 0
    packed = sparse and bool(rng.integers(0, 2))
    gm, gn = int(rng.choice([1, 128])), int(rng.choice([1, 128]))
    out = torch.float32 if rng.integers(0, 2) else torch.bfloat16
    check_fp8(sparse, m, n, k, gm=gm, gn=gn, out_dtype=out, seed=s % 1000, packed=packed,
              m_major=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("case", _draws(902, 8), ids=lambda c: f"d{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_sweep_int8(case):
    i, m, n, k, s = case
    rng = np.random.default_rng(s)
    check_int8(m, n, k, gm=int(rng.choice([1, 128])), gn=int(rng.choice([1, 128])),
               out_dtype=torch.float32 if rng.integers(0, 2) else torch.bfloat16, seed=s % 1000,
               packed=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("case", _draws(903, 12, wide=True), ids=lambda c: f"d{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_sweep_weight_only(case):
    i, m, n, k, s = case
    rng = np.random.default_rng(s)
    out = torch.float32 if rng.integers(0, 2) else torch.bfloat16
    bias = bool(rng.integers(0, 2))
    if i % 3 == 2:
        check_w4(m, n, k, out=out, bias=bias, seed=s % 1000)
    else:
        check_w8(m, n, k, gn=int(rng.choice([1, 128])), int8=bool(i % 3), out=out, bias=bias, seed=s % 1000)
