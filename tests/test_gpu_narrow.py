"""Narrow outputs: N of 1, 3 and 17 W rows (every 16-row block and every
large-M tile partial in N) through each GEMM family, at decode and large M,
against the oracle."""
import pytest
import torch

from test_gpu_gemm import check as check_fp8
from test_gpu_int8 import check as check_int8
from test_gpu_w8a16 import check as check_w8, check_w4

pytestmark = pytest.mark.gpu

SHAPES = [(m, n) for m in (1, 65, 130) for n in (1, 3, 17)]


@pytest.mark.parametrize("m,n", SHAPES)
@pytest.mark.parametrize("kind", ["dense", "sparse", "packed"])
def test_narrow_fp8(m, n, kind):
    check_fp8(kind != "dense", m, n, 256, gn=128 if kind == "packed" else 1, out_dtype=torch.float32,
              seed=m + n, packed=kind == "packed")


@pytest.mark.parametrize("m,n", SHAPES)
def test_narrow_int8(m, n):
    check_int8(m, n, 256, out_dtype=torch.float32, seed=m + n, packed=True)


@pytest.mark.parametrize("m,n", SHAPES)
def test_narrow_weight_only(m, n):
    check_w8(m, n, 256, gn=1, int8=bool(n % 2), out=torch.float32, bias=True, seed=m + n)
    check_w4(m, n, 256, out=torch.float32, seed=m + n + 1)
