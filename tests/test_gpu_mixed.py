"""GPU parity of the fused int4 + bf16 add against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, assert_within_tolerance, down, say, up, up_scales

pytestmark = pytest.mark.gpu


def check(m, n, k1, k2, seed):
    say(f"mixed M={m} N={n} K1={k1} K2={k2} seed={seed}")
    d = workloads.mixed_add(seed=seed, m=m, n=n, k1=k1, k2=k2)
    x1, sx1 = oracle.int4_quant_groupwise(d["x1"], 128)
    w1, sw1 = oracle.int4_quant_groupwise(d["w1"], 128)
    ref, bound = oracle.mixed_gemm_add(x1, sx1, w1, sw1, d["x2"], d["w2"], bound=True)
    x2 = up(d["x2"]) if k2 else None
    w2 = up(d["w2"]) if k2 else None
    y = down(sg.mixed_gemm_add(up(x1), up_scales(sx1), up(w1), up_scales(sw1), x2, w2))
    assert_within_tolerance(y, ref, bound, "mixed")
    return y


# K1 / 128 odd (the last int4 double stage has one K block), K2 a multiple of
# 32 but not of 64 (the last bf16 stage has one half), several tiles in M and
# N with ragged tails, K2 = 0, and int4 / bf16 stage counts of either parity.
@pytest.mark.parametrize("m,n,k1,k2", [(1, 256, 128, 32), (37, 300, 256, 64), (128, 256, 256, 96),
                                       (200, 513, 384, 0), (129, 256, 128, 128), (300, 700, 640, 192),
                                       (257, 520, 896, 160), (64, 1030, 512, 32)])
def test_mixed_ragged(m, n, k1, k2):
    check(m, n, k1, k2, seed=m + n)


def test_mixed_padded_output_untouched():
    """Partial tiles store inside [M, N] only; a wider output row (ld not a
    multiple of 8 elements) takes the element-wise store path."""
    m, n, k1, k2 = 150, 300, 256, 64
    d = workloads.mixed_add(seed=17, m=m, n=n, k1=k1, k2=k2)
    x1, sx1 = oracle.int4_quant_groupwise(d["x1"], 128)
    w1, sw1 = oracle.int4_quant_groupwise(d["w1"], 128)
    ref, bound = oracle.mixed_gemm_add(x1, sx1, w1, sw1, d["x2"], d["w2"], bound=True)
    ybuf = torch.full((m + 2, n + 5), 3.0, dtype=torch.bfloat16, device=DEV)
    sg.mixed_gemm_add(up(x1), up_scales(sx1), up(w1), up_scales(sw1), up(d["x2"]), up(d["w2"]), y=ybuf[:m, :n])
    yb = down(ybuf)
    assert np.all(yb[m:, :] == 3.0) and np.all(yb[:, n:] == 3.0)
    assert_within_tolerance(yb[:m, :n], ref, bound, "mixed padded")


def test_mixed_full_size():
    """L = 2048, D1 = 4096, D2 = 64, D = 4096 (the issue's example shape)."""
    check(2048, 4096, 4096, 64, seed=5)


def test_mixed_end_to_end_with_gpu_int4_quantiser():
    d = workloads.mixed_add(seed=6, m=64, n=256, k1=512, k2=64)
    x1, sx1 = sg.int4_quant_groupwise(up(d["x1"]))
    w1, sw1 = sg.int4_quant_groupwise(up(d["w1"]))
    y = down(sg.mixed_gemm_add(x1, sx1, w1, sw1, up(d["x2"]), up(d["w2"])))
    ox1, osx1 = oracle.int4_quant_groupwise(d["x1"], 128)
    ow1, osw1 = oracle.int4_quant_groupwise(d["w1"], 128)
    ref, bound = oracle.mixed_gemm_add(ox1, osx1, ow1, osw1, d["x2"], d["w2"], bound=True)
    assert_within_tolerance(y, ref, bound, "mixed end-to-end")
