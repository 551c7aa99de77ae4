"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph over the
binding's launches, as the benchmark replays its steps): activation
quantisation and the packed 2:4 FP8 GEMM, and the fused-quantisation decode
GEMM.  Each graph is replayed several times, with the program's own eager
work and synchronisations in between, and every replay must equal the eager
result bit for bit (the library records no memset and allocates nothing, so
a replay repeats exactly the eager launches)."""
import numpy as np
import pytest
import torch

import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def layer(seed, m, n, k):
    d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
    x, w = torch.from_numpy(d["x"]).to(DEV), torch.from_numpy(d["w"]).to(DEV)
    wv, meta = sg.sparse24_prune_compress(w)
    wq, sw = sg.fp8_quant_groupwise(wv, gr=128, gc=64)
    return x, sg.sparse24_pack_gfx950(wq, meta), sw


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    return g


@pytest.mark.parametrize("m,n,k", [(2048, 4096, 4096), (300, 512, 384)])
def test_quantise_then_gemm_replays_equal_eager(m, n, k):
    say(f"graph quant+gemm {m}x{n}x{k}")
    x, wp, sw = layer(7, m, n, k)
    xq = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    sx = torch.empty((k // 128, m), dtype=torch.float32, device=DEV).t()
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def step():
        sg.fp8_quant_groupwise(x, gr=1, gc=128, q=xq, s=sx)
        sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, wp, n, sw, 1, 128, y=y)

    step()
    torch.cuda.synchronize()
    want = y.view(torch.int16).cpu().numpy().copy()
    g = capture(step)
    for r in range(3):
        y.zero_()                                  # eager work between replays
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.view(torch.int16).cpu().numpy(), want), f"replay {r}"
        del junk


def test_fused_quant_decode_replays_equal_eager():
    m, n, k = 16, 2048, 1024
    x, wp, sw = layer(8, m, n, k)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def step():
        sg.fp8_sparse24_gemm_packed_quant_x(x, wp, n, sw, 128, y=y)

    step()
    torch.cuda.synchronize()
    want = y.view(torch.int16).cpu().numpy().copy()
    g = capture(step)
    for r in range(3):
        y.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.view(torch.int16).cpu().numpy(), want), f"replay {r}"
