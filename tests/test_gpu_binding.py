"""The Python binding refuses ill-formed tensors with SgError before any call
into the library: wrong code dtypes, outputs of the wrong shape or dtype,
scale tensors that are too small, on the host or not fp32, weights whose K
does not match X, and empty problems."""
import pytest
import torch

import sparse_gemm_layers_amd as sg
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

M, N, K = 64, 256, 512


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8, device=DEV)


def i8(*shape):
    return torch.zeros(shape, dtype=torch.int8, device=DEV)


def f32(*shape, dev=DEV):
    return torch.ones(shape, dtype=torch.float32, device=dev)


def scales(rows, kb):
    return f32(kb, rows).t()


GOOD = dict(xq=lambda: u8(M, K), sx=lambda: scales(M, K // 128), wq=lambda: u8(N, K),
            sw=lambda: scales(N // 128, K // 128))


def dense(**kw):
    a = {k: v() for k, v in GOOD.items()}
    a.update(kw)
    return sg.fp8_gemm_groupwise(a["xq"], a["sx"], a["wq"], a["sw"], 1, 128, y=a.get("y"),
                                 out_dtype=a.get("out_dtype", torch.bfloat16), form=a.get("form", "y"))


def test_valid_call_passes():
    torch.cuda.synchronize()
    assert dense().shape == (M, N)


# Each case builds its tensors when it runs (lambdas), so collecting the tests
# needs no GPU.
@pytest.mark.parametrize("what,kw", [
    ("W with another K", lambda: dict(wq=u8(N, K - 128))),
    ("int8 X codes to the FP8 GEMM", lambda: dict(xq=i8(M, K))),
    ("float X", lambda: dict(xq=f32(M, K))),
    ("X scales with too few rows", lambda: dict(sx=scales(M - 1, K // 128))),
    ("X scales with too few K blocks", lambda: dict(sx=scales(M, K // 128 - 1))),
    ("W scales with too few row blocks", lambda: dict(sw=scales(1, K // 128))),
    ("float16 scales", lambda: dict(sx=scales(M, K // 128).half())),
    ("host scales", lambda: dict(sw=f32(N // 128, K // 128, dev="cpu"))),
    ("1-D scales", lambda: dict(sx=f32(M))),
    ("output of the wrong shape", lambda: dict(y=torch.empty((M, N - 16), dtype=torch.bfloat16, device=DEV))),
    ("transposed output of the Y shape",
     lambda: dict(form="yt", y=torch.empty((M, N), dtype=torch.bfloat16, device=DEV))),
    ("int32 output", lambda: dict(y=torch.empty((M, N), dtype=torch.int32, device=DEV))),
    ("unknown form", lambda: dict(form="z")),
    ("empty X", lambda: dict(xq=u8(0, K), sx=scales(1, K // 128))),
])
def test_dense_gemm_rejects(what, kw):
    say(f"binding rejects: {what}")
    with pytest.raises(sg.SgError):
        dense(**kw())


def test_sparse_gemm_rejects_mismatched_codes_and_metadata():
    xq, sx, sw = u8(M, K), scales(M, K // 128), scales(N // 128, K // 128)
    with pytest.raises(sg.SgError):     # values for another K
        sg.fp8_sparse24_gemm_groupwise(xq, sx, u8(N, K // 2 + 16), u8(N, K // 8), sw)
    with pytest.raises(sg.SgError):     # metadata for another K
        sg.fp8_sparse24_gemm_groupwise(xq, sx, u8(N, K // 2), u8(N, K // 16), sw)
    with pytest.raises(sg.SgError):     # metadata rows != N
        sg.fp8_sparse24_gemm_groupwise(xq, sx, u8(N, K // 2), u8(N - 1, K // 8), sw)
    with pytest.raises(sg.SgError):     # int8 values to the FP8 GEMM
        sg.fp8_sparse24_gemm_groupwise(xq, sx, i8(N, K // 2), u8(N, K // 8), sw)
    with pytest.raises(sg.SgError):     # FP8 codes to the int8 GEMM
        sg.int8_sparse24_gemm_groupwise(xq, sx, i8(N, K // 2), u8(N, K // 8), sw)


def test_packed_gemm_rejects_short_or_mistyped_weights():
    xq, sx, sw = u8(M, K), scales(M, K // 128), scales(N // 128, K // 128)
    need = sg.sparse24_packed_bytes(N, K)
    with pytest.raises(sg.SgError):
        sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, u8(need - 1), N, sw)
    with pytest.raises(sg.SgError):
        sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, i8(need), N, sw)
    with pytest.raises(sg.SgError):
        sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, u8(need), 0, sw)


def test_quantisers_and_pruner_reject_bad_outputs():
    x = f32(4, 256)
    with pytest.raises(sg.SgError):
        sg.fp8_quant_groupwise(x, q=i8(4, 256))
    with pytest.raises(sg.SgError):
        sg.fp8_quant_groupwise(x, q=u8(4, 128))
    with pytest.raises(sg.SgError):
        sg.fp8_quant_groupwise(x, s=scales(3, 2))
    with pytest.raises(sg.SgError):
        sg.int8_quant_groupwise(x, q=u8(4, 256))
    with pytest.raises(sg.SgError):
        sg.int4_quant_groupwise(x, q=u8(4, 256))
    with pytest.raises(sg.SgError):
        sg.fp8_quant_groupwise(f32(0, 256))
    with pytest.raises(sg.SgError):
        sg.sparse24_prune_compress(x, vals=torch.empty((4, 128), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(sg.SgError):
        sg.sparse24_prune_compress(x, meta=u8(4, 16))
    with pytest.raises(sg.SgError):
        sg.sparse24_prune_compress(i8(4, 256))


def test_batched_and_grouped_reject_mismatches():
    L = 3
    xq, sx = u8(L, M, K), f32(L, M, K // 128)
    with pytest.raises(sg.SgError):     # scales for 2 problems, 3 given
        sg.fp8_sparse24_gemm_groupwise_packed_batched(xq, f32(2, M, K // 128),
                                                      u8(sg.sparse24_packed_bytes(N, K)), N,
                                                      scales(N // 128, K // 128))
    with pytest.raises(sg.SgError):     # output of the wrong batch
        sg.fp8_gemm_groupwise_batched(xq, sx, u8(N, K), scales(N // 128, K // 128),
                                      y=torch.empty((2, M, N), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(sg.SgError):     # weights for 2 problems, 3 given
        sg.fp8_gemm_groupwise_batched(xq, sx, u8(2, N, K), scales(N // 128, K // 128))
    wp = u8(2, sg.sparse24_packed_bytes(N, K))
    with pytest.raises(sg.SgError):     # every group empty
        sg.fp8_sparse24_gemm_groupwise_packed_grouped(u8(0, K), scales(1, K // 128), [0, 0], wp, N,
                                                      scales(N // 128, K // 128))
    with pytest.raises(sg.SgError):     # sizes that do not sum to X's rows
        sg.fp8_sparse24_gemm_groupwise_packed_grouped(u8(10, K), scales(10, K // 128), [4, 5], wp, N,
                                                      scales(N // 128, K // 128))


def test_weight_only_and_mixed_reject_mismatches():
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sg.SgError):
        sg.w8a16_sparse24_gemm_groupwise(x, u8(N, K // 2), u8(N, K // 4), scales(N // 128, K // 128))
    with pytest.raises(sg.SgError):
        sg.w4a16_sparse24_gemm_groupwise(x, u8(N, K // 2), u8(N, K // 8), scales(N, K // 128))
    x1, w1 = u8(M, K // 2), u8(N, K // 2)
    x2 = torch.zeros((M, 64), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((N, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sg.SgError):     # fp32 output
        sg.mixed_gemm_add(x1, scales(M, K // 128), w1, scales(N, K // 128), x2, w2,
                          y=torch.empty((M, N), dtype=torch.float32, device=DEV))
    with pytest.raises(sg.SgError):     # W1 scales per 128 rows instead of per row
        sg.mixed_gemm_add(x1, scales(M, K // 128), w1, scales(N // 128, K // 128), x2, w2)
    with pytest.raises(sg.SgError):     # X2 with another K2 than W2
        sg.mixed_gemm_add(x1, scales(M, K // 128), w1, scales(N, K // 128), x2[:, :32], w2)
