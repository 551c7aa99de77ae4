"""The C-ABI library loads, exports every entry point include/sg.h declares,
and rejects invalid arguments on the host before any HIP call.

These tests pass fake (never dereferenced) device addresses, so they only run
where no GPU is visible: every call here must return before touching HIP."""
import ctypes
import os
import re

import pytest
import torch

import sparse_gemm_layers_amd as sg
from sparse_gemm_layers_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("sg.h", "sg_probe.h")]

OK, NULL, SHAPE, UNSUP, ALIGN, HIP = range(6)
P = ctypes.c_void_p(0x100000)          # 16-byte aligned fake address
P2 = ctypes.c_void_p(0x200000)
P3 = ctypes.c_void_p(0x300000)
ODD = ctypes.c_void_p(0x100004)        # 4- but not 16-byte aligned

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer checks run only without a GPU")


def declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sg_[a-z0-9_]+)\s*\(", src)))


def test_include_holds_only_the_known_headers():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["sg.h", "sg_probe.h"]


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "sg_abi_version", "sg_status_str", "sg_fp8_quant_groupwise", "sg_int4_quant_groupwise",
        "sg_sparse24_prune_compress", "sg_fp8_gemm_groupwise", "sg_fp8_sparse24_gemm_groupwise",
        "sg_mixed_gemm_add", "sg_sparse24_packed_bytes", "sg_sparse24_pack_gfx950",
        "sg_fp8_sparse24_gemm_groupwise_packed", "sg_probe_matrix_ops", "sg_probe_matrix_rate",
        "sg_int8_quant_groupwise", "sg_int8_sparse24_gemm_groupwise", "sg_int8_sparse24_gemm_groupwise_packed",
        "sg_fp8_gemm_groupwise_batched", "sg_fp8_sparse24_gemm_groupwise_batched",
        "sg_fp8_sparse24_gemm_groupwise_packed_batched", "sg_fp8_sparse24_gemm_groupwise_packed_grouped",
        "sg_w8a16_sparse24_gemm_groupwise", "sg_w8a16_sparse24_gemm_groupwise_packed",
        "sg_w4a16_sparse24_gemm_groupwise", "sg_w4a16_sparse24_gemm_groupwise_packed",
        "sg_sparse24_w4_packed_bytes", "sg_sparse24_pack_w4",
        "sg_fp8_sparse24_gemm_packed_quant_x", "sg_probe_stream_read"])


def test_library_exports_every_declared_symbol():
    lib = sg.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(B._SIGS) == set(declared_functions())


def test_status_strings_and_version():
    lib = sg.lib()
    assert lib.sg_abi_version() == 3
    for code, word in [(OK, b"SG_OK"), (NULL, b"SG_ERR_NULL"), (SHAPE, b"SG_ERR_SHAPE"),
                       (UNSUP, b"SG_ERR_UNSUPPORTED"), (ALIGN, b"SG_ERR_ALIGN"), (HIP, b"SG_ERR_HIP")]:
        assert lib.sg_status_str(code).startswith(word)
    assert lib.sg_status_str(99) == b"unknown sg_status"


def quant(**kw):
    a = dict(x=P, dt=0, rows=4, cols=256, ldx=256, gr=1, gc=128, q=P2, ldq=256, s=P3, ssr=1, ssc=4)
    a.update(kw)
    return sg.lib().sg_fp8_quant_groupwise(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["gr"], a["gc"],
                                           a["q"], a["ldq"], a["s"], a["ssr"], a["ssc"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(q=None), NULL), (dict(s=None), NULL),
    (dict(dt=2), UNSUP), (dict(dt=7), UNSUP), (dict(gr=2), UNSUP), (dict(gc=32), UNSUP),
    (dict(cols=200), SHAPE), (dict(cols=0), SHAPE), (dict(rows=-1), SHAPE), (dict(ldx=128), SHAPE),
    (dict(ldq=100), SHAPE), (dict(x=ODD), ALIGN), (dict(ldx=258), ALIGN), (dict(ldq=264), ALIGN),
    (dict(rows=0), SHAPE),
    (dict(gc=256, rows=0), SHAPE), (dict(gr=0, gc=256, rows=0), SHAPE), (dict(gr=3, gc=256), UNSUP),
    (dict(cols=200, gc=200, ldx=208, ldq=208, rows=0), UNSUP), (dict(gr=4, gc=256, ldq=100), SHAPE),
    (dict(gc=128, cols=256, gr=4), UNSUP),
])
def test_fp8_quant_validation(kw, code):
    assert quant(**kw) == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(q=None), NULL), (dict(dt=2), UNSUP), (dict(gr=2), UNSUP), (dict(gc=32), UNSUP),
    (dict(cols=200), SHAPE), (dict(ldq=100), SHAPE), (dict(x=ODD), ALIGN), (dict(ldq=264), ALIGN),
    (dict(rows=0), SHAPE), (dict(rows=-3), SHAPE),
])
def test_int8_quant_validation(kw, code):
    a = dict(x=P, dt=0, rows=4, cols=256, ldx=256, gr=1, gc=128, q=P2, ldq=256, s=P3, ssr=1, ssc=4)
    a.update(kw)
    assert sg.lib().sg_int8_quant_groupwise(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["gr"], a["gc"],
                                            a["q"], a["ldq"], a["s"], a["ssr"], a["ssc"], None) == code


def int4q(**kw):
    a = dict(x=P, dt=1, rows=4, cols=256, ldx=256, gc=128, q=P2, ldq=128, s=P3, ssr=2, ssc=1)
    a.update(kw)
    return sg.lib().sg_int4_quant_groupwise(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["gc"], a["q"],
                                            a["ldq"], a["s"], a["ssr"], a["ssc"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(dt=2), UNSUP), (dict(cols=64), SHAPE), (dict(ldq=64), SHAPE),
    (dict(ldq=130), ALIGN), (dict(x=ODD), ALIGN), (dict(rows=0), SHAPE),
    (dict(gc=32), UNSUP), (dict(gc=64, cols=200, ldx=208, ldq=104), SHAPE),
    (dict(gc=64, cols=320, ldx=320, ldq=160, rows=0), SHAPE),
])
def test_int4_quant_validation(kw, code):
    assert int4q(**kw) == code


def prune(**kw):
    a = dict(w=P, dt=0, rows=8, k=64, ldw=64, v=P2, ldv=32, m=P3, ldm=8)
    a.update(kw)
    return sg.lib().sg_sparse24_prune_compress(a["w"], a["dt"], a["rows"], a["k"], a["ldw"], a["v"], a["ldv"],
                                               a["m"], a["ldm"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(w=None), NULL), (dict(v=None), NULL), (dict(m=None), NULL), (dict(dt=3), UNSUP), (dict(dt=9), UNSUP),
    (dict(k=12), SHAPE), (dict(k=0), SHAPE), (dict(ldw=32), SHAPE), (dict(ldv=16), SHAPE), (dict(ldm=4), SHAPE),
    (dict(v=ODD), ALIGN), (dict(ldw=66), ALIGN), (dict(ldv=34), ALIGN), (dict(rows=0), SHAPE),
    (dict(rows=-1), SHAPE),
    # e4m3 codes (dt 2): byte rows, 16-byte aligned leading dimension
    (dict(dt=2, rows=0), SHAPE), (dict(dt=2, ldw=72), ALIGN), (dict(dt=2, ldv=34), ALIGN),
    (dict(dt=2, ldm=4), SHAPE), (dict(dt=2, w=None), NULL),
])
def test_prune_validation(kw, code):
    assert prune(**kw) == code


def gemm(sparse=False, **kw):
    a = dict(M=64, N=256, K=256, x=P, ldx=256, sx=P3, sxm=1, sxk=64, gm=1, w=P2, ldw=256, meta=P3, ldm=32,
             sw=P3, swn=2, swk=1, gn=128, y=P, ydt=1, ldy=256, form=0)
    a.update(kw)
    lib = sg.lib()
    if sparse:
        ldw = a["ldw"] if "ldw" in kw else a["K"] // 2
        return lib.sg_fp8_sparse24_gemm_groupwise(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["sx"], a["sxm"],
                                                  a["sxk"], a["gm"], a["w"], ldw, a["meta"], a["ldm"], a["sw"],
                                                  a["swn"], a["swk"], a["gn"], a["y"], a["ydt"], a["ldy"],
                                                  a["form"], None)
    return lib.sg_fp8_gemm_groupwise(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["sx"], a["sxm"], a["sxk"],
                                     a["gm"], a["w"], a["ldw"], a["sw"], a["swn"], a["swk"], a["gn"], a["y"],
                                     a["ydt"], a["ldy"], a["form"], None)


GEMM_CASES = [
    (dict(x=None), NULL), (dict(sx=None), NULL), (dict(w=None), NULL), (dict(sw=None), NULL), (dict(y=None), NULL),
    (dict(gm=64), UNSUP), (dict(gn=2), UNSUP), (dict(ydt=2), UNSUP), (dict(form=2), UNSUP),
    (dict(K=0), SHAPE), (dict(K=200), SHAPE), (dict(M=-1), SHAPE), (dict(ldx=128), SHAPE),
    (dict(ldy=100), SHAPE), (dict(form=1, ldy=32), SHAPE),
    (dict(x=ODD), ALIGN), (dict(ldx=264), ALIGN), (dict(y=ctypes.c_void_p(0x100001)), ALIGN),
    (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(N=-5), SHAPE),
]


@no_gpu
@pytest.mark.parametrize("kw,code", GEMM_CASES + [(dict(ldw=128), SHAPE), (dict(w=ODD), ALIGN)])
def test_dense_gemm_validation(kw, code):
    assert gemm(False, **kw) == code


@no_gpu
@pytest.mark.parametrize("kw,code", GEMM_CASES + [
    (dict(meta=None), NULL), (dict(ldw=64), SHAPE), (dict(ldm=16), SHAPE), (dict(meta=ODD), ALIGN),
    (dict(ldm=40), ALIGN)])
def test_sparse_gemm_validation(kw, code):
    assert gemm(True, **kw) == code


@no_gpu
@pytest.mark.parametrize("kw,code", GEMM_CASES + [
    (dict(meta=None), NULL), (dict(ldw=64), SHAPE), (dict(ldm=16), SHAPE), (dict(meta=ODD), ALIGN)])
def test_int8_sparse_gemm_validation(kw, code):
    a = dict(M=64, N=256, K=256, x=P, ldx=256, sx=P3, sxm=1, sxk=64, gm=1, w=P2, meta=P3, ldm=32,
             sw=P3, swn=2, swk=1, gn=128, y=P, ydt=1, ldy=256, form=0)
    a.update(kw)
    ldw = a["ldw"] if "ldw" in kw else a["K"] // 2
    assert sg.lib().sg_int8_sparse24_gemm_groupwise(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["sx"], a["sxm"],
                                                    a["sxk"], a["gm"], a["w"], ldw, a["meta"], a["ldm"], a["sw"],
                                                    a["swn"], a["swk"], a["gn"], a["y"], a["ydt"], a["ldy"],
                                                    a["form"], None) == code


def mixed(**kw):
    a = dict(M=16, N=256, K1=256, K2=64, x1=P, ldx1=128, sx1=P3, sxm=2, sxk=1, w1=P2, ldw1=128, sw1=P3, swn=2,
             swk=1, x2=P, ldx2=64, w2=P2, ldw2=64, y=P, ldy=256)
    a.update(kw)
    return sg.lib().sg_mixed_gemm_add(a["M"], a["N"], a["K1"], a["K2"], a["x1"], a["ldx1"], a["sx1"], a["sxm"],
                                      a["sxk"], a["w1"], a["ldw1"], a["sw1"], a["swn"], a["swk"], a["x2"],
                                      a["ldx2"], a["w2"], a["ldw2"], a["y"], a["ldy"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x1=None), NULL), (dict(x2=None), NULL), (dict(K2=0, x2=None, w2=None, M=0), SHAPE),
    (dict(K1=100), SHAPE), (dict(K2=48), SHAPE), (dict(ldx1=64), SHAPE), (dict(ldx2=32), SHAPE),
    (dict(ldy=100), SHAPE), (dict(x1=ODD), ALIGN), (dict(ldw2=68), ALIGN), (dict(N=0), SHAPE),
])
def test_mixed_validation(kw, code):
    assert mixed(**kw) == code


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(4, 128)
    with pytest.raises(sg.SgError):
        sg.fp8_quant_groupwise(x)


def test_packed_bytes():
    lib = sg.lib()
    assert lib.sg_sparse24_packed_bytes(4096, 4096) == 256 * 32 * 1280
    assert lib.sg_sparse24_packed_bytes(300, 384) == 19 * 3 * 1280
    assert lib.sg_sparse24_packed_bytes(0, 128) == -1
    assert lib.sg_sparse24_packed_bytes(10, 100) == -1 and lib.sg_sparse24_packed_bytes(-1, 128) == -1


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(wv=None), NULL), (dict(packed=None), NULL), (dict(K=100), SHAPE), (dict(ldwv=32), SHAPE),
    (dict(ldwm=24), ALIGN), (dict(packed=ODD), ALIGN), (dict(N=0), SHAPE),
])
def test_pack_validation(kw, code):
    a = dict(wv=P, ldwv=64, meta=P2, ldwm=16, N=8, K=128, packed=P3)
    a.update(kw)
    assert sg.lib().sg_sparse24_pack_gfx950(a["wv"], a["ldwv"], a["meta"], a["ldwm"], a["N"], a["K"],
                                            a["packed"], None) == code


@no_gpu
@pytest.mark.parametrize("kw,code", [(dict(w=None), NULL), (dict(w=ODD), ALIGN), (dict(K=200), SHAPE),
                                     (dict(M=0), SHAPE)])
def test_packed_gemm_validation(kw, code):
    a = dict(M=64, N=256, K=256, x=P, ldx=256, sx=P3, w=P2, sw=P3, y=P)
    a.update(kw)
    assert sg.lib().sg_fp8_sparse24_gemm_groupwise_packed(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["sx"], 1, 64,
                                                          1, a["w"], a["sw"], 2, 1, 128, a["y"], 1, 256, 0,
                                                          None) == code


@no_gpu
def test_probe_rejects_bad_arguments_on_the_host():
    lib = sg.lib()
    assert lib.sg_probe_matrix_rate(0, 10, None, P, None) == NULL
    assert lib.sg_probe_matrix_rate(0, 10, P, None, None) == NULL
    assert lib.sg_probe_matrix_rate(6, 10, P, P2, None) == UNSUP
    assert lib.sg_probe_matrix_rate(-1, 10, P, P2, None) == UNSUP
    assert lib.sg_probe_matrix_rate(0, 0, P, P2, None) == SHAPE
    assert lib.sg_probe_stream_read(None, 64, 4, P, None) == NULL
    assert lib.sg_probe_stream_read(P, 64, 4, None, None) == NULL
    assert lib.sg_probe_stream_read(P, 8, 4, P2, None) == SHAPE
    assert lib.sg_probe_stream_read(P, 72, 4, P2, None) == SHAPE
    assert lib.sg_probe_stream_read(P, 64, 0, P2, None) == SHAPE
    assert lib.sg_probe_stream_read(ODD, 64, 4, P2, None) == ALIGN


def test_probe_operation_counts():
    lib = sg.lib()
    # 1024 workgroups x 8 waves x 8 instructions per round
    assert lib.sg_probe_matrix_ops(0, 1) == 2 * 16 * 16 * 128 * 8 * 8 * 1024
    assert lib.sg_probe_matrix_ops(1, 3) == 3 * 2 * 16 * 16 * 128 * 8 * 8 * 1024
    assert lib.sg_probe_matrix_ops(2, 1) == 2 * 16 * 16 * 64 * 8 * 8 * 1024
    assert lib.sg_probe_matrix_ops(6, 1) == -1 and lib.sg_probe_matrix_ops(0, 0) == -1


def batched(kind, **kw):
    a = dict(L=3, M=64, N=256, K=256, x=P, ldx=256, xb=64 * 256, sx=P3, sxm=1, sxk=64, sxb=64 * 2, gm=1, w=P2,
             ldw=256, wb=256 * 256, meta=P3, ldm=32, mb=256 * 32, sw=P3, swn=2, swk=1, swb=4, gn=128, bias=None,
             bb=0, y=P, ydt=1, ldy=256, yb=64 * 256, form=0)
    a.update(kw)
    lib = sg.lib()
    if kind == "dense":
        return lib.sg_fp8_gemm_groupwise_batched(
            a["L"], a["M"], a["N"], a["K"], a["x"], a["ldx"], a["xb"], a["sx"], a["sxm"], a["sxk"], a["sxb"], a["gm"],
            a["w"], a["ldw"], a["wb"], a["sw"], a["swn"], a["swk"], a["swb"], a["gn"], a["bias"], a["bb"], a["y"],
            a["ydt"], a["ldy"], a["yb"], a["form"], None)
    if kind == "sparse":
        ldw = a["ldw"] if "ldw" in kw else a["K"] // 2
        return lib.sg_fp8_sparse24_gemm_groupwise_batched(
            a["L"], a["M"], a["N"], a["K"], a["x"], a["ldx"], a["xb"], a["sx"], a["sxm"], a["sxk"], a["sxb"], a["gm"],
            a["w"], ldw, a["wb"], a["meta"], a["ldm"], a["mb"], a["sw"], a["swn"], a["swk"], a["swb"], a["gn"],
            a["bias"], a["bb"], a["y"], a["ydt"], a["ldy"], a["yb"], a["form"], None)
    return lib.sg_fp8_sparse24_gemm_groupwise_packed_batched(
        a["L"], a["M"], a["N"], a["K"], a["x"], a["ldx"], a["xb"], a["sx"], a["sxm"], a["sxk"], a["sxb"], a["gm"],
        a["w"], a["wb"], a["sw"], a["swn"], a["swk"], a["swb"], a["gn"], a["bias"], a["bb"], a["y"], a["ydt"],
        a["ldy"], a["yb"], a["form"], None)


BATCH_CASES = [
    (dict(L=-1), SHAPE), (dict(L=65536), SHAPE), (dict(xb=-16), SHAPE), (dict(sxb=-1), SHAPE),
    (dict(swb=-1), SHAPE), (dict(yb=-1), SHAPE), (dict(wb=-16), SHAPE),
    (dict(xb=8), ALIGN), (dict(wb=24), ALIGN),
    (dict(L=0), SHAPE), (dict(M=0), SHAPE), (dict(N=0), SHAPE),
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(K=200), SHAPE), (dict(gm=64), UNSUP),
    (dict(bias=P2, bb=-1), SHAPE), (dict(bias=ctypes.c_void_p(0x200002)), ALIGN),
]


@no_gpu
@pytest.mark.parametrize("kind", ["dense", "sparse", "packed"])
@pytest.mark.parametrize("kw,code", BATCH_CASES)
def test_batched_gemm_validation(kind, kw, code):
    assert batched(kind, **kw) == code


@no_gpu
def test_batched_sparse_metadata_stride_must_be_aligned():
    assert batched("sparse", mb=8) == ALIGN and batched("sparse", meta=None) == NULL


def test_k_constant_scale_views():
    s = torch.arange(5, dtype=torch.float32)
    v = sg.k_constant_scales(s, 5, 512)
    assert v.shape == (5, 4) and v.stride() == (1, 0) and torch.equal(v[:, 3], s)
    t = sg.k_constant_scales(torch.ones(1), 7, 256)
    assert t.shape == (7, 2) and t.stride() == (0, 0)
    with pytest.raises(sg.SgError):
        sg.k_constant_scales(torch.ones(3), 5, 128)


def grouped(sizes, **kw):
    a = dict(N=256, K=256, x=P, ldx=256, sx=P3, sxm=1, sxk=512, w=P2, wb=16 * 2 * 1280, sw=P3, swn=2, swk=1, swb=4,
             gn=128, bias=None, bb=0, y=P, ydt=1, ldy=256, form=0)
    a.update(kw)
    arr = (ctypes.c_int64 * max(len(sizes), 1))(*sizes)
    G = a.pop("G", len(sizes))
    return sg.lib().sg_fp8_sparse24_gemm_groupwise_packed_grouped(
        G, ctypes.cast(arr, ctypes.c_void_p) if a.get("nosizes") is None else None, a["N"], a["K"], a["x"],
        a["ldx"], a["sx"], a["sxm"], a["sxk"], a["w"], a["wb"], a["sw"], a["swn"], a["swk"], a["swb"], a["gn"],
        a["bias"], a["bb"], a["y"], a["ydt"], a["ldy"], a["form"], None)


@no_gpu
@pytest.mark.parametrize("sizes,kw,code", [
    ([10, -1], {}, SHAPE), ([1] * 65, {}, SHAPE), ([5], dict(G=-1), SHAPE), ([5], dict(nosizes=1), NULL),
    ([0, 0, 0], {}, SHAPE), ([], {}, SHAPE), ([5, 7], dict(x=None), NULL), ([5, 7], dict(w=None), NULL),
    ([5, 7], dict(w=ODD), ALIGN), ([5, 7], dict(wb=8), ALIGN), ([5, 7], dict(swb=-1), SHAPE),
    ([5, 7], dict(K=200), SHAPE), ([5, 7], dict(gn=3), UNSUP), ([5, 7], dict(bb=-2, bias=P2), SHAPE),
    ([5, 7], dict(N=0), SHAPE),
])
def test_grouped_gemm_validation(sizes, kw, code):
    assert grouped(sizes, **kw) == code


def w8a16(**kw):
    a = dict(M=16, N=256, K=256, x=P, ldx=256, w=P2, ldw=128, meta=P3, ldm=32, wdt=2, sw=P3, swn=2, swk=1, gn=128,
             bias=None, y=P, ydt=1, ldy=256, form=0)
    a.update(kw)
    return sg.lib().sg_w8a16_sparse24_gemm_groupwise(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["w"], a["ldw"],
                                                     a["meta"], a["ldm"], a["wdt"], a["sw"], a["swn"], a["swk"], a["gn"],
                                                     a["bias"], a["y"], a["ydt"], a["ldy"], a["form"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(meta=None), NULL), (dict(sw=None), NULL), (dict(y=None), NULL),
    (dict(wdt=0), UNSUP), (dict(wdt=1), UNSUP), (dict(gn=64), UNSUP), (dict(ydt=2), UNSUP), (dict(form=3), UNSUP),
    (dict(K=200), SHAPE), (dict(ldx=128), SHAPE), (dict(ldw=64), SHAPE), (dict(ldm=16), SHAPE), (dict(ldy=100), SHAPE),
    (dict(M=65535 * 16 + 1), SHAPE), (dict(swk=-1), SHAPE),
    (dict(x=ODD), ALIGN), (dict(ldx=260), ALIGN), (dict(ldw=136), ALIGN), (dict(ldm=34), ALIGN), (dict(ldm=36), ALIGN),
    (dict(bias=ctypes.c_void_p(0x100002)), ALIGN), (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(wdt=3, M=0), SHAPE),
])
def test_w8a16_validation(kw, code):
    assert w8a16(**kw) == code


def w8a16_packed(**kw):
    a = dict(M=16, N=256, K=256, x=P, ldx=256, w=P2, wdt=2, sw=P3, swn=2, swk=1, gn=128, bias=None, y=P, ydt=1,
             ldy=256, form=0)
    a.update(kw)
    return sg.lib().sg_w8a16_sparse24_gemm_groupwise_packed(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["w"],
                                                            a["wdt"], a["sw"], a["swn"], a["swk"], a["gn"],
                                                            a["bias"], a["y"], a["ydt"], a["ldy"], a["form"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(sw=None), NULL), (dict(y=None), NULL),
    (dict(wdt=0), UNSUP), (dict(wdt=1), UNSUP), (dict(gn=64), UNSUP), (dict(ydt=2), UNSUP), (dict(form=3), UNSUP),
    (dict(K=200), SHAPE), (dict(ldx=128), SHAPE), (dict(ldy=100), SHAPE), (dict(M=65535 * 16 + 1), SHAPE),
    (dict(swk=-1), SHAPE), (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(wdt=3, K=0), SHAPE),
    # (K / 128) * 16 chunks of 1280 bytes must stay below 2^31 (a tile's 32-bit offsets)
    (dict(K=128 * 104858, ldx=128 * 104858), SHAPE), (dict(ldx=1 << 24, K=256), SHAPE),
    (dict(x=ODD), ALIGN), (dict(ldx=260), ALIGN), (dict(w=ODD), ALIGN), (dict(bias=ctypes.c_void_p(0x100002)), ALIGN),
])
def test_w8a16_packed_validation(kw, code):
    assert w8a16_packed(**kw) == code


def test_w4_packed_bytes():
    lib = sg.lib()
    assert lib.sg_sparse24_w4_packed_bytes(14336, 4096) == 896 * 32 * 768
    assert lib.sg_sparse24_w4_packed_bytes(300, 384) == 19 * 3 * 768
    assert lib.sg_sparse24_w4_packed_bytes(0, 128) == -1 and lib.sg_sparse24_w4_packed_bytes(10, 100) == -1


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(wv=None), NULL), (dict(meta=None), NULL), (dict(packed=None), NULL), (dict(K=100), SHAPE),
    (dict(ldwv=16), SHAPE), (dict(ldwm=8), SHAPE), (dict(ldwv=40), ALIGN), (dict(ldwm=24), ALIGN),
    (dict(packed=ODD), ALIGN), (dict(wv=ODD), ALIGN), (dict(N=0), SHAPE),
])
def test_pack_w4_validation(kw, code):
    a = dict(wv=P, ldwv=32, meta=P2, ldwm=16, N=8, K=128, packed=P3)
    a.update(kw)
    assert sg.lib().sg_sparse24_pack_w4(a["wv"], a["ldwv"], a["meta"], a["ldwm"], a["N"], a["K"], a["packed"],
                                        None) == code


def w4a16_packed(**kw):
    a = dict(M=16, N=256, K=256, x=P, ldx=256, w=P2, sw=P3, swn=2, swk=1, bias=None, y=P, ydt=1, ldy=256, form=0)
    a.update(kw)
    return sg.lib().sg_w4a16_sparse24_gemm_groupwise_packed(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["w"],
                                                            a["sw"], a["swn"], a["swk"], a["bias"], a["y"],
                                                            a["ydt"], a["ldy"], a["form"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(sw=None), NULL), (dict(y=None), NULL),
    (dict(ydt=2), UNSUP), (dict(form=2), UNSUP), (dict(K=200), SHAPE), (dict(ldx=128), SHAPE),
    (dict(ldy=100), SHAPE), (dict(swn=-1), SHAPE), (dict(M=0), SHAPE), (dict(N=0), SHAPE),
    (dict(M=65535 * 16 + 1), SHAPE), (dict(K=128 * 174763, ldx=128 * 174763), SHAPE),
    (dict(x=ODD), ALIGN), (dict(ldx=260), ALIGN), (dict(w=ODD), ALIGN),
])
def test_w4a16_packed_validation(kw, code):
    assert w4a16_packed(**kw) == code


def w4a16(**kw):
    a = dict(M=16, N=256, K=256, x=P, ldx=256, w=P2, ldw=64, meta=P3, ldm=32, sw=P3, swn=2, swk=1, bias=None,
             y=P, ydt=1, ldy=256, form=0)
    a.update(kw)
    return sg.lib().sg_w4a16_sparse24_gemm_groupwise(a["M"], a["N"], a["K"], a["x"], a["ldx"], a["w"], a["ldw"],
                                                     a["meta"], a["ldm"], a["sw"], a["swn"], a["swk"], a["bias"],
                                                     a["y"], a["ydt"], a["ldy"], a["form"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(meta=None), NULL), (dict(sw=None), NULL),
    (dict(ydt=2), UNSUP), (dict(form=2), UNSUP), (dict(K=200), SHAPE), (dict(ldw=32), SHAPE), (dict(ldm=16), SHAPE),
    (dict(swn=-1), SHAPE), (dict(ldw=72), ALIGN), (dict(w=ODD), ALIGN), (dict(M=0), SHAPE), (dict(N=0), SHAPE),
])
def test_w4a16_validation(kw, code):
    assert w4a16(**kw) == code


def quant_x(**kw):
    a = dict(M=16, N=256, K=256, x=P, xdt=0, ldx=256, w=P2, sw=P3, swn=2, swk=1, gn=128, y=P, ydt=1, ldy=256,
             form=0)
    a.update(kw)
    return sg.lib().sg_fp8_sparse24_gemm_packed_quant_x(a["M"], a["N"], a["K"], a["x"], a["xdt"], a["ldx"], a["w"],
                                                        a["sw"], a["swn"], a["swk"], a["gn"], a["y"], a["ydt"],
                                                        a["ldy"], a["form"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(sw=None), NULL), (dict(y=None), NULL),
    (dict(xdt=2), UNSUP), (dict(xdt=3), UNSUP), (dict(gn=1), UNSUP), (dict(ydt=2), UNSUP), (dict(form=2), UNSUP),
    (dict(M=65), UNSUP), (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(K=0), SHAPE), (dict(K=200), SHAPE),
    (dict(ldx=128), SHAPE), (dict(ldy=100), SHAPE), (dict(form=1, ldy=8), SHAPE), (dict(swn=-1), SHAPE),
    (dict(ldx=1 << 26, K=128), SHAPE),
    (dict(x=ODD), ALIGN), (dict(ldx=258), ALIGN), (dict(xdt=1, ldx=260), ALIGN), (dict(w=ODD), ALIGN),
    (dict(y=ctypes.c_void_p(0x100001)), ALIGN),
])
def test_quant_x_gemm_validation(kw, code):
    assert quant_x(**kw) == code
