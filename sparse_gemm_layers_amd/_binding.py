"""ctypes binding of libsg.so.  Argument marshalling only.

Scale tensors are 2-D views [row_blocks, k_blocks] with arbitrary strides; by
default they are allocated "M-major" (contiguous along rows, one column per K
block), the layout CUTLASS PR #2095 ("Improvements for: Groupwise scaling
along M for FP8 gemm", PR description) moved to.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SG_LIBRARY selects another build of the same library (the host-sanitizer
# build of the CPU-only ABI tests); by default the in-tree libsg.so.
LIB_PATH = os.environ.get("SG_LIBRARY") or os.path.join(_HERE, "libsg.so")

SG_F32, SG_BF16, SG_E4M3, SG_I8 = 0, 1, 2, 3
SG_OUT_Y, SG_OUT_YT = 0, 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_ptr = ctypes.c_void_p

_SIGS = {
    "sg_status_str": ([_int], ctypes.c_char_p),
    "sg_abi_version": ([], _int),
    "sg_fp8_quant_groupwise": ([_ptr, _int, _i64, _i64, _i64, _int, _int, _ptr, _i64, _ptr, _i64, _i64, _ptr], _int),
    "sg_int4_quant_groupwise": ([_ptr, _int, _i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _i64, _ptr], _int),
    "sg_sparse24_prune_compress": ([_ptr, _int, _i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr], _int),
    "sg_fp8_gemm_groupwise": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _i64,
                               _int, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_fp8_sparse24_gemm_groupwise": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _int, _ptr, _i64, _ptr,
                                        _i64, _ptr, _i64, _i64, _int, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_sparse24_packed_bytes": ([_i64, _i64], _i64),
    "sg_sparse24_pack_gfx950": ([_ptr, _i64, _ptr, _i64, _i64, _i64, _ptr, _ptr], _int),
    "sg_sparse24_w4_packed_bytes": ([_i64, _i64], _i64),
    "sg_sparse24_pack_w4": ([_ptr, _i64, _ptr, _i64, _i64, _i64, _ptr, _ptr], _int),
    "sg_fp8_sparse24_gemm_groupwise_packed": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _int, _ptr, _ptr,
                                               _i64, _i64, _int, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_fp8_sparse24_gemm_packed_quant_x": ([_i64, _i64, _i64, _ptr, _int, _i64, _ptr, _ptr, _i64, _i64, _int,
                                             _ptr, _int, _i64, _int, _ptr], _int),
    "sg_mixed_gemm_add": ([_i64, _i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64,
                           _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr], _int),
    "sg_int8_quant_groupwise": ([_ptr, _int, _i64, _i64, _i64, _int, _int, _ptr, _i64, _ptr, _i64, _i64, _ptr], _int),
    "sg_int8_sparse24_gemm_groupwise": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _int, _ptr, _i64, _ptr,
                                         _i64, _ptr, _i64, _i64, _int, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_int8_sparse24_gemm_groupwise_packed": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _int, _ptr, _ptr,
                                                _i64, _i64, _int, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_fp8_gemm_groupwise_batched": ([_i64, _i64, _i64, _i64, _ptr, _i64, _i64, _ptr, _i64, _i64, _i64, _int,
                                       _ptr, _i64, _i64, _ptr, _i64, _i64, _i64, _int, _ptr, _i64, _ptr, _int,
                                       _i64, _i64, _int, _ptr], _int),
    "sg_fp8_sparse24_gemm_groupwise_batched": ([_i64, _i64, _i64, _i64, _ptr, _i64, _i64, _ptr, _i64, _i64, _i64,
                                                _int, _ptr, _i64, _i64, _ptr, _i64, _i64, _ptr, _i64, _i64, _i64,
                                                _int, _ptr, _i64, _ptr, _int, _i64, _i64, _int, _ptr], _int),
    "sg_fp8_sparse24_gemm_groupwise_packed_batched": ([_i64, _i64, _i64, _i64, _ptr, _i64, _i64, _ptr, _i64, _i64,
                                                       _i64, _int, _ptr, _i64, _ptr, _i64, _i64, _i64, _int, _ptr,
                                                       _i64, _ptr, _int, _i64, _i64, _int, _ptr], _int),
    "sg_fp8_sparse24_gemm_groupwise_packed_grouped": ([_i64, _ptr, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _ptr,
                                                       _i64, _ptr, _i64, _i64, _i64, _int, _ptr, _i64, _ptr, _int,
                                                       _i64, _int, _ptr], _int),
    "sg_w8a16_sparse24_gemm_groupwise": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _ptr, _i64,
                                          _i64, _int, _ptr, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_w8a16_sparse24_gemm_groupwise_packed": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _int, _ptr, _i64, _i64, _int,
                                                 _ptr, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_w4a16_sparse24_gemm_groupwise_packed": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _ptr, _i64, _i64, _ptr, _ptr,
                                                 _int, _i64, _int, _ptr], _int),
    "sg_w4a16_sparse24_gemm_groupwise": ([_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _i64,
                                          _ptr, _ptr, _int, _i64, _int, _ptr], _int),
    "sg_probe_matrix_ops": ([_int, _int], _i64),
    "sg_probe_matrix_rate": ([_int, _int, _ptr, _ptr, _ptr], _int),
    "sg_probe_stream_read": ([_ptr, _i64, _int, _ptr, _ptr], _int),
}

_lib = None


class SgError(RuntimeError):
    pass


def lib():
    """The loaded libsg.so (ctypes.CDLL) with every entry point typed."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_gemm_layers_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise SgError(f"{what}: {lib().sg_status_str(status).decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _gpu2d(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SgError(f"{name} must be a GPU tensor")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise SgError(f"{name} must be 2-D with unit column stride")
    return t


def _dtype_code(t, name):
    if t.dtype == torch.float32:
        return SG_F32
    if t.dtype == torch.bfloat16:
        return SG_BF16
    raise SgError(f"{name}: dtype {t.dtype} not supported (float32 or bfloat16)")


_NAMES = {torch.float32: "float32", torch.bfloat16: "bfloat16", torch.uint8: "uint8", torch.int8: "int8",
          torch.int16: "int16", torch.uint16: "uint16"}


def _want(t, name, dtypes, shape, device):
    """t must be a GPU tensor on `device` with one of `dtypes` and exactly
    `shape` (None entries: any size)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SgError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise SgError(f"{name} is on {t.device}, the operands on {device}")
    if t.dtype not in dtypes:
        raise SgError(f"{name}: dtype {t.dtype} not supported ({' or '.join(_NAMES[d] for d in dtypes)})")
    if t.dim() != len(shape) or any(w is not None and w != h for w, h in zip(shape, t.shape)):
        want = ", ".join("*" if w is None else str(w) for w in shape)
        raise SgError(f"{name} must have shape [{want}], got {list(t.shape)}")
    return t


def _want_scales(s, name, rows, kb, device, batch=None):
    """fp32 GPU scales [rows, kb] (any strides), or [L, rows, kb] / a shared
    [rows, kb] when batch = L; rows may be larger than needed."""
    if not isinstance(s, torch.Tensor) or not s.is_cuda or s.dtype != torch.float32:
        raise SgError(f"{name} must be a float32 GPU tensor")
    if s.device != device:
        raise SgError(f"{name} is on {s.device}, the operands on {device}")
    if batch is not None and s.dim() == 3:
        if s.shape[0] not in (1, batch):
            raise SgError(f"{name} holds {s.shape[0]} problems, not {batch}")
        s2 = s.shape[1:]
    elif s.dim() == 2:
        s2 = s.shape
    else:
        raise SgError(f"{name} must be 2-D [rows, K/128]" + (" or 3-D [L, rows, K/128]" if batch else ""))
    if s2[0] < rows or s2[1] < kb:
        raise SgError(f"{name} must cover [{rows}, {kb}] scales, got {list(s.shape)}")
    return s


def _positive(**sizes):
    for k, v in sizes.items():
        if v <= 0:
            raise SgError(f"{k} must be at least 1, got {v}")


_CODES = (torch.uint8,)
_I8 = (torch.int8,)
_FB = (torch.float32, torch.bfloat16)


def _row_stride(t):
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _scales(rows, cols, device):
    """Empty fp32 scale view [rows, cols] stored M-major (contiguous along rows)."""
    return torch.empty((cols, rows), dtype=torch.float32, device=device).t()


def fp8_quant_groupwise(x, gr: int = 1, gc: int = 128, q=None, s=None):
    """x [rows, cols] float32/bfloat16 -> (codes uint8 [rows, cols], scales fp32
    [ceil(rows/gr), cols/gc]).  One scale per gr x gc block: amax / 448."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    _positive(rows=rows, cols=cols, gr=gr, gc=gc)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = _scales(-(-rows // gr), cols // gc, x.device)
    _gpu2d(_want(q, "q", _CODES, (rows, cols), x.device), "q")
    _want_scales(s, "s", -(-rows // gr), cols // gc, x.device)
    st = lib().sg_fp8_quant_groupwise(_p(x), _dtype_code(x, "x"), rows, cols, _row_stride(x), gr, gc,
                                      _p(q), _row_stride(q), _p(s), s.stride(0), s.stride(1), _stream(x))
    _check(st, "sg_fp8_quant_groupwise")
    return q, s


def int8_quant_groupwise(x, gr: int = 1, gc: int = 128, q=None, s=None):
    """x [rows, cols] float32/bfloat16 -> (codes int8 [rows, cols], scales fp32
    [ceil(rows/gr), cols/gc]).  One scale per gr x gc block: amax / 127."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    _positive(rows=rows, cols=cols, gr=gr, gc=gc)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if s is None:
        s = _scales(-(-rows // gr), cols // gc, x.device)
    _gpu2d(_want(q, "q", _I8, (rows, cols), x.device), "q")
    _want_scales(s, "s", -(-rows // gr), cols // gc, x.device)
    st = lib().sg_int8_quant_groupwise(_p(x), _dtype_code(x, "x"), rows, cols, _row_stride(x), gr, gc,
                                       _p(q), _row_stride(q), _p(s), s.stride(0), s.stride(1), _stream(x))
    _check(st, "sg_int8_quant_groupwise")
    return q, s


def int4_quant_groupwise(x, gc: int = 128, q=None, s=None):
    """x [rows, cols] -> (packed int4 uint8 [rows, cols/2], scales fp32 [rows, cols/gc]); gc 128 or 64."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    _positive(rows=rows, cols=cols, gc=gc)
    if q is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = _scales(rows, cols // gc, x.device)
    _gpu2d(_want(q, "q", _CODES, (rows, cols // 2), x.device), "q")
    _want_scales(s, "s", rows, cols // gc, x.device)
    st = lib().sg_int4_quant_groupwise(_p(x), _dtype_code(x, "x"), rows, cols, _row_stride(x), gc, _p(q),
                                       _row_stride(q), _p(s), s.stride(0), s.stride(1), _stream(x))
    _check(st, "sg_int4_quant_groupwise")
    return q, s


def sparse24_prune_compress(w, vals=None, meta=None):
    """w [rows, k] float32, bfloat16 or uint8 (e4m3 codes) -> (values [rows, k/2]
    same dtype, metadata uint8 [rows, k/8])."""
    _gpu2d(w, "w")
    rows, k = w.shape
    _positive(rows=rows, k=k)
    dt = SG_E4M3 if w.dtype == torch.uint8 else _dtype_code(w, "w")
    if vals is None:
        vals = torch.empty((rows, k // 2), dtype=w.dtype, device=w.device)
    if meta is None:
        meta = torch.empty((rows, k // 8), dtype=torch.uint8, device=w.device)
    _gpu2d(_want(vals, "vals", (w.dtype,), (rows, k // 2), w.device), "vals")
    _gpu2d(_want(meta, "meta", _CODES, (rows, k // 8), w.device), "meta")
    st = lib().sg_sparse24_prune_compress(_p(w), dt, rows, k, _row_stride(w), _p(vals),
                                          _row_stride(vals), _p(meta), _row_stride(meta), _stream(w))
    _check(st, "sg_sparse24_prune_compress")
    return vals, meta


def _out(y, M, N, out_dtype, form, device):
    if form not in ("y", "yt", SG_OUT_Y, SG_OUT_YT):
        raise SgError(f"form must be 'y' or 'yt', got {form!r}")
    yt = form in ("yt", SG_OUT_YT)
    if y is None:
        y = torch.empty((N, M) if yt else (M, N), dtype=out_dtype, device=device)
    _gpu2d(_want(y, "y", _FB, (N, M) if yt else (M, N), device), "y")
    return y, (SG_OUT_YT if yt else SG_OUT_Y), _dtype_code(y, "y")


def _gemm_operands(xq, x_dtypes, M, N, K, sx, gran_m, sw, gran_n):
    """Shape and dtype checks shared by the single-problem GEMMs."""
    _positive(M=M, N=N, K=K)
    if K % 128:
        raise SgError(f"K must be a multiple of 128, got {K}")
    _want(xq, "xq", x_dtypes, (M, K), xq.device)
    if gran_m not in (1, 128) or gran_n not in (1, 128):
        raise SgError("gran_m and gran_n must be 1 or 128")
    _want_scales(sx, "sx", -(-M // gran_m), K // 128, xq.device)
    if sw is not None:
        _want_scales(sw, "sw", -(-N // gran_n), K // 128, xq.device)


def fp8_gemm_groupwise(xq, sx, wq, sw, gran_m: int = 1, gran_n: int = 128, out_dtype=torch.bfloat16,
                       form: str = "y", y=None):
    """Y = X . W^T with groupwise scales.  xq uint8 [M, K], sx fp32 [ceil(M/gran_m), K/128],
    wq uint8 [N, K], sw fp32 [ceil(N/gran_n), K/128].  form "y" -> Y [M, N], "yt" -> Y^T [N, M]."""
    _gpu2d(xq, "xq")
    _gpu2d(wq, "wq")
    M, K = xq.shape
    N = wq.shape[0]
    _gemm_operands(xq, _CODES, M, N, K, sx, gran_m, sw, gran_n)
    _want(wq, "wq", _CODES, (N, K), xq.device)
    y, f, ydt = _out(y, M, N, out_dtype, form, xq.device)
    st = lib().sg_fp8_gemm_groupwise(M, N, K, _p(xq), _row_stride(xq), _p(sx), sx.stride(0), sx.stride(1),
                                     gran_m, _p(wq), _row_stride(wq), _p(sw), sw.stride(0), sw.stride(1),
                                     gran_n, _p(y), ydt, _row_stride(y), f, _stream(xq))
    _check(st, "sg_fp8_gemm_groupwise")
    return y


def fp8_sparse24_gemm_groupwise(xq, sx, wv, wmeta, sw, gran_m: int = 1, gran_n: int = 128,
                                out_dtype=torch.bfloat16, form: str = "y", y=None):
    """The same GEMM with W as 2:4-compressed codes wv uint8 [N, K/2] and metadata
    wmeta uint8 [N, K/8]."""
    _gpu2d(xq, "xq")
    _gpu2d(wv, "wv")
    _gpu2d(wmeta, "wmeta")
    M, K = xq.shape
    N = wv.shape[0]
    _gemm_operands(xq, _CODES, M, N, K, sx, gran_m, sw, gran_n)
    _want(wv, "wv", _CODES, (N, K // 2), xq.device)
    _want(wmeta, "wmeta", _CODES, (N, K // 8), xq.device)
    y, f, ydt = _out(y, M, N, out_dtype, form, xq.device)
    st = lib().sg_fp8_sparse24_gemm_groupwise(M, N, K, _p(xq), _row_stride(xq), _p(sx), sx.stride(0),
                                              sx.stride(1), gran_m, _p(wv), _row_stride(wv), _p(wmeta),
                                              _row_stride(wmeta), _p(sw), sw.stride(0), sw.stride(1), gran_n,
                                              _p(y), ydt, _row_stride(y), f, _stream(xq))
    _check(st, "sg_fp8_sparse24_gemm_groupwise")
    return y


def k_constant_scales(s, rows: int, k: int):
    """A [rows, K/128] view of rowwise scales s [rows] (or tensorwise s [1]) that
    repeats them over every K block (K-block stride 0), the layout the GEMM entry
    points take for scales constant along K (pass gran 1)."""
    if not isinstance(s, torch.Tensor) or s.dim() != 1 or s.shape[0] not in (1, rows):
        raise SgError("scales must be 1-D with one entry per row, or one entry")
    return s[:, None].expand(rows, k // 128)


def _gpu3d(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SgError(f"{name} must be a GPU tensor")
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise SgError(f"{name} must be 3-D [L, rows, cols] with unit column stride")
    return t


def _bstride(t):
    """Batch stride of a 3-D operand, 0 for a 2-D operand shared by every problem."""
    return 0 if t.dim() == 2 or t.shape[0] == 1 else t.stride(0)


def _mat(t, name):
    """(rows, row stride) of a [L, rows, cols] or shared [rows, cols] operand."""
    if t.dim() == 2:
        _gpu2d(t, name)
        return t.shape[0], _row_stride(t)
    _gpu3d(t, name)
    return t.shape[1], (t.stride(1) if t.shape[1] > 1 else max(t.shape[2], 1))


def _sc(t):
    """(row stride, K-block stride, batch stride) of [L, rows, KB] or shared [rows, KB] scales."""
    if t.dim() == 2:
        return t.stride(0), t.stride(1), 0
    return t.stride(1), t.stride(2), _bstride(t)


def _out_batched(y, L, M, N, out_dtype, form, device):
    if form not in ("y", "yt", SG_OUT_Y, SG_OUT_YT):
        raise SgError(f"form must be 'y' or 'yt', got {form!r}")
    yt = form in ("yt", SG_OUT_YT)
    if y is None:
        y = torch.empty((L, N, M) if yt else (L, M, N), dtype=out_dtype, device=device)
    _gpu3d(_want(y, "y", _FB, (L, N, M) if yt else (L, M, N), device), "y")
    return y, (SG_OUT_YT if yt else SG_OUT_Y), _dtype_code(y, "y")


def _want_shared(t, name, dtypes, L, rows, cols, device):
    """[L, rows, cols] (one per problem; L may be 1) or [rows, cols] (shared)."""
    if isinstance(t, torch.Tensor) and t.dim() == 3:
        _want(t, name, dtypes, (None, rows, cols), device)
        if t.shape[0] not in (1, L):
            raise SgError(f"{name} holds {t.shape[0]} problems, not {L}")
        return t
    return _want(t, name, dtypes, (rows, cols), device)


def _batched_operands(xq, x_dtypes, sx, gran_m, sw, gran_n):
    _gpu3d(xq, "xq")
    L, M, K = xq.shape
    _positive(L=L, M=M, K=K)
    if K % 128:
        raise SgError(f"K must be a multiple of 128, got {K}")
    _want(xq, "xq", x_dtypes, (L, M, K), xq.device)
    if gran_m not in (1, 128) or gran_n not in (1, 128):
        raise SgError("gran_m and gran_n must be 1 or 128")
    _want_scales(sx, "sx", -(-M // gran_m), K // 128, xq.device, batch=L)
    return L, M, K


def _bias(bias, N):
    """(pointer, batch stride) of an optional fp32 bias [L, N] or shared [N]."""
    if bias is None:
        return None, 0
    if not isinstance(bias, torch.Tensor) or not bias.is_cuda or bias.dtype != torch.float32 \
            or bias.dim() not in (1, 2) or bias.shape[-1] != N or (N > 1 and bias.stride(-1) != 1):
        raise SgError("bias must be a float32 GPU tensor [L, N] or [N]")
    return _p(bias), (0 if bias.dim() == 1 or bias.shape[0] == 1 else bias.stride(0))


def fp8_gemm_groupwise_batched(xq, sx, wq, sw, gran_m: int = 1, gran_n: int = 128, out_dtype=torch.bfloat16,
                               form: str = "y", y=None, bias=None):
    """L independent GEMMs: xq uint8 [L, M, K], sx [L, ceil(M/gran_m), K/128];
    wq uint8 [L, N, K] and sw [L, ., K/128], or 2-D to share one weight.  Returns
    y [L, M, N] ("y") or [L, N, M] ("yt")."""
    L, M, K = _batched_operands(xq, _CODES, sx, gran_m, sw, gran_n)
    N, ldw = _mat(wq, "wq")
    _positive(N=N)
    _want_shared(wq, "wq", _CODES, L, N, K, xq.device)
    _want_scales(sw, "sw", -(-N // gran_n), K // 128, xq.device, batch=L)
    y, f, ydt = _out_batched(y, L, M, N, out_dtype, form, xq.device)
    sxm, sxk, sxb = _sc(sx)
    swn, swk, swb = _sc(sw)
    bp, bb = _bias(bias, N)
    st = lib().sg_fp8_gemm_groupwise_batched(L, M, N, K, _p(xq), _mat(xq, "xq")[1], _bstride(xq), _p(sx), sxm, sxk,
                                             sxb, gran_m, _p(wq), ldw, _bstride(wq), _p(sw), swn, swk, swb, gran_n,
                                             bp, bb, _p(y), ydt, _mat(y, "y")[1], _bstride(y), f, _stream(xq))
    _check(st, "sg_fp8_gemm_groupwise_batched")
    return y


def fp8_sparse24_gemm_groupwise_batched(xq, sx, wv, wmeta, sw, gran_m: int = 1, gran_n: int = 128,
                                        out_dtype=torch.bfloat16, form: str = "y", y=None, bias=None):
    """Batched 2:4 GEMM: wv [L, N, K/2] and wmeta [L, N, K/8] (or 2-D, shared)."""
    L, M, K = _batched_operands(xq, _CODES, sx, gran_m, sw, gran_n)
    N, ldwv = _mat(wv, "wv")
    _, ldwm = _mat(wmeta, "wmeta")
    _positive(N=N)
    _want_shared(wv, "wv", _CODES, L, N, K // 2, xq.device)
    _want_shared(wmeta, "wmeta", _CODES, L, N, K // 8, xq.device)
    _want_scales(sw, "sw", -(-N // gran_n), K // 128, xq.device, batch=L)
    y, f, ydt = _out_batched(y, L, M, N, out_dtype, form, xq.device)
    sxm, sxk, sxb = _sc(sx)
    swn, swk, swb = _sc(sw)
    bp, bb = _bias(bias, N)
    st = lib().sg_fp8_sparse24_gemm_groupwise_batched(
        L, M, N, K, _p(xq), _mat(xq, "xq")[1], _bstride(xq), _p(sx), sxm, sxk, sxb, gran_m, _p(wv), ldwv,
        _bstride(wv), _p(wmeta), ldwm, _bstride(wmeta), _p(sw), swn, swk, swb, gran_n, bp, bb, _p(y), ydt,
        _mat(y, "y")[1], _bstride(y), f, _stream(xq))
    _check(st, "sg_fp8_sparse24_gemm_groupwise_batched")
    return y


def fp8_sparse24_gemm_groupwise_packed_batched(xq, sx, wpacked, n: int, sw, gran_m: int = 1, gran_n: int = 128,
                                               out_dtype=torch.bfloat16, form: str = "y", y=None, bias=None):
    """Batched 2:4 GEMM with packed weights: wpacked uint8 [L, bytes] (one packed
    weight per problem) or 1-D (shared)."""
    L, M, K = _batched_operands(xq, _CODES, sx, gran_m, sw, gran_n)
    _positive(N=n)
    _want_packed(wpacked, n, K, xq.device, batch=L)
    _want_scales(sw, "sw", -(-n // gran_n), K // 128, xq.device, batch=L)
    wpb = 0 if wpacked.dim() == 1 or wpacked.shape[0] == 1 else wpacked.stride(0)
    y, f, ydt = _out_batched(y, L, M, n, out_dtype, form, xq.device)
    sxm, sxk, sxb = _sc(sx)
    swn, swk, swb = _sc(sw)
    bp, bb = _bias(bias, n)
    st = lib().sg_fp8_sparse24_gemm_groupwise_packed_batched(
        L, M, n, K, _p(xq), _mat(xq, "xq")[1], _bstride(xq), _p(sx), sxm, sxk, sxb, gran_m, _p(wpacked), wpb,
        _p(sw), swn, swk, swb, gran_n, bp, bb, _p(y), ydt, _mat(y, "y")[1], _bstride(y), f, _stream(xq))
    _check(st, "sg_fp8_sparse24_gemm_groupwise_packed_batched")
    return y


def fp8_sparse24_gemm_groupwise_packed_grouped(xq, sx, m_sizes, wpacked, n: int, sw, gran_n: int = 128,
                                               out_dtype=torch.bfloat16, form: str = "y", y=None, bias=None):
    """Grouped 2:4 GEMM: xq uint8 [sum(m_sizes), K] with the groups' rows one
    after another, sx [sum(m_sizes), K/128] (one scale row per X row), one packed
    weight per group wpacked [G, bytes] and its scales sw [G, ., K/128] (or 2-D /
    1-D to share); returns y [sum, N] ("y") or [N, sum] ("yt")."""
    sizes = [int(v) for v in m_sizes]
    if not isinstance(xq, torch.Tensor) or not xq.is_cuda or xq.dim() != 2 or sum(sizes) != xq.shape[0]:
        raise SgError("xq must be a 2-D GPU tensor whose rows m_sizes sums to")
    if any(v < 0 for v in sizes):
        raise SgError("m_sizes must be non-negative")
    _gpu2d(xq, "xq")
    M, K = xq.shape
    G = len(sizes)
    _gemm_operands(xq, _CODES, M, n, K, sx, 1, None, gran_n)
    _want_scales(sw, "sw", -(-n // gran_n), K // 128, xq.device, batch=G)
    _want_packed(wpacked, n, K, xq.device, batch=G)
    wpb = 0 if wpacked.dim() == 1 or wpacked.shape[0] == 1 else wpacked.stride(0)
    y, f, ydt = _out(y, M, n, out_dtype, form, xq.device)
    swn, swk, swb = _sc(sw)
    bp, bb = _bias(bias, n)
    arr = (ctypes.c_int64 * max(G, 1))(*sizes)
    st = lib().sg_fp8_sparse24_gemm_groupwise_packed_grouped(
        G, ctypes.cast(arr, ctypes.c_void_p), n, K, _p(xq), _row_stride(xq), _p(sx), sx.stride(0), sx.stride(1),
        _p(wpacked), wpb, _p(sw), swn, swk, swb, gran_n, bp, bb, _p(y), ydt, _row_stride(y), f, _stream(xq))
    _check(st, "sg_fp8_sparse24_gemm_groupwise_packed_grouped")
    return y


def w8a16_sparse24_gemm_groupwise(x, wv, wmeta, sw, gran_n: int = 128, out_dtype=torch.bfloat16, form: str = "y",
                                   y=None, bias=None):
    """Weight-only 2:4 GEMM: x bfloat16 [M, K] (not quantised) times 2:4 codes
    wv [N, K/2] (uint8: e4m3, int8: int8) with metadata wmeta [N, K/8] and W
    scales sw [ceil(N/gran_n), K/128]."""
    _gpu2d(x, "x")
    _gpu2d(wv, "wv")
    _gpu2d(wmeta, "wmeta")
    if x.dtype != torch.bfloat16:
        raise SgError("x must be bfloat16")
    if wv.dtype == torch.uint8:
        wdt = SG_E4M3
    elif wv.dtype == torch.int8:
        wdt = SG_I8
    else:
        raise SgError("wv must be uint8 (e4m3 codes) or int8")
    M, K = x.shape
    N = wv.shape[0]
    _positive(M=M, N=N, K=K)
    if K % 128 or gran_n not in (1, 128):
        raise SgError("K must be a multiple of 128 and gran_n 1 or 128")
    _want(wv, "wv", (wv.dtype,), (N, K // 2), x.device)
    _want(wmeta, "wmeta", _CODES, (N, K // 8), x.device)
    _want_scales(sw, "sw", -(-N // gran_n), K // 128, x.device)
    y, f, ydt = _out(y, M, N, out_dtype, form, x.device)
    bp, _ = _bias(bias, N)
    st = lib().sg_w8a16_sparse24_gemm_groupwise(M, N, K, _p(x), _row_stride(x), _p(wv), _row_stride(wv), _p(wmeta),
                                                _row_stride(wmeta), wdt, _p(sw), sw.stride(0), sw.stride(1), gran_n,
                                                bp, _p(y), ydt, _row_stride(y), f, _stream(x))
    _check(st, "sg_w8a16_sparse24_gemm_groupwise")
    return y


def w8a16_sparse24_gemm_groupwise_packed(x, wpacked, n: int, sw, gran_n: int = 128, int8: bool = False,
                                         out_dtype=torch.bfloat16, form: str = "y", y=None, bias=None):
    """The weight-only 2:4 GEMM with the weight in the gfx950 packed form
    (sparse24_pack_gfx950 of the [N, K/2] codes and [N, K/8] metadata): x
    bfloat16 [M, K]; wpacked uint8 [bytes]; int8 names the packed code type
    (e4m3 otherwise).  Equals w8a16_sparse24_gemm_groupwise on the unpacked
    weight bit for bit."""
    _gpu2d(x, "x")
    if x.dtype != torch.bfloat16:
        raise SgError("x must be bfloat16")
    M, K = x.shape
    _positive(M=M, N=n, K=K)
    if K % 128 or gran_n not in (1, 128):
        raise SgError("K must be a multiple of 128 and gran_n 1 or 128")
    _want(x, "x", (torch.bfloat16,), (M, K), x.device)
    _want_packed(wpacked, n, K, x.device)
    _want_scales(sw, "sw", -(-n // gran_n), K // 128, x.device)
    y, f, ydt = _out(y, M, n, out_dtype, form, x.device)
    bp, _ = _bias(bias, n)
    st = lib().sg_w8a16_sparse24_gemm_groupwise_packed(M, n, K, _p(x), _row_stride(x), _p(wpacked),
                                                       SG_I8 if int8 else SG_E4M3, _p(sw), sw.stride(0),
                                                       sw.stride(1), gran_n, bp, _p(y), ydt, _row_stride(y), f,
                                                       _stream(x))
    _check(st, "sg_w8a16_sparse24_gemm_groupwise_packed")
    return y


def w4a16_sparse24_gemm_groupwise(x, wv4, wmeta, sw, out_dtype=torch.bfloat16, form: str = "y", y=None,
                                   bias=None):
    """Weight-only 2:4 GEMM with int4 codes: x bfloat16 [M, K]; wv4 uint8 [N, K/4]
    (2:4-compressed values quantised with int4_quant_groupwise(gc=64)); wmeta
    uint8 [N, K/8]; sw fp32 [N, K/128]."""
    _gpu2d(x, "x")
    _gpu2d(wv4, "wv4")
    _gpu2d(wmeta, "wmeta")
    if x.dtype != torch.bfloat16 or wv4.dtype != torch.uint8:
        raise SgError("x must be bfloat16 and wv4 uint8")
    M, K = x.shape
    N = wv4.shape[0]
    _positive(M=M, N=N, K=K)
    if K % 128:
        raise SgError(f"K must be a multiple of 128, got {K}")
    _want(wv4, "wv4", _CODES, (N, K // 4), x.device)
    _want(wmeta, "wmeta", _CODES, (N, K // 8), x.device)
    _want_scales(sw, "sw", N, K // 128, x.device)
    y, f, ydt = _out(y, M, N, out_dtype, form, x.device)
    bp, _ = _bias(bias, N)
    st = lib().sg_w4a16_sparse24_gemm_groupwise(M, N, K, _p(x), _row_stride(x), _p(wv4), _row_stride(wv4), _p(wmeta),
                                                _row_stride(wmeta), _p(sw), sw.stride(0), sw.stride(1), bp, _p(y), ydt,
                                                _row_stride(y), f, _stream(x))
    _check(st, "sg_w4a16_sparse24_gemm_groupwise")
    return y


def sparse24_w4_packed_bytes(n: int, k: int) -> int:
    return int(lib().sg_sparse24_w4_packed_bytes(n, k))


def _want_w4_packed(wpacked, n, k, device):
    need = sparse24_w4_packed_bytes(n, k)
    if need < 0:
        raise SgError(f"no blocked int4 form for N = {n}, K = {k}")
    if not isinstance(wpacked, torch.Tensor) or not wpacked.is_cuda or wpacked.dtype != torch.uint8 \
            or wpacked.dim() != 1 or wpacked.shape[0] < need or wpacked.stride(0) != 1:
        raise SgError(f"wpacked must be a uint8 GPU tensor [bytes] of at least {need} bytes")
    if wpacked.device != device:
        raise SgError(f"wpacked is on {wpacked.device}, the operands on {device}")


def sparse24_pack_w4(wv4, wmeta, packed=None):
    """int4 2:4 codes wv4 uint8 [N, K/4] + metadata uint8 [N, K/8] -> the
    blocked form (uint8, sparse24_w4_packed_bytes(N, K) bytes) that
    w4a16_sparse24_gemm_groupwise_packed takes."""
    _gpu2d(wv4, "wv4")
    _gpu2d(wmeta, "wmeta")
    n, k = wv4.shape[0], wv4.shape[1] * 4
    nbytes = sparse24_w4_packed_bytes(n, k)
    if nbytes < 0:
        raise SgError("sparse24_pack_w4: N must be at least 1 and K a positive multiple of 128")
    _want(wv4, "wv4", (torch.uint8,), (n, k // 4), wv4.device)
    _want(wmeta, "wmeta", _CODES, (n, k // 8), wv4.device)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=wv4.device)
    _want_w4_packed(packed, n, k, wv4.device)
    st = lib().sg_sparse24_pack_w4(_p(wv4), _row_stride(wv4), _p(wmeta), _row_stride(wmeta), n, k, _p(packed),
                                   _stream(wv4))
    _check(st, "sg_sparse24_pack_w4")
    return packed


def w4a16_sparse24_gemm_groupwise_packed(x, wpacked, n: int, sw, out_dtype=torch.bfloat16, form: str = "y", y=None,
                                         bias=None):
    """The W4A16 GEMM with the weight in the blocked form of sparse24_pack_w4:
    x bfloat16 [M, K]; wpacked uint8 [bytes]; sw fp32 [N, K/128].  Equals
    w4a16_sparse24_gemm_groupwise on the unpacked weight bit for bit."""
    _gpu2d(x, "x")
    if x.dtype != torch.bfloat16:
        raise SgError("x must be bfloat16")
    M, K = x.shape
    _positive(M=M, N=n, K=K)
    if K % 128:
        raise SgError(f"K must be a multiple of 128, got {K}")
    _want_w4_packed(wpacked, n, K, x.device)
    _want_scales(sw, "sw", n, K // 128, x.device)
    y, f, ydt = _out(y, M, n, out_dtype, form, x.device)
    bp, _ = _bias(bias, n)
    st = lib().sg_w4a16_sparse24_gemm_groupwise_packed(M, n, K, _p(x), _row_stride(x), _p(wpacked), _p(sw),
                                                       sw.stride(0), sw.stride(1), bp, _p(y), ydt, _row_stride(y), f,
                                                       _stream(x))
    _check(st, "sg_w4a16_sparse24_gemm_groupwise_packed")
    return y


def sparse24_packed_bytes(n: int, k: int) -> int:
    return int(lib().sg_sparse24_packed_bytes(n, k))


def _want_packed(wpacked, n, k, device, batch=None):
    """A contiguous uint8 GPU buffer holding one packed weight ([bytes]), or one
    per problem ([L, bytes], when batch = L)."""
    need = sparse24_packed_bytes(n, k)
    if need < 0:
        raise SgError(f"no packed form for N = {n}, K = {k}")
    if not isinstance(wpacked, torch.Tensor) or not wpacked.is_cuda or wpacked.dtype != torch.uint8 \
            or wpacked.dim() not in ((1, 2) if batch else (1,)) or wpacked.shape[-1] < need \
            or wpacked.stride(-1) != 1:
        raise SgError(f"wpacked must be a uint8 GPU tensor [{'L, ' if batch else ''}bytes] of at least "
                      f"{need} bytes per packed weight")
    if wpacked.device != device:
        raise SgError(f"wpacked is on {wpacked.device}, the operands on {device}")
    if batch and wpacked.dim() == 2 and wpacked.shape[0] not in (1, batch):
        raise SgError(f"wpacked holds {wpacked.shape[0]} weights, not {batch}")
    return wpacked


def sparse24_pack_gfx950(wv, wmeta, packed=None):
    """Compressed codes wv uint8 [N, K/2] + metadata uint8 [N, K/8] -> the gfx950
    packed weight (uint8, sparse24_packed_bytes(N, K) bytes)."""
    _gpu2d(wv, "wv")
    _gpu2d(wmeta, "wmeta")
    n, k = wv.shape[0], wv.shape[1] * 2
    nbytes = sparse24_packed_bytes(n, k)
    if nbytes < 0:
        raise SgError("sparse24_pack_gfx950: N must be at least 1 and K a positive multiple of 128")
    _want(wv, "wv", (torch.uint8, torch.int8), (n, k // 2), wv.device)
    _want(wmeta, "wmeta", _CODES, (n, k // 8), wv.device)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=wv.device)
    _want_packed(packed, n, k, wv.device)
    st = lib().sg_sparse24_pack_gfx950(_p(wv), _row_stride(wv), _p(wmeta), _row_stride(wmeta), n, k, _p(packed),
                                       _stream(wv))
    _check(st, "sg_sparse24_pack_gfx950")
    return packed


def fp8_sparse24_gemm_groupwise_packed(xq, sx, wpacked, n: int, sw, gran_m: int = 1, gran_n: int = 128,
                                       out_dtype=torch.bfloat16, form: str = "y", y=None):
    """2:4-sparse FP8 GEMM with the weight in the gfx950 packed form (N rows)."""
    _gpu2d(xq, "xq")
    M, K = xq.shape
    _gemm_operands(xq, _CODES, M, n, K, sx, gran_m, sw, gran_n)
    _want_packed(wpacked, n, K, xq.device)
    y, f, ydt = _out(y, M, n, out_dtype, form, xq.device)
    st = lib().sg_fp8_sparse24_gemm_groupwise_packed(M, n, K, _p(xq), _row_stride(xq), _p(sx), sx.stride(0),
                                                     sx.stride(1), gran_m, _p(wpacked), _p(sw), sw.stride(0),
                                                     sw.stride(1), gran_n, _p(y), ydt, _row_stride(y), f,
                                                     _stream(xq))
    _check(st, "sg_fp8_sparse24_gemm_groupwise_packed")
    return y


def fp8_sparse24_gemm_packed_quant_x(x, wpacked, n: int, sw, gran_n: int = 128, out_dtype=torch.bfloat16,
                                     form: str = "y", y=None):
    """The packed 2:4 FP8 GEMM with X quantised inside it: x float32/bfloat16
    [M, K] (M <= 64), quantised per 1 x 128 block as fp8_quant_groupwise(x, 1,
    128) does; the result equals fp8_sparse24_gemm_groupwise_packed on those
    codes bit for bit."""
    _gpu2d(x, "x")
    M, K = x.shape
    _positive(M=M, N=n, K=K)
    if K % 128 or gran_n != 128:
        raise SgError("K must be a multiple of 128 and gran_n 128")
    _want(x, "x", _FB, (M, K), x.device)
    _want_packed(wpacked, n, K, x.device)
    _want_scales(sw, "sw", -(-n // 128), K // 128, x.device)
    y, f, ydt = _out(y, M, n, out_dtype, form, x.device)
    st = lib().sg_fp8_sparse24_gemm_packed_quant_x(M, n, K, _p(x), _dtype_code(x, "x"), _row_stride(x), _p(wpacked),
                                                   _p(sw), sw.stride(0), sw.stride(1), gran_n, _p(y), ydt,
                                                   _row_stride(y), f, _stream(x))
    _check(st, "sg_fp8_sparse24_gemm_packed_quant_x")
    return y


def int8_sparse24_gemm_groupwise(xq, sx, wv, wmeta, sw, gran_m: int = 1, gran_n: int = 128,
                                 out_dtype=torch.bfloat16, form: str = "y", y=None):
    """The 2:4-sparse GEMM with int8 codes: xq int8 [M, K], wv int8 [N, K/2],
    metadata wmeta uint8 [N, K/8]; scales as for the FP8 GEMM."""
    _gpu2d(xq, "xq")
    _gpu2d(wv, "wv")
    _gpu2d(wmeta, "wmeta")
    M, K = xq.shape
    N = wv.shape[0]
    _gemm_operands(xq, _I8, M, N, K, sx, gran_m, sw, gran_n)
    _want(wv, "wv", _I8, (N, K // 2), xq.device)
    _want(wmeta, "wmeta", _CODES, (N, K // 8), xq.device)
    y, f, ydt = _out(y, M, N, out_dtype, form, xq.device)
    st = lib().sg_int8_sparse24_gemm_groupwise(M, N, K, _p(xq), _row_stride(xq), _p(sx), sx.stride(0),
                                               sx.stride(1), gran_m, _p(wv), _row_stride(wv), _p(wmeta),
                                               _row_stride(wmeta), _p(sw), sw.stride(0), sw.stride(1), gran_n,
                                               _p(y), ydt, _row_stride(y), f, _stream(xq))
    _check(st, "sg_int8_sparse24_gemm_groupwise")
    return y


def int8_sparse24_gemm_groupwise_packed(xq, sx, wpacked, n: int, sw, gran_m: int = 1, gran_n: int = 128,
                                        out_dtype=torch.bfloat16, form: str = "y", y=None):
    """2:4-sparse int8 GEMM with the weight in the gfx950 packed form (N rows;
    sparse24_pack_gfx950 packs int8 codes as it packs e4m3 codes)."""
    _gpu2d(xq, "xq")
    M, K = xq.shape
    _gemm_operands(xq, _I8, M, n, K, sx, gran_m, sw, gran_n)
    _want_packed(wpacked, n, K, xq.device)
    y, f, ydt = _out(y, M, n, out_dtype, form, xq.device)
    st = lib().sg_int8_sparse24_gemm_groupwise_packed(M, n, K, _p(xq), _row_stride(xq), _p(sx), sx.stride(0),
                                                      sx.stride(1), gran_m, _p(wpacked), _p(sw), sw.stride(0),
                                                      sw.stride(1), gran_n, _p(y), ydt, _row_stride(y), f,
                                                      _stream(xq))
    _check(st, "sg_int8_sparse24_gemm_groupwise_packed")
    return y


def mixed_gemm_add(x1, sx1, w1, sw1, x2, w2, y=None):
    """Y = X1 . W1^T (int4, per-(row, 128) scales) + X2 . W2^T (bf16), bf16 out [M, N].
    x1 uint8 [M, K1/2], w1 uint8 [N, K1/2], x2 bf16 [M, K2], w2 bf16 [N, K2]."""
    _gpu2d(x1, "x1")
    _gpu2d(w1, "w1")
    M, K1 = x1.shape[0], x1.shape[1] * 2
    N = w1.shape[0]
    K2 = x2.shape[1] if x2 is not None else 0
    _positive(M=M, N=N, K1=K1)
    if K1 % 128:
        raise SgError(f"K1 must be a multiple of 128, got {K1}")
    dev = x1.device
    _want(x1, "x1", _CODES, (M, K1 // 2), dev)
    _want(w1, "w1", _CODES, (N, K1 // 2), dev)
    _want_scales(sx1, "sx1", M, K1 // 128, dev)
    _want_scales(sw1, "sw1", N, K1 // 128, dev)
    if K2:
        _gpu2d(x2, "x2")
        _gpu2d(w2, "w2")
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        _want(x2, "x2", bf, (M, K2), dev)
        _want(w2, "w2", bf, (N, K2), dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _gpu2d(_want(y, "y", (torch.bfloat16,), (M, N), dev), "y")
    st = lib().sg_mixed_gemm_add(M, N, K1, K2, _p(x1), _row_stride(x1), _p(sx1), sx1.stride(0), sx1.stride(1),
                                 _p(w1), _row_stride(w1), _p(sw1), sw1.stride(0), sw1.stride(1),
                                 _p(x2) if K2 else None, _row_stride(x2) if K2 else 0,
                                 _p(w2) if K2 else None, _row_stride(w2) if K2 else 0,
                                 _p(y), _row_stride(y), _stream(x1))
    _check(st, "sg_mixed_gemm_add")
    return y


# ------------------------------------------------------------ measurement helpers

PROBE_WORKGROUPS = 1024
PROBE_KINDS = {"mfma_fp8": 0, "smfmac_fp8": 1, "mfma_i8": 2, "smfmac_promoted": 3, "smfmac_rescaled": 4,
               "mfma_fp6": 5}


def probe_matrix_ops(kind, iters):
    """Dense-equivalent operations of one probe_matrix_rate launch."""
    return lib().sg_probe_matrix_ops(PROBE_KINDS[kind], iters)


def probe_matrix_rate(kind, iters, sink, clocks):
    """Enqueues one matrix-core rate probe (sg_probe.h).  sink: float32 device
    tensor of PROBE_WORKGROUPS * 512 elements; clocks: int64 device tensor of
    4 * PROBE_WORKGROUPS elements (shader clock and real-time counter at the
    start and end of each workgroup's first wave)."""
    for t, n, nm in ((sink, PROBE_WORKGROUPS * 512, "sink"), (clocks, 4 * PROBE_WORKGROUPS, "clocks")):
        if not t.is_cuda or t.numel() < n or not t.is_contiguous():
            raise SgError(f"{nm} must be a contiguous device tensor of at least {n} elements")
    st = lib().sg_probe_matrix_rate(PROBE_KINDS[kind], iters, _p(sink), _p(clocks), _stream(sink))
    _check(st, "sg_probe_matrix_rate")


def probe_stream_read(src, workgroups, sink):
    """Enqueues one streaming read of the whole of src (a contiguous device
    tensor, 16-byte aligned, a multiple of 16 bytes) by `workgroups`
    workgroups; sink: float32 device tensor of at least workgroups * 256."""
    if not src.is_cuda or not src.is_contiguous() or not sink.is_cuda or sink.numel() < workgroups * 256:
        raise SgError("src must be a contiguous device tensor and sink hold workgroups * 256 floats")
    st = lib().sg_probe_stream_read(_p(src), src.numel() * src.element_size(), workgroups, _p(sink), _stream(src))
    _check(st, "sg_probe_stream_read")
