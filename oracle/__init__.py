"""Plain, slow CPU oracle for the FP8 groupwise / 2:4-sparse GEMM layers.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``sparse_gemm_layers_amd``) never imports, calls or links anything here, and
this package imports nothing from the product path: the two share no code.

Everything is NumPy on the CPU.  Floating-point work is done in fp64 unless a
step is defined in fp32 (the quantisers' scale and divide, which the method
fixes to fp32 so that the codes are unique).  Each function cites the passage
of the source pages it follows; the pages are

* "[QST] CUTLASS support for fp8 sparse matrix (for W) multiplication for
  A*W=Y with GPU (SM90a/89) sparse tensor core" (CUTLASS issue #2029),
* "Improvements for: Groupwise scaling along M for FP8 gemm" (CUTLASS PR #2095),
* "[QST] How to implement a fused mixed precision matrix multiplication such as
  w4a4 + w16a16?" (CUTLASS issue #2058),
* "Introduce new W8A8-FP-CSR quantization API" (torchao PR #3258).

``pack.py`` additionally defines the library's own gfx950 packed weight layouts (the
FP8 / int8 one and the int4 blocked one: byte permutations of the compressed
values and metadata).

Parity status: every public function here is pinned by a ``-m "not gpu"`` test
against something other than itself (an independent codec, closed forms,
exact rational brute force, or identities the pages state).  None is
"parity unpinned".
"""

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode
from .bf16 import bf16_decode
from .quant import fp8_quant_groupwise, int4_quant_groupwise, int4_decode, int8_quant_groupwise
from .sparse24 import prune24, compress24, decompress24, prune_compress24
from .pack import pack24_gfx950, unpack24_gfx950, packed_bytes, pack24_w4_blocked, unpack24_w4_blocked, \
    w4_packed_bytes
from .gemm import (
    expand_scales,
    fp8_gemm_groupwise,
    fp8_sparse24_gemm_groupwise,
    int8_gemm_groupwise,
    int8_sparse24_gemm_groupwise,
    fp8_gemm_rowwise,
    fp8_sparse24_gemm_rowwise,
    int8_sparse24_gemm_rowwise,
    add_bias,
    w8a16_sparse24_gemm_groupwise,
    w4a16_sparse24_gemm_groupwise,
    mixed_gemm_add,
    within_tolerance,
)

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "bf16_decode",
    "fp8_quant_groupwise", "int4_quant_groupwise", "int4_decode", "int8_quant_groupwise",
    "prune24", "compress24", "decompress24", "prune_compress24",
    "pack24_gfx950", "unpack24_gfx950", "packed_bytes", "pack24_w4_blocked", "unpack24_w4_blocked",
    "w4_packed_bytes",
    "expand_scales", "fp8_gemm_groupwise", "fp8_sparse24_gemm_groupwise",
    "int8_gemm_groupwise", "int8_sparse24_gemm_groupwise", "fp8_gemm_rowwise",
    "fp8_sparse24_gemm_rowwise", "int8_sparse24_gemm_rowwise", "add_bias", "w8a16_sparse24_gemm_groupwise",
    "w4a16_sparse24_gemm_groupwise", "mixed_gemm_add", "within_tolerance",
]
