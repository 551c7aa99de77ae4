"""sparse_gemm_layers_amd: FP8 (e4m3) groupwise-scaled and 2:4-sparse
linear-layer GEMMs for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libsg.so`` (declared in
``include/sg.h``; the measurement helpers in ``include/sg_probe.h``).  The functions only marshal arguments: PyTorch supplies
device memory and the current HIP stream; every step runs in the library's
HIP kernels.  There is no CPU fallback: if ``libsg.so`` is missing or the
tensors are not on a GPU, the call raises.
"""

from ._binding import (
    SgError,
    lib,
    fp8_quant_groupwise,
    int4_quant_groupwise,
    sparse24_prune_compress,
    fp8_gemm_groupwise,
    fp8_sparse24_gemm_groupwise,
    sparse24_packed_bytes,
    sparse24_pack_gfx950,
    fp8_sparse24_gemm_groupwise_packed,
    fp8_sparse24_gemm_packed_quant_x,
    mixed_gemm_add,
    int8_quant_groupwise,
    int8_sparse24_gemm_groupwise,
    int8_sparse24_gemm_groupwise_packed,
    probe_matrix_ops,
    probe_matrix_rate,
    probe_stream_read,
    k_constant_scales,
    fp8_gemm_groupwise_batched,
    fp8_sparse24_gemm_groupwise_batched,
    fp8_sparse24_gemm_groupwise_packed_batched,
    fp8_sparse24_gemm_groupwise_packed_grouped,
    w8a16_sparse24_gemm_groupwise,
    w8a16_sparse24_gemm_groupwise_packed,
    w4a16_sparse24_gemm_groupwise,
    w4a16_sparse24_gemm_groupwise_packed,
    sparse24_w4_packed_bytes,
    sparse24_pack_w4,
)

__all__ = [
    "SgError", "lib", "fp8_quant_groupwise", "int4_quant_groupwise",
    "sparse24_prune_compress", "fp8_gemm_groupwise", "fp8_sparse24_gemm_groupwise",
    "sparse24_packed_bytes", "sparse24_pack_gfx950", "fp8_sparse24_gemm_groupwise_packed",
    "fp8_sparse24_gemm_packed_quant_x",
    "mixed_gemm_add", "int8_quant_groupwise", "int8_sparse24_gemm_groupwise",
    "int8_sparse24_gemm_groupwise_packed", "probe_matrix_ops", "probe_matrix_rate", "probe_stream_read", "k_constant_scales",
    "fp8_gemm_groupwise_batched", "fp8_sparse24_gemm_groupwise_batched",
    "fp8_sparse24_gemm_groupwise_packed_batched", "fp8_sparse24_gemm_groupwise_packed_grouped",
    "w8a16_sparse24_gemm_groupwise", "w8a16_sparse24_gemm_groupwise_packed", "w4a16_sparse24_gemm_groupwise",
    "w4a16_sparse24_gemm_groupwise_packed", "sparse24_w4_packed_bytes", "sparse24_pack_w4",
]
