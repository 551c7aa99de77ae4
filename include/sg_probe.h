/*
 * sg_probe.h -- measurement helpers of sparse_gemm_layers_amd (not part of the
 * method): the sustained matrix-core rate of the instructions the GEMM kernels
 * use, and the shader clock while they run.  The benchmark reports these next
 * to MI355X's published peaks, so that a roofline fraction can be read against
 * what the chip sustains as well as against its datasheet.
 *
 * Conventions as in sg.h: caller-owned device buffers, asynchronous on
 * `stream`, host-side validation before any HIP call.
 */
#ifndef SPARSE_GEMM_LAYERS_AMD_SG_PROBE_H
#define SPARSE_GEMM_LAYERS_AMD_SG_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "sg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of one probe launch (512 threads each, two waves per SIMD). */
#define SG_PROBE_WORKGROUPS 1024

typedef enum {
  SG_PROBE_MFMA_FP8 = 0,    /* v_mfma_f32_16x16x128_f8f6f4 with e4m3 operands (dense FP8)  */
  SG_PROBE_SMFMAC_FP8 = 1,  /* v_smfmac_f32_16x16x128_fp8_fp8 (2:4-sparse FP8)             */
  SG_PROBE_MFMA_I8 = 2,     /* v_mfma_i32_16x16x64_i8 (the int4 part of the mixed add)       */
  /* The 2:4 GEMM's unit of work, a 16 x 16 x 128 sparse product with its
   * per-K-block promotion (4 fp32 results per lane): */
  SG_PROBE_SMFMAC_PROMOTED = 3,  /* from zero, then acc += p * (sw * sx)  (4 FMAs)           */
  SG_PROBE_SMFMAC_RESCALED = 4,  /* acc *= r (4 multiplies), then accumulated in the matrix core */
  SG_PROBE_MFMA_FP6 = 5          /* v_mfma_f32_16x16x128_f8f6f4 with e3m2 (bf6) operands: the
                                    exact route for int4 values, whose integers -8..7 e3m2 holds */
} sg_probe_kind;

/* Dense-equivalent operations of one sg_probe_matrix_rate launch (2 per
 * multiply-add; the sparse instruction counts its full K), or -1 for an
 * invalid kind or iters < 1. */
int64_t sg_probe_matrix_ops(int kind, int iters);

/* Launches SG_PROBE_WORKGROUPS workgroups; every wave issues `iters` rounds of
 * eight independent instructions of the given kind on register operands.
 *   sink   : device float[SG_PROBE_WORKGROUPS * 512], receives one value per
 *            thread so that the work cannot be optimised away.
 *   clocks : device uint64[4 * SG_PROBE_WORKGROUPS]; for workgroup b the first
 *            wave stores shader-clock cycles at start and end (entries 4b, 4b+1)
 *            and the constant 100 MHz real-time counter at start and end
 *            (4b+2, 4b+3).
 * Returns SG_ERR_NULL for a null buffer, SG_ERR_UNSUPPORTED for an unknown
 * kind, SG_ERR_SHAPE for iters < 1. */
sg_status sg_probe_matrix_rate(int kind, int iters, float* sink, uint64_t* clocks, hipStream_t stream);

/* Streaming read of `bytes` bytes at src (16-byte aligned, bytes a multiple of
 * 16) by `workgroups` workgroups of 256 threads: each thread reads 16-byte
 * chunks in a grid-stride loop, four loads in flight, and stores one value
 * derived from them to sink[workgroups * 256] (device float) so that the
 * reads cannot be optimised away.  Gives the HBM read rate a kernel that only
 * streams reaches, for a buffer of a given size.  SG_ERR_NULL, SG_ERR_SHAPE
 * (bytes < 16 or not a multiple of 16, workgroups < 1) or SG_ERR_ALIGN. */
sg_status sg_probe_stream_read(const void* src, int64_t bytes, int workgroups, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
