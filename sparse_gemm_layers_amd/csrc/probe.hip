// Measurement helpers: sustained rate of the matrix-core instructions the GEMM
// kernels use, and the shader clock while they run (declared in sg_probe.h).
#include "common.h"
#include "sg_probe.h"

namespace sg {

template <int KIND>
__global__ void __launch_bounds__(512) k_probe_matrix(int iters, float* sink, uint64_t* clocks) {
  const int l = threadIdx.x & 63;
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  // e4m3 1.0 (0x38) operands; int8 operands 1; sparse index: groups keep elements 0 and 1
  const int fp8_one = 0x38383838, i8_one = 0x01010101;
  float total = 0.f;
  if constexpr (KIND == SG_PROBE_MFMA_FP6) {
    // e3m2 1.0 is 0b001100; any 6-bit pattern serves the rate, so the packed
    // operand words are filled with one repeated byte
    const int w0 = 0x0c30c30c, w1 = 0x30c30c30, w2 = (int)0xc30c30c3u;
    const v8i a = {w0, w1, w2, w0, w1, w2 + (l & 1), 0, 0};
    const v8i b = {w0, w1, w2, w0, w1, w2, 0, 0};
    v4f acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[k], 3, 3, 0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) total += acc[k][0] + acc[k][3];
  } else if constexpr (KIND == SG_PROBE_MFMA_FP8) {
    const v8i a = {fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one + (l & 1)};
    const v8i b = {fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one};
    v4f acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[k], 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) total += acc[k][0] + acc[k][3];
  } else if constexpr (KIND == SG_PROBE_SMFMAC_FP8) {
    const v4i a = {fp8_one, fp8_one, fp8_one, fp8_one + (l & 1)};
    const v8i b = {fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one};
    const int idx = 0x44444444;   // every group of four keeps elements 0 and 1
    v4f acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, acc[k], idx, 0, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) total += acc[k][0] + acc[k][3];
  } else if constexpr (KIND == SG_PROBE_SMFMAC_PROMOTED || KIND == SG_PROBE_SMFMAC_RESCALED) {
    const v4i a = {fp8_one, fp8_one, fp8_one, fp8_one + (l & 1)};
    const v8i b = {fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one, fp8_one};
    const int idx = 0x44444444;
    // per-lane scales that the compiler cannot fold (each lane's own value)
    const float c = 1.0f + 0x1p-20f * (float)l, r = 1.0f - 0x1p-21f * (float)l;
    v4f acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (KIND == SG_PROBE_SMFMAC_PROMOTED) {
          // an empty asm that "changes" b keeps the product inside the loop
          // (the operands are otherwise the same every round)
          v8i bb = b;
          asm volatile("" : "+v"(bb));
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          const v4f p = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, bb, z, idx, 0, 0);
          acc[k] += p * c;
        } else {
          acc[k] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, acc[k] * r, idx, 0, 0);
        }
      }
#pragma unroll
    for (int k = 0; k < 8; ++k) total += acc[k][0] + acc[k][3];
  } else {
    const v4i a = {i8_one, i8_one, i8_one, i8_one + (l & 1)};
    const v4i b = {i8_one, i8_one, i8_one, i8_one};
    v4i acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (v4i){0, 0, 0, 0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[k], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) total += (float)(acc[k][0] + acc[k][3]);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * 512 + threadIdx.x] = total;
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x] = c0;
    clocks[4 * blockIdx.x + 1] = c1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

// Grid-stride streaming read: four 16-byte loads in flight per thread.
__global__ void __launch_bounds__(256) k_probe_stream(const uint4* __restrict__ src, int64_t chunks,
                                                      float* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t h = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < chunks; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    h ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < chunks; i += stride) {
    const uint4 a = src[i];
    h ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)(h & 0xffffu);
}

}  // namespace sg

using namespace sg;

extern "C" int64_t sg_probe_matrix_ops(int kind, int iters) {
  if (iters < 1) return -1;
  int64_t per;   // dense-equivalent operations of one instruction
  switch (kind) {
    case SG_PROBE_MFMA_FP8: per = 2LL * 16 * 16 * 128; break;
    case SG_PROBE_SMFMAC_FP8: per = 2LL * 16 * 16 * 128; break;
    case SG_PROBE_MFMA_I8: per = 2LL * 16 * 16 * 64; break;
    case SG_PROBE_SMFMAC_PROMOTED:
    case SG_PROBE_SMFMAC_RESCALED:
    case SG_PROBE_MFMA_FP6: per = 2LL * 16 * 16 * 128; break;
    default: return -1;
  }
  return per * 8 * iters * 8 * (int64_t)SG_PROBE_WORKGROUPS;   // 8 waves per workgroup, 8 per round
}

extern "C" sg_status sg_probe_matrix_rate(int kind, int iters, float* sink, uint64_t* clocks, hipStream_t stream) {
  if (!sink || !clocks) return SG_ERR_NULL;
  if (kind < SG_PROBE_MFMA_FP8 || kind > SG_PROBE_MFMA_FP6) return SG_ERR_UNSUPPORTED;
  if (iters < 1) return SG_ERR_SHAPE;
  clear_hip_error();
  constexpr int G = SG_PROBE_WORKGROUPS;
  switch (kind) {
    case SG_PROBE_MFMA_FP8: k_probe_matrix<SG_PROBE_MFMA_FP8><<<G, 512, 0, stream>>>(iters, sink, clocks); break;
    case SG_PROBE_SMFMAC_FP8: k_probe_matrix<SG_PROBE_SMFMAC_FP8><<<G, 512, 0, stream>>>(iters, sink, clocks); break;
    case SG_PROBE_MFMA_I8: k_probe_matrix<SG_PROBE_MFMA_I8><<<G, 512, 0, stream>>>(iters, sink, clocks); break;
    case SG_PROBE_SMFMAC_PROMOTED:
      k_probe_matrix<SG_PROBE_SMFMAC_PROMOTED><<<G, 512, 0, stream>>>(iters, sink, clocks);
      break;
    case SG_PROBE_SMFMAC_RESCALED:
      k_probe_matrix<SG_PROBE_SMFMAC_RESCALED><<<G, 512, 0, stream>>>(iters, sink, clocks);
      break;
    default: k_probe_matrix<SG_PROBE_MFMA_FP6><<<G, 512, 0, stream>>>(iters, sink, clocks); break;
  }
  return launch_status();
}

extern "C" sg_status sg_probe_stream_read(const void* src, int64_t bytes, int workgroups, float* sink,
                                          hipStream_t stream) {
  if (!src || !sink) return SG_ERR_NULL;
  if (bytes < 16 || bytes % 16 || workgroups < 1) return SG_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return SG_ERR_ALIGN;
  clear_hip_error();
  k_probe_stream<<<(unsigned)workgroups, 256, 0, stream>>>(static_cast<const uint4*>(src), bytes / 16, sink);
  return launch_status();
}
