// Epilogue helpers shared by the GEMM kernels: fp32 -> bf16/fp32 stores of
// one lane's 4 consecutive output rows, in the Y [M, N] or Y^T [N, M] layout,
// predicated on the partial M and N tiles.
#pragma once

#include "common.h"

namespace sg {

template <bool OUT_BF16>
__device__ __forceinline__ void store1(void* y, int64_t off, float v) {
  if (OUT_BF16)
    reinterpret_cast<uint16_t*>(y)[off] = (uint16_t)f32_to_bf16(v);
  else
    reinterpret_cast<float*>(y)[off] = v;
}

// Stores rows n..n+3 (consecutive) of column m of a 16x16 result tile.
template <bool OUT_BF16, bool OUT_T, typename Args>
__device__ __forceinline__ void store_quad(const Args& a, int64_t m, int64_t n, const v4f& v) {
  if (m >= a.M || n >= a.N) return;
  if (OUT_T) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < a.N) store1<OUT_BF16>(a.y, (n + e) * a.ldy + m, v[e]);
  } else {
    const int64_t off = m * a.ldy + n;
    if (a.vec_store && n + 3 < a.N) {
      if (OUT_BF16) {
        uint2 p;
        p.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
        p.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + off) = p;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + off) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) store1<OUT_BF16>(a.y, off + e, v[e]);
    }
  }
}

}  // namespace sg
