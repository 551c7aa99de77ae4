// Packs a 2:4-compressed FP8 weight (canonical values [N, K/2] + metadata
// [N, K/8]) into the gfx950 layout the sparse GEMM kernels stream: one
// 1280-byte chunk per 16-row block and 128-wide K block, a row block's chunks
// contiguous along K, each laid out as 16 rows of the kernels' LDS image
// (SMFMAC operand slices pre-permuted and bank-swizzled).  Packing is a byte permutation: torchao PR #3258 ("Introduce
// new W8A8-FP-CSR quantization API", jcaip: pack FP8 semi-structured weights
// with the hardware's packing kernel) and CUTLASS issue #2029 (klevzoff:
// values and metadata E go to the mainloop in the hardware's layout).
#include "gemm_common.h"

namespace sg {

// One thread per (row block, K block, local row); rows past N are written as zeros.
__global__ void __launch_bounds__(256) k_pack24(const uint8_t* __restrict__ wv, int64_t ldv,
                                                const uint8_t* __restrict__ meta, int64_t ldm, int64_t N, int KB,
                                                int64_t total, uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int r = (int)(i & (PK_ROWS - 1));
    const int64_t blk = i >> 4;                  // chunk index R * KB + kb
    const int kb = (int)(blk % KB);
    const int64_t n = (blk / KB) * PK_ROWS + r;
    uint4 v[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    uint4 m = {0u, 0u, 0u, 0u};
    if (n < N) {
      const uint4* src = reinterpret_cast<const uint4*>(wv + n * ldv + (int64_t)kb * 64);
      v[0] = src[0]; v[1] = src[1]; v[2] = src[2]; v[3] = src[3];
      m = *reinterpret_cast<const uint4*>(meta + n * ldm + (int64_t)kb * 16);
    }
    // the row's 64 bytes as eight 8-byte pieces q[0..7]
    const uint2 q[8] = {make_uint2(v[0].x, v[0].y), make_uint2(v[0].z, v[0].w), make_uint2(v[1].x, v[1].y),
                        make_uint2(v[1].z, v[1].w), make_uint2(v[2].x, v[2].y), make_uint2(v[2].z, v[2].w),
                        make_uint2(v[3].x, v[3].y), make_uint2(v[3].z, v[3].w)};
    uint8_t* base = out + blk * PK_CHUNK;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int p = sp_a_off(g) >> 3;        // pieces p and p + 2
      *reinterpret_cast<uint4*>(base + pk_val_off(r, g)) = make_uint4(q[p].x, q[p].y, q[p + 2].x, q[p + 2].y);
      *reinterpret_cast<int*>(base + PK_META + pk_meta_word(r, g)) = sp_meta_word(m, g);
    }
  }
}

// One thread per (row block, K block, local row) of a 2:4 int4 weight: the
// row's 32 code bytes and 16 metadata bytes of the K block, as stored, at
// their places in the blocked chunk; rows past N are written as zeros.
__global__ void __launch_bounds__(256) k_pack_w4(const uint8_t* __restrict__ wv4, int64_t ldv,
                                                 const uint8_t* __restrict__ meta, int64_t ldm, int64_t N, int KB,
                                                 int64_t total, uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int r = (int)(i & (PK_ROWS - 1));
    const int64_t blk = i >> 4;                  // chunk index R * KB + kb
    const int kb = (int)(blk % KB);
    const int64_t n = (blk / KB) * PK_ROWS + r;
    uint4 c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u}, m = {0u, 0u, 0u, 0u};
    if (n < N) {
      const uint4* src = reinterpret_cast<const uint4*>(wv4 + n * ldv + (int64_t)kb * 32);
      c0 = src[0];
      c1 = src[1];
      m = *reinterpret_cast<const uint4*>(meta + n * ldm + (int64_t)kb * 16);
    }
    uint8_t* base = out + blk * PK4_CHUNK;
    *reinterpret_cast<uint4*>(base + r * 32) = c0;
    *reinterpret_cast<uint4*>(base + r * 32 + 16) = c1;
    *reinterpret_cast<uint4*>(base + PK4_META + r * 16) = m;
  }
}

}  // namespace sg

using namespace sg;

extern "C" int64_t sg_sparse24_w4_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 128 != 0) return -1;
  return cdiv(N, PK_ROWS) * (K / 128) * PK4_CHUNK;
}

extern "C" sg_status sg_sparse24_pack_w4(const uint8_t* wv4, int64_t ldwv4, const uint8_t* wmeta, int64_t ldwm,
                                         int64_t N, int64_t K, uint8_t* packed, hipStream_t stream) {
  if (!wv4 || !wmeta || !packed) return SG_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 128 != 0 || ldwv4 < K / 4 || ldwm < K / 8) return SG_ERR_SHAPE;
  if (!aligned(wv4, 16) || !aligned(wmeta, 16) || !aligned(packed, 16) || ldwv4 % 16 || ldwm % 16)
    return SG_ERR_ALIGN;
  const int64_t total = cdiv(N, PK_ROWS) * PK_ROWS * (K / 128);
  clear_hip_error();
  k_pack_w4<<<grid_for(total, 256), 256, 0, stream>>>(wv4, ldwv4, wmeta, ldwm, N, (int)(K / 128), total, packed);
  return launch_status();
}

extern "C" int64_t sg_sparse24_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 128 != 0) return -1;
  return cdiv(N, PK_ROWS) * (K / 128) * PK_CHUNK;
}

extern "C" sg_status sg_sparse24_pack_gfx950(const uint8_t* wv, int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                             int64_t N, int64_t K, uint8_t* packed, hipStream_t stream) {
  if (!wv || !wmeta || !packed) return SG_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 128 != 0 || ldwv < K / 2 || ldwm < K / 8) return SG_ERR_SHAPE;
  if (!aligned(wv, 16) || !aligned(wmeta, 16) || !aligned(packed, 16) || ldwv % 16 || ldwm % 16)
    return SG_ERR_ALIGN;
  const int64_t total = cdiv(N, PK_ROWS) * PK_ROWS * (K / 128);
  clear_hip_error();
  k_pack24<<<grid_for(total, 256), 256, 0, stream>>>(wv, ldwv, wmeta, ldwm, N, (int)(K / 128), total, packed);
  return launch_status();
}
