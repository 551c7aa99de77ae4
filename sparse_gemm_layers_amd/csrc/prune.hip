// 2:4 magnitude pruning along K with compressed output (values + metadata).
//
// torchao PR #3258 "Introduce new W8A8-FP-CSR quantization API", jcaip's
// review: each group of 4 consecutive weights of a row keeps its two largest
// magnitudes, and only the kept values plus the sparsity metadata are stored.
// Equal magnitudes keep the lower index; NaN counts as larger than any number.
// Weights may be fp32, bf16 or e4m3 codes (already-quantised weights).
// Metadata: nibble = i0 | i1 << 2 for the kept positions i0 < i1; two groups
// per byte, the even group in the low nibble.  HBM-bound: each lane streams 8 consecutive weights (two groups)
// and writes 4 values and one metadata byte, all lanes contiguous.
#include "common.h"

namespace sg {

// Kept positions of one group, ranked by (magnitude key descending, index
// ascending): the first kept is the largest (lowest index among equals), the
// second the largest of the rest.  Always returns two distinct positions.
__device__ __forceinline__ void top2(const uint32_t m[4], int& i0, int& i1) {
  int b = 0;
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (m[j] > m[b]) b = j;
  int s = b == 0 ? 1 : 0;
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (j != b && m[j] > m[s]) s = j;
  i0 = min(b, s);
  i1 = max(b, s);
}

// Magnitude keys: the encoding with its sign bit cleared orders like |w| for
// all three formats (+0 and -0 give the same key), and every NaN is mapped to
// one key just above infinity (e4m3's only NaN magnitude, 0x7F, is already the
// largest code).  So NaN outranks every number and NaNs tie with each other.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ static void load8(const float* p, uint32_t bits[8], uint32_t key[8]) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    bits[0] = a.x; bits[1] = a.y; bits[2] = a.z; bits[3] = a.w;
    bits[4] = b.x; bits[5] = b.y; bits[6] = b.z; bits[7] = b.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = min(bits[i] & 0x7fffffffu, 0x7f800001u);
  }
  __device__ static void store4(float* p, const uint32_t v[4]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct Elem<uint16_t> {
  __device__ static void load8(const uint16_t* p, uint32_t bits[8], uint32_t key[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bits[2 * i] = w[i] & 0xffffu;
      bits[2 * i + 1] = w[i] >> 16;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = min(bits[i] & 0x7fffu, 0x7f81u);
  }
  __device__ static void store4(uint16_t* p, const uint32_t v[4]) {
    *reinterpret_cast<uint2*>(p) = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
  }
};
template <>
struct Elem<uint8_t> {   // e4m3 codes
  __device__ static void load8(const uint8_t* p, uint32_t bits[8], uint32_t key[8]) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bits[i] = (a.x >> (8 * i)) & 0xffu;
      bits[4 + i] = (a.y >> (8 * i)) & 0xffu;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = bits[i] & 0x7fu;
  }
  __device__ static void store4(uint8_t* p, const uint32_t v[4]) {
    *reinterpret_cast<uint32_t*>(p) = v[0] | (v[1] << 8) | (v[2] << 16) | (v[3] << 24);
  }
};

template <typename T>
__global__ void __launch_bounds__(256) k_prune24(const T* __restrict__ w, int64_t rows, int64_t k,
                                                 int64_t ldw, T* __restrict__ vals, int64_t ldv,
                                                 uint8_t* __restrict__ meta, int64_t ldm) {
  const int64_t per_row = k >> 3;
  const int64_t total = rows * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += stride) {
    const int64_t r = it / per_row, c = it - r * per_row;
    uint32_t bits[8], key[8];
    Elem<T>::load8(w + r * ldw + c * 8, bits, key);
    int a0, a1, b0, b1;
    top2(key, a0, a1);
    top2(key + 4, b0, b1);
    const uint32_t out[4] = {bits[a0], bits[a1], bits[4 + b0], bits[4 + b1]};
    Elem<T>::store4(vals + r * ldv + c * 4, out);
    meta[r * ldm + c] = (uint8_t)((a0 | (a1 << 2)) | ((b0 | (b1 << 2)) << 4));
  }
}

}  // namespace sg

using namespace sg;

extern "C" sg_status sg_sparse24_prune_compress(const void* w, sg_dtype dt, int64_t rows, int64_t k,
                                                int64_t ldw, void* vals, int64_t ldv, uint8_t* meta,
                                                int64_t ldm, hipStream_t stream) {
  if (!w || !vals || !meta) return SG_ERR_NULL;
  if (dt != SG_F32 && dt != SG_BF16 && dt != SG_E4M3) return SG_ERR_UNSUPPORTED;
  if (rows <= 0 || k <= 0 || k % 8 != 0 || ldw < k || ldv < k / 2 || ldm < k / 8) return SG_ERR_SHAPE;
  const int64_t es = (int64_t)dtype_size(dt);
  if (!aligned(w, 16) || !aligned(vals, 16) || (ldw * es) % 16 || ldv % 4) return SG_ERR_ALIGN;
  clear_hip_error();
  const unsigned g = grid_for(rows * (k / 8), 256);
  if (dt == SG_F32)
    k_prune24<float><<<g, 256, 0, stream>>>((const float*)w, rows, k, ldw, (float*)vals, ldv, meta, ldm);
  else if (dt == SG_BF16)
    k_prune24<uint16_t><<<g, 256, 0, stream>>>((const uint16_t*)w, rows, k, ldw, (uint16_t*)vals, ldv, meta,
                                               ldm);
  else
    k_prune24<uint8_t><<<g, 256, 0, stream>>>((const uint8_t*)w, rows, k, ldw, (uint8_t*)vals, ldv, meta, ldm);
  return launch_status();
}
