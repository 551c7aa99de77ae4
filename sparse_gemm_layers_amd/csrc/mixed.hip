// Fused mixed-precision add in one kernel:
//   Y = X1 . W1^T (int4, one fp32 scale per (row, 128-wide K group) on each
//       operand) + X2 . W2^T (bf16), fp32 accumulation, bf16 output.
// CUTLASS issue #2058 "[QST] How to implement a fused mixed precision matrix
// multiplication such as w4a4 + w16a16?" (hyx1999): the two GEMMs are summed,
// not chained; the low-bit part is dequantised in the epilogue of its K tiles.
//
// int4 part on the i8 matrix core: a packed byte b holds elements 2j (low
// nibble) and 2j+1 (high nibble).  (b << 4) & 0xF0 and b & 0xF0 are the two
// nibbles as signed int8 values times 16, so one v_mfma_i32_16x16x64_i8 on
// the "low" bytes and one on the "high" bytes give 256 * sum x1 w1 exactly
// (|partial| <= 2^21) for a 128-wide K block.  X1 and W1 are unpacked the same
// way, so pairing low with low and high with high covers every k once.  The
// partial is promoted per K block: acc += float(P) * (sx1 * sw1 * 2^-8).
// bf16 part: v_mfma_f32_16x16x32_bf16 accumulating straight into acc (no
// scales).
//
// Tile, waves and LDS staging follow the FP8 large-M kernel: 256 W rows x 128
// X rows, 4 waves in 2 x 2, W on the matrix-core A side.  Stage s < KB1 holds
// int4 block s (64 B per row); the following stages hold 64-wide bf16 blocks
// (128 B per row).
#include "gemm_common.h"

namespace sg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct MixedArgs {
  int64_t M, N, K1, K2;
  const uint8_t* x1;
  int64_t ldx1;
  const float* sx1;
  int64_t sx1_sm, sx1_sk;
  const uint8_t* w1;
  int64_t ldw1;
  const float* sw1;
  int64_t sw1_sn, sw1_sk;
  const uint16_t* x2;
  int64_t ldx2;
  const uint16_t* w2;
  int64_t ldw2;
  void* y;
  int64_t ldy;
  int vec_store;
};

namespace mixed {
constexpr int BN = 256, BM = 128;
// stage layout (bytes): X 128 rows x 128 B | W 256 rows x 128 B | sx 128 f | sw 256 f
// (int4 stages use the first 64 B of every row slot, i.e. a row stride of 64 B)
constexpr int X_OFF = 0;
constexpr int W_OFF = BM * 128;
constexpr int SX_OFF = W_OFF + BN * 128;
constexpr int SW_OFF = SX_OFF + BM * 4;
constexpr int BYTES = SW_OFF + BN * 4;
}  // namespace mixed

struct MixedStaged {
  uint4 x[4];
  uint4 w[8];
  float sx, sw;
};

__device__ __forceinline__ void mixed_load(const MixedArgs& a, int64_t n0, int64_t m0, int s, int KB1, int t,
                                           MixedStaged& st) {
  const uint4 zero = {0u, 0u, 0u, 0u};
  if (s < KB1) {
    // int4 block s: 64 B per row; X1 128 rows = 512 chunks, W1 256 rows = 1024 chunks
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 2, c = i & 3;
      const int64_t m = m0 + r;
      st.x[j] = m < a.M ? *reinterpret_cast<const uint4*>(a.x1 + m * a.ldx1 + (int64_t)s * 64 + c * 16) : zero;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 2, c = i & 3;
      const int64_t n = n0 + r;
      st.w[j] = n < a.N ? *reinterpret_cast<const uint4*>(a.w1 + n * a.ldw1 + (int64_t)s * 64 + c * 16) : zero;
    }
    const int64_t m = m0 + (t & 127), n = n0 + t;
    st.sx = (t < 128 && m < a.M) ? a.sx1[m * a.sx1_sm + (int64_t)s * a.sx1_sk] : 0.f;
    st.sw = n < a.N ? a.sw1[n * a.sw1_sn + (int64_t)s * a.sw1_sk] : 0.f;
  } else {
    // bf16 block b: 64 elements = 128 B per row, 16-byte chunks of 8 elements
    const int64_t k0 = (int64_t)(s - KB1) * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 3, c = i & 7;
      const int64_t m = m0 + r, k = k0 + c * 8;
      st.x[j] = (m < a.M && k < a.K2) ? *reinterpret_cast<const uint4*>(a.x2 + m * a.ldx2 + k) : zero;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 3, c = i & 7;
      const int64_t n = n0 + r, k = k0 + c * 8;
      st.w[j] = (n < a.N && k < a.K2) ? *reinterpret_cast<const uint4*>(a.w2 + n * a.ldw2 + k) : zero;
    }
  }
}

__device__ __forceinline__ void mixed_store(uint8_t* sm, int s, int KB1, int t, const MixedStaged& st) {
  using namespace mixed;
  if (s < KB1) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 2, c = i & 3;
      *reinterpret_cast<uint4*>(sm + X_OFF + r * 64 + ((c ^ ((r >> 1) & 3)) << 4)) = st.x[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 2, c = i & 3;
      *reinterpret_cast<uint4*>(sm + W_OFF + r * 64 + ((c ^ ((r >> 1) & 3)) << 4)) = st.w[j];
    }
    if (t < 128) reinterpret_cast<float*>(sm + SX_OFF)[t] = st.sx;
    reinterpret_cast<float*>(sm + SW_OFF)[t] = st.sw;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 3, c = i & 7;
      *reinterpret_cast<uint4*>(sm + X_OFF + r * 128 + ((c ^ (r & 7)) << 4)) = st.x[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 3, c = i & 7;
      *reinterpret_cast<uint4*>(sm + W_OFF + r * 128 + ((c ^ (r & 7)) << 4)) = st.w[j];
    }
  }
}

// Low / high nibbles of 16 packed bytes as two int8 operand vectors (x16).
__device__ __forceinline__ void unpack_int4(const uint4 p, v4i& lo, v4i& hi) {
  lo = (v4i){(int)((p.x << 4) & 0xf0f0f0f0u), (int)((p.y << 4) & 0xf0f0f0f0u),
             (int)((p.z << 4) & 0xf0f0f0f0u), (int)((p.w << 4) & 0xf0f0f0f0u)};
  hi = (v4i){(int)(p.x & 0xf0f0f0f0u), (int)(p.y & 0xf0f0f0f0u), (int)(p.z & 0xf0f0f0f0u),
             (int)(p.w & 0xf0f0f0f0u)};
}

__device__ __forceinline__ v8bf as_bf(uint4 u) {
  return __builtin_bit_cast(v8bf, u);
}

template <bool OUT_T>
__global__ void __launch_bounds__(256, 1) k_mixed(MixedArgs a, int tiles_m, int tiles_n) {
  using namespace mixed;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BYTES];

  const int T = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  const int G = 4;
  const int group = b / (G * tiles_m);
  const int first_n = group * G;
  const int gsize = min(tiles_n - first_n, G);
  const int in_g = b - group * G * tiles_m;
  const int tn = first_n + in_g % gsize;
  const int tm = in_g / gsize;
  const int64_t n0 = (int64_t)tn * BN, m0 = (int64_t)tm * BM;

  const int t = threadIdx.x, l = t & 63, wave = t >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int g = l >> 4, lr = l & 15;
  const int KB1 = (int)(a.K1 >> 7);
  const int NS = KB1 + (int)((a.K2 + 63) >> 6);

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  MixedStaged stg;
  mixed_load(a, n0, m0, 0, KB1, t, stg);
  mixed_store(smem, 0, KB1, t, stg);
  __syncthreads();

  for (int s = 0; s < NS; ++s) {
    const uint8_t* st = smem + (s & 1) * BYTES;
    if (s + 1 < NS) mixed_load(a, n0, m0, s + 1, KB1, t, stg);

    if (s < KB1) {
      const float* sxs = reinterpret_cast<const float*>(st + SX_OFF);
      const float* sws = reinterpret_cast<const float*>(st + SW_OFF);
      float sxj[4];
      v4i blo[4], bhi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wm * 64 + j * 16 + lr;
        sxj[j] = sxs[r] * 0.00390625f;  // 2^-8 undoes the x16 of both unpacked operands
        const uint4 p = *reinterpret_cast<const uint4*>(st + X_OFF + r * 64 + ((g ^ ((r >> 1) & 3)) << 4));
        unpack_int4(p, blo[j], bhi[j]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wn * 128 + i * 16 + lr;
        const uint4 p = *reinterpret_cast<const uint4*>(st + W_OFF + r * 64 + ((g ^ ((r >> 1) & 3)) << 4));
        v4i alo, ahi;
        unpack_int4(p, alo, ahi);
        const float4 sw4 = *reinterpret_cast<const float4*>(sws + wn * 128 + i * 16 + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i z = {0, 0, 0, 0};
          v4i pi = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo[j], z, 0, 0, 0);
          pi = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi[j], pi, 0, 0, 0);
          acc[i][j][0] = fmaf((float)pi[0], sw4.x * sxj[j], acc[i][j][0]);
          acc[i][j][1] = fmaf((float)pi[1], sw4.y * sxj[j], acc[i][j][1]);
          acc[i][j][2] = fmaf((float)pi[2], sw4.z * sxj[j], acc[i][j][2]);
          acc[i][j][3] = fmaf((float)pi[3], sw4.w * sxj[j], acc[i][j][3]);
        }
      }
    } else {
      // bf16 block: lane group g holds 16 elements (32 B); the first 8 feed one
      // MFMA and the next 8 the other, identically for both operands.
      uint4 bx[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wm * 64 + j * 16 + lr;
        const uint8_t* row = st + X_OFF + r * 128;
        bx[j][0] = *reinterpret_cast<const uint4*>(row + (((2 * g) ^ (r & 7)) << 4));
        bx[j][1] = *reinterpret_cast<const uint4*>(row + (((2 * g + 1) ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wn * 128 + i * 16 + lr;
        const uint8_t* row = st + W_OFF + r * 128;
        const uint4 a0 = *reinterpret_cast<const uint4*>(row + (((2 * g) ^ (r & 7)) << 4));
        const uint4 a1 = *reinterpret_cast<const uint4*>(row + (((2 * g + 1) ^ (r & 7)) << 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a0), as_bf(bx[j][0]), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a1), as_bf(bx[j][1]), acc[i][j], 0, 0, 0);
        }
      }
    }

    if (s + 1 < NS) mixed_store(smem + ((s + 1) & 1) * BYTES, s + 1, KB1, t, stg);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_quad<true, OUT_T>(a, m0 + wm * 64 + j * 16 + lr, n0 + wn * 128 + i * 16 + 4 * g, acc[i][j]);
}

}  // namespace sg

using namespace sg;

extern "C" sg_status sg_mixed_gemm_add(int64_t M, int64_t N, int64_t K1, int64_t K2, const uint8_t* x1,
                                       int64_t ldx1, const float* sx1, int64_t sx1_sm, int64_t sx1_sk,
                                       const uint8_t* w1, int64_t ldw1, const float* sw1, int64_t sw1_sn,
                                       int64_t sw1_sk, const uint16_t* x2, int64_t ldx2, const uint16_t* w2,
                                       int64_t ldw2, uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (!x1 || !sx1 || !w1 || !sw1 || !y) return SG_ERR_NULL;
  if (K2 > 0 && (!x2 || !w2)) return SG_ERR_NULL;
  if (M < 0 || N < 0 || K1 <= 0 || K1 % 128 != 0 || K2 < 0 || K2 % 32 != 0) return SG_ERR_SHAPE;
  if (ldx1 < K1 / 2 || ldw1 < K1 / 2 || ldy < N) return SG_ERR_SHAPE;
  if (K2 > 0 && (ldx2 < K2 || ldw2 < K2)) return SG_ERR_SHAPE;
  if (cdiv(M, 128) * cdiv(N, 256) > 0x7fffffffLL) return SG_ERR_SHAPE;
  if (!aligned(x1, 16) || !aligned(w1, 16) || ldx1 % 16 || ldw1 % 16 || !aligned(sx1, 4) ||
      !aligned(sw1, 4) || !aligned(y, 2))
    return SG_ERR_ALIGN;
  if (K2 > 0 && (!aligned(x2, 16) || !aligned(w2, 16) || ldx2 % 8 || ldw2 % 8)) return SG_ERR_ALIGN;
  if (M == 0 || N == 0) return SG_OK;
  MixedArgs a;
  a.M = M; a.N = N; a.K1 = K1; a.K2 = K2;
  a.x1 = x1; a.ldx1 = ldx1; a.sx1 = sx1; a.sx1_sm = sx1_sm; a.sx1_sk = sx1_sk;
  a.w1 = w1; a.ldw1 = ldw1; a.sw1 = sw1; a.sw1_sn = sw1_sn; a.sw1_sk = sw1_sk;
  a.x2 = x2; a.ldx2 = ldx2; a.w2 = w2; a.ldw2 = ldw2;
  a.y = y; a.ldy = ldy;
  a.vec_store = (ldy % 4 == 0) && aligned(y, 8);
  const int tm = (int)cdiv(M, mixed::BM), tn = (int)cdiv(N, mixed::BN);
  clear_hip_error();
  k_mixed<false><<<tm * tn, 256, 0, stream>>>(a, tm, tn);
  return launch_status();
}
