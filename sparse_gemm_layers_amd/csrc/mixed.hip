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
// Workgroup tile 256 W rows (n) x 128 X rows (m), W on the matrix-core A
// side, 8 waves in two K groups of a 2 x 2 wave grid (each wave 128 n x 64 m),
// like the FP8 sparse kernel: operands travel HBM -> LDS with buffer loads
// that write LDS directly, two "double stages" alternate, and group q
// multiplies half q of a double stage.  An int4 double stage holds two
// 128-wide K blocks (group q takes K block 2 it + q, promoted with its own
// scales); a bf16 double stage holds 64 columns of X2 and W2 (group q takes
// columns 32 q .. 32 q + 31).  At the end the two groups add their partial
// tiles and the finished tile is stored in whole rows.
#include "tile_epilogue.h"

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
  int vec16;      // y is 16-byte aligned and a row of y is a multiple of 16 bytes
};

namespace mixed {
// int4 K block (one half of a double stage), bytes:
//   X1 128 rows x 64 B, W1 256 rows x 64 B: 16-byte chunk c of row r at c ^ swz4(r)
//   sx 128 floats (+ a dummy copy written by the waves that have no sx rows), sw 256 floats
constexpr int X1_OFF = 0;
constexpr int W1_OFF = TILE_M * 64;
constexpr int SX_OFF = W1_OFF + TILE_N * 64;
constexpr int SW_OFF = SX_OFF + 2 * TILE_M * 4;
constexpr int HALF = SW_OFF + TILE_N * 4;
// bf16 double stage (64 columns): X2 128 rows x 128 B, W2 256 rows x 128 B,
// 16-byte chunk c of row r at c ^ swz8q(r)
constexpr int X2_OFF = 0;
constexpr int W2_OFF = TILE_M * 128;
// one double-stage buffer; it also holds a K group's partial tile at the end
constexpr int BUF = 65536;
static_assert(2 * HALF <= BUF && W2_OFF + TILE_N * 128 <= BUF, "stages fit the buffers");
}  // namespace mixed

#if SG_DEVICE_PASS
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mixed_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void mixed_lds_void;

// Per-lane source offsets, fixed for the whole K loop (the K block or the
// column block enters through the scalar offset).  Every wave issues six
// 1 KB loads per double stage (64 lanes x 16 B) and, for int4 stages, two
// 256-byte scale loads.
struct MixedPlan {
  uint32_t io[3];       // int4: X1 slot, W1 slots (same for both halves)
  uint32_t bo[6];       // bf16: X2 slots 0-1, W2 slots 2-5
  uint32_t so[2], sdst[2];
  int sk[2];            // 0: sx1, 1: sw1
};

__device__ __forceinline__ MixedPlan mixed_plan(const MixedArgs& a, int64_t n0, int64_t m0, int wave, int l) {
  using namespace mixed;
  MixedPlan p;
  {   // int4: load jj = 0 fills X1 slot `wave`, jj = 1, 2 W1 slots 8 (jj - 1) + wave; 16 rows of 64 B per slot
    const int r = 16 * wave + (l >> 2), c = (l & 3) ^ swz4(r);
    p.io[0] = (uint32_t)(r * a.ldx1 + c * 16);
#pragma unroll
    for (int jj = 1; jj < 3; ++jj) {
      const int rw = 16 * (8 * (jj - 1) + wave) + (l >> 2), cw = (l & 3) ^ swz4(rw);
      p.io[jj] = (uint32_t)(rw * a.ldw1 + cw * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 6; ++j) {   // bf16: 8 rows of 128 B per slot
    const int slot = j < 2 ? 8 * j + wave : 8 * (j - 2) + wave;
    const int r = 8 * slot + (l >> 3), c = (l & 7) ^ swz8q(r);
    p.bo[j] = (uint32_t)(r * (j < 2 ? a.ldx2 : a.ldw2) * 2 + c * 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sidx = 2 * wave + j, h = sidx >> 3, t = sidx & 7;
    if (t < 2 || t >= 6) {
      const int tp = t < 2 ? t : t - 6;
      const int64_t m = min(m0 + tp * 64 + l, a.M - 1);
      p.so[j] = (uint32_t)(m * a.sx1_sm * 4);
      p.sdst[j] = h * HALF + SX_OFF + (t < 2 ? 0 : TILE_M * 4) + tp * 256;
      p.sk[j] = 0;
    } else {
      const int64_t n = min(n0 + (t - 2) * 64 + l, a.N - 1);
      p.so[j] = (uint32_t)(n * a.sw1_sn * 4);
      p.sdst[j] = h * HALF + SW_OFF + (t - 2) * 256;
      p.sk[j] = 1;
    }
  }
  return p;
}

struct MixedRes {
  __amdgpu_buffer_rsrc_t x1, w1, x2, w2, sx, sw;
};

// int4 K blocks kb0, kb0 + 1 (the second clamped to the last block).
__device__ __forceinline__ void mixed_issue_int4(uint8_t* st, const MixedPlan& p, const MixedRes& r,
                                                 const MixedArgs& a, int kb0, int KB1, int wave) {
  using namespace mixed;
  const int kbh[2] = {kb0, min(kb0 + 1, KB1 - 1)};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint8_t* hs = st + h * HALF;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.x1, (mixed_lds_void*)(hs + X1_OFF + wave * 1024), 16, p.io[0],
                                             kbh[h] * 64, 0, 0);
#pragma unroll
    for (int jj = 1; jj < 3; ++jj)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.w1, (mixed_lds_void*)(hs + W1_OFF + (8 * (jj - 1) + wave) * 1024),
                                               16, p.io[jj], kbh[h] * 64, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int h = (2 * wave + j) >> 3;
    if (p.sk[j] == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sx, (mixed_lds_void*)(st + p.sdst[j]), 4, p.so[j],
                                               (int)(kbh[h] * a.sx1_sk * 4), 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sw, (mixed_lds_void*)(st + p.sdst[j]), 4, p.so[j],
                                               (int)(kbh[h] * a.sw1_sk * 4), 0, 0);
  }
}

// bf16 columns 64 b .. 64 b + 63 (columns past K2 are loaded but not used).
__device__ __forceinline__ void mixed_issue_bf16(uint8_t* st, const MixedPlan& p, const MixedRes& r, int b,
                                                 int wave) {
  using namespace mixed;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int slot = j < 2 ? 8 * j + wave : 8 * (j - 2) + wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 2 ? r.x2 : r.w2,
                                             (mixed_lds_void*)(st + (j < 2 ? X2_OFF : W2_OFF) + slot * 1024), 16,
                                             p.bo[j], b * 128, 0, 0);
  }
}
#endif  // SG_DEVICE_PASS

// Low / high nibbles of 16 packed bytes as two int8 operand vectors (x16).
__device__ __forceinline__ void unpack_int4(const uint4 p, v4i& lo, v4i& hi) {
  lo = (v4i){(int)((p.x << 4) & 0xf0f0f0f0u), (int)((p.y << 4) & 0xf0f0f0f0u),
             (int)((p.z << 4) & 0xf0f0f0f0u), (int)((p.w << 4) & 0xf0f0f0f0u)};
  hi = (v4i){(int)(p.x & 0xf0f0f0f0u), (int)(p.y & 0xf0f0f0f0u), (int)(p.z & 0xf0f0f0f0u),
             (int)(p.w & 0xf0f0f0f0u)};
}

__device__ __forceinline__ v8bf as_bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

template <typename T>
__device__ __forceinline__ T mx_ld(const uint8_t* st, uint32_t off) {
  return *reinterpret_cast<const T*>(st + off);
}

// Lane-constant LDS offsets (the swizzles depend on the row modulo 16 only,
// and every sub-tile starts at a multiple of 16 rows).
struct MixedLane {
  uint32_t x1, w1, sx, sw;   // int4 half: X1 row wm*64 + lr chunk g, W1 row wn*128 + lr chunk g, scales
  uint32_t x2, w2;           // bf16: chunk 4 q + g of X2 row wm*64 + lr / W2 row wn*128 + lr
};

__device__ __forceinline__ MixedLane mixed_lane(int wn, int wm, int g, int lr, int q) {
  using namespace mixed;
  MixedLane o;
  const int xr = wm * 64 + lr, wr = wn * 128 + lr;
  o.x1 = X1_OFF + xr * 64 + ((g ^ swz4(lr)) << 4);
  o.w1 = W1_OFF + wr * 64 + ((g ^ swz4(lr)) << 4);
  o.sx = SX_OFF + xr * 4;
  o.sw = SW_OFF + (wn * 128 + 4 * g) * 4;
  o.x2 = X2_OFF + xr * 128 + (((4 * q + g) ^ swz8q(lr)) << 4);
  o.w2 = W2_OFF + wr * 128 + (((4 * q + g) ^ swz8q(lr)) << 4);
  return o;
}

__device__ __forceinline__ void promote(v4f& acc, const v4i& p, const float4& sw4, float sx) {
  acc[0] = fmaf((float)p[0], sw4.x * sx, acc[0]);
  acc[1] = fmaf((float)p[1], sw4.y * sx, acc[1]);
  acc[2] = fmaf((float)p[2], sw4.z * sx, acc[2]);
  acc[3] = fmaf((float)p[3], sw4.w * sx, acc[3]);
}

// One int4 K block: two i8 MFMAs per sub-tile give 256 * sum x1 w1 exactly;
// the partial is promoted with the block's scales.  Sub-tile row i is
// promoted after the MFMAs of row i + 1 are issued, and the scheduling
// barrier keeps that order (left alone, the compiler issues all 64 MFMAs
// first and needs 128 registers for their results).
__device__ __forceinline__ void mixed_int4_block(const uint8_t* st, v4f (&acc)[8][4], const MixedLane& o) {
  float sxj[4];
  v4i blo[4], bhi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sxj[j] = mx_ld<float>(st, o.sx + j * 64) * 0.00390625f;   // 2^-8 undoes the x16 of both operands
    unpack_int4(mx_ld<uint4>(st, o.x1 + j * 1024), blo[j], bhi[j]);
  }
  uint4 anext = mx_ld<uint4>(st, o.w1);
  float4 swnext = mx_ld<float4>(st, o.sw);
  v4i pr[2][4];      // MFMA results of rows i (pr[i & 1]) and i - 1
  float4 swr[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 araw = anext;
    const float4 sw4 = swnext;
    if (i + 1 < 8) {
      anext = mx_ld<uint4>(st, o.w1 + (i + 1) * 1024);
      swnext = mx_ld<float4>(st, o.sw + (i + 1) * 64);
    }
    v4i alo, ahi;
    unpack_int4(araw, alo, ahi);
    swr[i & 1] = sw4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i z = {0, 0, 0, 0};
      pr[i & 1][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo[j], z, 0, 0, 0);
      pr[i & 1][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi[j], pr[i & 1][j], 0, 0, 0);
    }
    if (i > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) promote(acc[i - 1][j], pr[(i - 1) & 1][j], swr[(i - 1) & 1], sxj[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) promote(acc[7][j], pr[1][j], swr[1], sxj[j]);
}

// 32 bf16 columns (lane group g holds 8 of them, the same ones for A and B).
__device__ __forceinline__ void mixed_bf16_block(const uint8_t* st, v4f (&acc)[8][4], const MixedLane& o) {
  uint4 bx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bx[j] = mx_ld<uint4>(st, o.x2 + j * 2048);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 av = mx_ld<uint4>(st, o.w2 + i * 2048);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(av), as_bf(bx[j]), acc[i][j], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(512) k_mixed(MixedArgs a, int tiles_m, int tiles_n) {
#if SG_DEVICE_PASS
  using namespace mixed;
  __shared__ __attribute__((aligned(1024))) uint8_t db0[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t db1[BUF];

  int tn, tm;
  tile_coords(tiles_m, tiles_n, tn, tm);
  const int64_t n0 = (int64_t)tn * TILE_N, m0 = (int64_t)tm * TILE_M;

  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = wave >> 2, w4 = wave & 3;
  const int wn = w4 & 1, wm = w4 >> 1;
  const int g = l >> 4, lr = l & 15;
  const int KB1 = (int)(a.K1 >> 7);
  const int NIT1 = (KB1 + 1) >> 1;
  const int NIT2 = (int)((a.K2 + 63) >> 6);

  const int64_t mrows = min((int64_t)TILE_M, a.M - m0), nrows = min((int64_t)TILE_N, a.N - n0);
  MixedRes rs;
  rs.x1 = mixed_rsrc(a.x1 + m0 * a.ldx1, (uint32_t)(mrows * a.ldx1));
  rs.w1 = mixed_rsrc(a.w1 + n0 * a.ldw1, (uint32_t)(nrows * a.ldw1));
  rs.x2 = mixed_rsrc(a.K2 ? a.x2 + m0 * a.ldx2 : a.x2, a.K2 ? (uint32_t)(mrows * a.ldx2 * 2) : 0u);
  rs.w2 = mixed_rsrc(a.K2 ? a.w2 + n0 * a.ldw2 : a.w2, a.K2 ? (uint32_t)(nrows * a.ldw2 * 2) : 0u);
  rs.sx = mixed_rsrc(a.sx1, 0xffffffffu);
  rs.sw = mixed_rsrc(a.sw1, 0xffffffffu);
  const MixedPlan plan = mixed_plan(a, n0, m0, wave, l);
  const MixedLane lo = mixed_lane(wn, wm, g, lr, q);

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // int4 double stages it = 0 .. NIT1 - 1 (K blocks 2 it, 2 it + 1) in db0,
  // db1, db0, ...; the last one's successor is the first bf16 stage.
  mixed_issue_int4(db0, plan, rs, a, 0, KB1, wave);
  for (int it0 = 0; it0 < NIT1; it0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = it0 + u;
      if (it < NIT1) {
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 1 < NIT1) mixed_issue_int4(u == 0 ? db1 : db0, plan, rs, a, 2 * (it + 1), KB1, wave);
        else if (NIT2 > 0) mixed_issue_bf16(u == 0 ? db1 : db0, plan, rs, 0, wave);
        if (2 * it + q < KB1) mixed_int4_block((u == 0 ? db0 : db1) + q * HALF, acc, lo);
      }
    }
  }
  // bf16 stages b = 0 .. NIT2 - 1 continue the alternation (stage NIT1 + b).
  for (int b = 0; b < NIT2; ++b) {
    uint8_t* const cur = ((NIT1 + b) & 1) ? db1 : db0;
    uint8_t* const nxt = ((NIT1 + b) & 1) ? db0 : db1;
    wait_vmcnt<0>();
    __syncthreads();
    if (b + 1 < NIT2) mixed_issue_bf16(nxt, plan, rs, b + 1, wave);
    if ((int64_t)b * 64 + 32 * q < a.K2) mixed_bf16_block(cur, acc, lo);
  }

  // Add the two groups' partial tiles (group 0 finishes sub-tile rows i < 4,
  // group 1 rows i >= 4) and store the staged tile.
  __syncthreads();
  if (q == 0) xchg_out<4>(reinterpret_cast<float4*>(db0), acc, w4, l);
  else xchg_out<0>(reinterpret_cast<float4*>(db1), acc, w4, l);
  __syncthreads();
  if (q == 0) x2_finish<0, true, false, BUF>(db1, db0, db1, acc, w4, l, wn, wm, g, lr);
  else x2_finish<1, true, false, BUF>(db0, db0, db1, acc, w4, l, wn, wm, g, lr);
  __syncthreads();
  store_staged<true, false, BUF>(a, db0, db1, m0, n0, t);
#endif  // SG_DEVICE_PASS
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
  if (M <= 0 || N <= 0 || K1 <= 0 || K1 % 128 != 0 || K2 < 0 || K2 % 32 != 0) return SG_ERR_SHAPE;
  if (ldx1 < K1 / 2 || ldw1 < K1 / 2 || ldy < N) return SG_ERR_SHAPE;
  if (K2 > 0 && (ldx2 < K2 || ldw2 < K2)) return SG_ERR_SHAPE;
  if (cdiv(M, 128) * cdiv(N, 256) > 0x7fffffffLL) return SG_ERR_SHAPE;
  // Tiles and scales are addressed with 32-bit buffer offsets.
  if (ldx1 >= (1LL << 23) || ldw1 >= (1LL << 23) || ldx2 >= (1LL << 22) || ldw2 >= (1LL << 22)) return SG_ERR_SHAPE;
  if (sx1_sm < 0 || sx1_sk < 0 || sw1_sn < 0 || sw1_sk < 0) return SG_ERR_SHAPE;
  if (((M - 1) * sx1_sm + (K1 / 128 - 1) * sx1_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (((N - 1) * sw1_sn + (K1 / 128 - 1) * sw1_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (!aligned(x1, 16) || !aligned(w1, 16) || ldx1 % 16 || ldw1 % 16 || !aligned(sx1, 4) ||
      !aligned(sw1, 4) || !aligned(y, 2))
    return SG_ERR_ALIGN;
  if (K2 > 0 && (!aligned(x2, 16) || !aligned(w2, 16) || ldx2 % 8 || ldw2 % 8)) return SG_ERR_ALIGN;
  MixedArgs a;
  a.M = M; a.N = N; a.K1 = K1; a.K2 = K2;
  a.x1 = x1; a.ldx1 = ldx1; a.sx1 = sx1; a.sx1_sm = sx1_sm; a.sx1_sk = sx1_sk;
  a.w1 = w1; a.ldw1 = ldw1; a.sw1 = sw1; a.sw1_sn = sw1_sn; a.sw1_sk = sw1_sk;
  a.x2 = x2; a.ldx2 = ldx2; a.w2 = w2; a.ldw2 = ldw2;
  a.y = y; a.ldy = ldy;
  a.vec16 = (ldy % 8 == 0) && aligned(y, 16);
  const int tm = (int)cdiv(M, TILE_M), tn = (int)cdiv(N, TILE_N);
  clear_hip_error();
  k_mixed<<<tm * tn, 512, 0, stream>>>(a, tm, tn);
  return launch_status();
}
