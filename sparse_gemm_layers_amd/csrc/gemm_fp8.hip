// FP8 (e4m3) GEMM with groupwise scales, Y = X . W^T, for a dense weight and
// for a 2:4-compressed weight (values + metadata), on gfx950 matrix cores.
//
// Method (CUTLASS PR #2095 "Improvements for: Groupwise scaling along M for
// FP8 gemm": ScaleGranularityM/N of 1 or 128, one scale per 128-wide K block;
// the K tile's FP8 products start from a zero accumulator and are promoted,
// scaled, into fp32 accumulators):
//   for each 128-wide K block kb:
//     P = W_tile . X_tile^T over kb       (one MFMA/SMFMAC per 16x16 sub-tile, from 0)
//     acc += P * (sx[m, kb] * sw[n, kb])  (fp32 FMA, the promotion)
// The matrix core adds the products of one instruction with only about 12
// bits below the largest product, so partials never carry across K blocks
// inside the instruction: promotion happens after every 128-wide K block.
//
// Operand roles: the weight W is always the matrix-core A operand (rows of
// the 16x16 output tile = n) and X the B operand (columns = m).  This is the
// swap+transpose of CUTLASS issue #2029 ("[QST] CUTLASS support for fp8
// sparse matrix (for W) ...": hwu36 - the sparse FP8 operand must be the left
// one; klevzoff - compute C^T = B^T A^T): gfx950's SMFMAC also takes the
// sparse operand on the A side.  Each lane then owns one output column m, so
// the per-token X scale is one value per lane.  Both output forms (Y and Y^T)
// are stores of the same tile.
//
// gfx950 operand layouts used below (lane l, g = l / 16):
//   dense  v_mfma_f32_16x16x128_f8f6f4: A row / B column l%16, k = 32 g + byte
//   sparse v_smfmac_f32_16x16x128_fp8_fp8: A row l%16 holds 16 compressed
//          bytes: [b, b+8) and [b+16, b+24) of the row's 64 compressed bytes of
//          the K block, b = 32 (g&1) + 8 (g>>1); its 32-bit index holds the
//          metadata nibbles of those 8 groups: bytes {b/4, b/4+1, b/4+4, b/4+5}
//          of the row's 16 metadata bytes (nibble order unchanged).
//          B column l%16, k = 32 g + byte.
//   result: lane l holds D[4 g + i][l % 16], i = 0..3.
#include <type_traits>

#include "tile_epilogue.h"

namespace sg {

struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* x;
  int64_t ldx;
  const float* sx;
  int64_t sx_sm, sx_sk;
  int gm_shift;  // 0 for gran_m == 1, 7 for 128
  const uint8_t* w;  // dense codes [N, K] or compressed codes [N, K/2]
  int64_t ldw;
  const uint8_t* meta;  // [N, K/8] (sparse only)
  int64_t ldm;
  const float* sw;
  int64_t sw_sn, sw_sk;
  int gn_shift;
  void* y;
  int64_t ldy;
  int vec_store;  // Y-form: 4 consecutive n may be stored as one vector
  int vec16;      // y is 16-byte aligned and a row of y is a multiple of 16 bytes
  // Batched problems (grid z = problem index): problem z's operands start this
  // far after problem 0's, in bytes for x, w, meta and y, in floats for the
  // scales; all zero for a single problem.
  int64_t bx, bw, bm, bsx, bsw, by;
  int L;
  // Optional bias (NULL: none): bias[n] is added to every output row after
  // the scales; problem z's bias starts bbs floats after problem 0's.
  const float* bias;
  int64_t bbs;
};

#if SG_DEVICE_PASS
__device__ __forceinline__ void to_batch(GemmArgs& a) {
  const int64_t z = blockIdx.z;
  a.x += z * a.bx;
  a.w += z * a.bw;
  a.meta += z * a.bm;
  a.sx += z * a.bsx;
  a.sw += z * a.bsw;
  a.y = static_cast<uint8_t*>(a.y) + z * a.by;
  if (a.bias) a.bias += z * a.bbs;
}

// v (output rows n .. n + 3 of one column) plus the bias; rows past N read
// bias[N - 1] (they are not stored).
__device__ __forceinline__ v4f with_bias(const GemmArgs& a, int64_t n, v4f v) {
  if (a.bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += a.bias[min(n + e, a.N - 1)];
  }
  return v;
}
#endif

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ v4f mma_dense(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// Accumulating forms, for scales constant along K: the K blocks' products
// add up in the matrix core's fp32 C operand (the int8 form keeps an exact
// int32 sum in the same registers).
__device__ __forceinline__ v4f mma_dense_acc(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <bool I8>
__device__ __forceinline__ v4f mma_sparse_acc(const v4i& a, const v8i& b, const v4f& c, int idx) {
  if constexpr (I8)
    return __builtin_bit_cast(v4f, __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, __builtin_bit_cast(v4i, c), idx, 0, 0));
  else
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c, idx, 0, 0);
}

// The partial of one 16 x 16 x 128 block of a 2:4-sparse A (W) and dense B
// (X), from zero: e4m3 operands (fp32 result), or int8 operands (the exact
// int32 sum, converted to fp32 exactly: |P| <= 64 * 127^2 < 2^24).
template <bool I8>
__device__ __forceinline__ v4f mma_sparse(const v4i& a, const v8i& b, int idx) {
  if constexpr (I8) {
    const v4i z = {0, 0, 0, 0};
    const v4i p = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, z, idx, 0, 0);
    return (v4f){(float)p[0], (float)p[1], (float)p[2], (float)p[3]};
  } else {
    v4f p = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, p, idx, 0, 0);
  }
}


// ================================================= large-M stage layout
// Workgroup tile: 256 W rows (n) x 128 X rows (m).  Operands travel HBM -> LDS
// with buffer loads that write LDS directly (no staging registers); buffer
// resources are based at the tile's first row and sized to the rows that
// exist, so rows past M or N read as zero (the partial tiles) without any
// branch.  One stage holds one 128-wide K block:
//   X    : 128 rows x 128 B; 16-byte chunk c of row r stored at chunk c ^ swz8(r)
//   W    : dense 256 rows x 128 B (same swizzle as X), or
//          sparse 256 rows x 64 B of values; chunk c of row r at c ^ ((r >> 1) & 3)
//          (the packed form holds 16-row chunks of the packed layout instead)
//   meta : sparse only, 256 rows x 16 B, unswizzled
//   sx   : 128 floats, scale of X row r for the stage's K block (+ a copy slot)
//   sw   : 256 floats, scale of W row r
constexpr int BN = TILE_N, BM = TILE_M;
constexpr unsigned RSRC_WORD3 = 0x00020000u;   // gfx9-family raw buffer, 32-bit dwords

typedef __attribute__((address_space(3))) void lds_void;

template <bool SPARSE>
struct Stage {
  static constexpr int X_OFF = 0;
  static constexpr int W_OFF = BM * 128;
  static constexpr int W_BYTES = SPARSE ? BN * 64 : BN * 128;
  static constexpr int M_OFF = W_OFF + W_BYTES;
  static constexpr int M_BYTES = SPARSE ? BN * 16 : 0;
  static constexpr int SX_OFF = M_OFF + M_BYTES;               // 2 x 128 floats (second is a dummy copy)
  static constexpr int SW_OFF = SX_OFF + 2 * BM * 4;
  static constexpr int BYTES = SW_OFF + BN * 4;
};

#if SG_DEVICE_PASS
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)RSRC_WORD3);
}

#endif  // SG_DEVICE_PASS

// Lane-constant LDS byte offsets of the wave's operands within a sparse
// stage.  The swizzles only depend on the row modulo 16, and every sub-tile
// starts at a multiple of 16 rows, so each lane's swizzled offset is fixed;
// sub-tiles are reached by immediate offsets.
struct LaneOffsets {
  uint32_t x0, x1;   // X row wm*64 + lr: the two 16-byte chunks of lane group g
  uint32_t w0, w1;   // W row wn*128 + lr: the two 8-byte halves of the A operand
  uint32_t mt;       // metadata word pair of lane group g
  uint32_t sx;       // X scale of row wm*64 + lr
};

__device__ __forceinline__ LaneOffsets lane_offsets(int wn, int wm, int g, int lr) {
  using L = Stage<true>;
  LaneOffsets o;
  const int xr = wm * 64 + lr, wr = wn * 128 + lr;
  o.x0 = L::X_OFF + xr * 128 + (((2 * g) ^ swz8(lr)) << 4);
  o.x1 = L::X_OFF + xr * 128 + (((2 * g + 1) ^ swz8(lr)) << 4);
  const int sw = (lr >> 1) & 3;
  const int a0 = sp_a_off(g), a1 = a0 + 16;
  o.w0 = L::W_OFF + wr * 64 + ((((a0 >> 4) ^ sw) << 4) | (a0 & 15));
  o.w1 = L::W_OFF + wr * 64 + ((((a1 >> 4) ^ sw) << 4) | (a1 & 15));
  o.mt = L::M_OFF + wr * 16 + 8 * (g & 1);
  o.sx = L::SX_OFF + xr * 4;
  return o;
}

// Packed weights: the stage's W area holds the packed block verbatim, so a
// lane's A operand is one 16-byte read and its index one 4-byte read.
__device__ __forceinline__ LaneOffsets lane_offsets_packed(int wn, int wm, int g, int lr) {
  using L = Stage<true>;
  LaneOffsets o = lane_offsets(wn, wm, g, lr);
  o.w0 = L::W_OFF + pk_val_off(wn * 128 + lr, g);
  o.w1 = 0;
  o.mt = L::W_OFF + LDS_META + pk_meta_word(wn * 128 + lr, g);
  return o;
}

template <typename T>
__device__ __forceinline__ T lds_ld(const uint8_t* st, uint32_t off) {
  return *reinterpret_cast<const T*>(st + off);
}

// Multiplies one sparse LDS stage into the wave's 8 x 4 sub-tiles and
// promotes (GRAN_N = 128 or 1: 128-row or per-row W scales of the K block),
// or accumulates in the matrix core (GRAN_N = 0: scales constant along K,
// applied after the K loop).
template <int GRAN_N, bool PACKED, bool I8>
__device__ __forceinline__ void compute_stage(const uint8_t* st, v4f (&acc)[8][4], const LaneOffsets& o,
                                              int wn, int g, uint32_t msel) {
  using L = Stage<true>;
  constexpr bool ROWS = GRAN_N == 0;
  float sxj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sxj[j] = ROWS ? 1.f : lds_ld<float>(st, o.sx + j * 64);

  v8i bx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 lo = lds_ld<uint4>(st, o.x0 + j * 2048);
    const uint4 hi = lds_ld<uint4>(st, o.x1 + j * 2048);
    bx[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  float s128[4];
  if (GRAN_N == 128) {
    const float swv = lds_ld<float>(st, L::SW_OFF + wn * 512);
#pragma unroll
    for (int j = 0; j < 4; ++j) s128[j] = sxj[j] * swv;
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 swr = make_float4(0.f, 0.f, 0.f, 0.f);
    if (GRAN_N == 1) swr = lds_ld<float4>(st, L::SW_OFF + (wn * 128 + i * 16 + 4 * g) * 4);
    v4f p[4];
    if (PACKED) {
      const uint4 av = lds_ld<uint4>(st, o.w0 + i * 1024);
      const int idx = lds_ld<int>(st, o.mt + i * 256);
      const v4i aa = {(int)av.x, (int)av.y, (int)av.z, (int)av.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (ROWS) acc[i][j] = mma_sparse_acc<I8>(aa, bx[j], acc[i][j], idx);
        else p[j] = mma_sparse<I8>(aa, bx[j], idx);
      }
    } else {
      const uint2 v0 = lds_ld<uint2>(st, o.w0 + i * 1024);
      const uint2 v1 = lds_ld<uint2>(st, o.w1 + i * 1024);
      const uint2 mw = lds_ld<uint2>(st, o.mt + i * 256);
      const int idx = (int)__builtin_amdgcn_perm(mw.y, mw.x, msel);
      const v4i aa = {(int)v0.x, (int)v0.y, (int)v1.x, (int)v1.y};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (ROWS) acc[i][j] = mma_sparse_acc<I8>(aa, bx[j], acc[i][j], idx);
        else p[j] = mma_sparse<I8>(aa, bx[j], idx);
      }
    }
    if (ROWS) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (GRAN_N == 128) {
        acc[i][j] += p[j] * s128[j];
      } else {
        acc[i][j][0] = fmaf(p[j][0] * swr.x, sxj[j], acc[i][j][0]);
        acc[i][j][1] = fmaf(p[j][1] * swr.y, sxj[j], acc[i][j][1]);
        acc[i][j][2] = fmaf(p[j][2] * swr.z, sxj[j], acc[i][j][2]);
        acc[i][j][3] = fmaf(p[j][3] * swr.w, sxj[j], acc[i][j][3]);
      }
    }
  }
}

// The same stage with the promotion folded into the accumulator (128-row W
// scale blocks, FP8 codes).  The accumulator of sub-tile column j is kept in
// units of the current K block's scale product c_j = sx[m, kb] * sw[kb]: per
// K block it is rescaled by c_prev / c_j (one multiply per element) and the
// SMFMAC adds the block's products into it directly, so no partial has to be
// cleared first.  On gfx950 the sparse instruction does not overlap VALU work,
// and clearing the partials costs as much as the multiplies, so this form
// needs about a third less VALU time per promoted unit.  The true sum is
// acc * c_last.  clo / chi collect the smallest and largest bit pattern of the
// scale products met; the result stands only if every product was a positive
// normal number within a factor 2^60 of the others (checked by the caller
// after the K loop), so that the rescaled sums stay far inside the fp32
// range.
template <bool PACKED>
__device__ __forceinline__ void compute_stage_scaled(const uint8_t* st, v4f (&acc)[8][4], const LaneOffsets& o,
                                                     int wn, int g, uint32_t msel, float (&cprev)[4], uint32_t& clo,
                                                     uint32_t& chi) {
  using L = Stage<true>;
  const float swv = lds_ld<float>(st, L::SW_OFF + wn * 512);
  float r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c = lds_ld<float>(st, o.sx + j * 64) * swv;
    r[j] = cprev[j] * __builtin_amdgcn_rcpf(c);
    cprev[j] = c;
    clo = min(clo, __float_as_uint(c));
    chi = max(chi, __float_as_uint(c));
  }
  v8i bx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 lo = lds_ld<uint4>(st, o.x0 + j * 2048);
    const uint4 hi = lds_ld<uint4>(st, o.x1 + j * 2048);
    bx[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v4i aa;
    int idx;
    if (PACKED) {
      const uint4 av = lds_ld<uint4>(st, o.w0 + i * 1024);
      idx = lds_ld<int>(st, o.mt + i * 256);
      aa = (v4i){(int)av.x, (int)av.y, (int)av.z, (int)av.w};
    } else {
      const uint2 v0 = lds_ld<uint2>(st, o.w0 + i * 1024);
      const uint2 v1 = lds_ld<uint2>(st, o.w1 + i * 1024);
      const uint2 mw = lds_ld<uint2>(st, o.mt + i * 256);
      idx = (int)__builtin_amdgcn_perm(mw.y, mw.x, msel);
      aa = (v4i){(int)v0.x, (int)v0.y, (int)v1.x, (int)v1.y};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mma_sparse_acc<false>(aa, bx[j], acc[i][j] * r[j], idx);
  }
}

// Scales constant along K: multiplies the wave's RI x 4 sub-tiles by
// sx (X row of the lane's column) * sw (W rows 16 i + 4 g .. + 3), read from
// a landed stage (every stage holds the same scales).  int8 sums are
// converted from their exact int32 first.
template <bool I8, int RI>
__device__ __forceinline__ void rows_scale(const uint8_t* st, v4f (&acc)[RI][4], uint32_t sx_off, uint32_t sw_off) {
  float sxj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sxj[j] = lds_ld<float>(st, sx_off + j * 64);
#pragma unroll
  for (int i = 0; i < RI; ++i) {
    const float4 w = lds_ld<float4>(st, sw_off + i * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4f v = acc[i][j];
      if (I8) {
        const v4i q = __builtin_bit_cast(v4i, v);
        v = (v4f){(float)q[0], (float)q[1], (float)q[2], (float)q[3]};
      }
      acc[i][j] = (v4f){v[0] * (w.x * sxj[j]), v[1] * (w.y * sxj[j]), v[2] * (w.z * sxj[j]), v[3] * (w.w * sxj[j])};
    }
    asm volatile("" ::: "memory");   // one row's W scales live at a time (all 128 results are)
  }
}

// ================================================ sparse kernel, 2 waves / SIMD
// 256 x 128 workgroup tile, 8 waves: two K groups of 4 waves in a 2 x 2 grid,
// each wave 128 n x 64 m = 8 x 4 sub-tiles of 16 x 16.  Group q multiplies the
// K blocks kb = 2 it + q, so two waves share every SIMD and one wave's LDS,
// barrier and matrix-core latencies hide behind the other's work.  A "double
// stage" holds K blocks 2 it and 2 it + 1 (two copies of the single-stage
// layout); two double stages alternate in LDS.  At the end the two groups add
// their partial tiles through LDS, each group finishing half of the rows, and
// the finished tile is staged in LDS once more for whole-row stores.
namespace x2 {
constexpr int HALF = Stage<true>::BYTES;   // one K block
constexpr int DBL = 2 * HALF;              // double stage
}  // namespace x2

#if SG_DEVICE_PASS
struct PlanX2 {
  uint32_t xo[4], wo[5], mo, so[2];
  uint32_t sdst[2];     // LDS offsets (within the double stage) of the two scale loads
  int sk[2];            // which scale: 0 = sx, 1 = sw
};

template <bool PACKED>
__device__ __forceinline__ PlanX2 make_plan_x2(const GemmArgs& a, int64_t n0, int64_t m0, int wave, int l) {
  using L = Stage<true>;
  PlanX2 p;
  // packed weights: 20 LDS slots of 1 KB per K block, 40 per double stage,
  // 5 per wave (q = 8 j + wave).  Slot s < 16 takes the values of the tile's
  // row block s (the first 1024 bytes of its chunk), slot 16 + s the index
  // words of row blocks 4 s .. 4 s + 3 (the last 256 bytes of their chunks).
  // Offsets are relative to the tile's first chunk of K block 0.
  const uint32_t rbs = (uint32_t)(a.K >> 7) * PK_CHUNK;     // bytes per row block
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int slot = (8 * j + wave) % 20;
    p.wo[j] = slot < 16 ? slot * rbs + l * 16
                        : (4 * (slot - 16) + (l >> 4)) * rbs + PK_META + (l & 15) * 16;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (8 * j + wave) & 15;      // 1 KB slot within the K block's X / W area
    {
      const int s = slot * 64 + l;
      const int r = s >> 3, c = (s & 7) ^ swz8(r);
      p.xo[j] = (uint32_t)(r * a.ldx + c * 16);
    }
    if (!PACKED) {
      const int s = slot * 64 + l;
      const int r = s >> 2, c = (s & 3) ^ ((r >> 1) & 3);
      p.wo[j] = (uint32_t)(r * a.ldw + c * 16);
    }
  }
  p.mo = PACKED ? 0u : (uint32_t)((((wave & 3) * 64) + l) * a.ldm);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sidx = 2 * wave + j, h = sidx >> 3, t = sidx & 7;
    if (t < 2 || t >= 6) {         // sx rows 64 t' .. 64 t' + 63 (t >= 6: the dummy copy)
      const int tp = t < 2 ? t : t - 6;
      const int64_t m = min(m0 + tp * 64 + l, a.M - 1);
      p.so[j] = (uint32_t)(((m >> a.gm_shift) * a.sx_sm) * 4);
      p.sdst[j] = h * x2::HALF + L::SX_OFF + (t < 2 ? 0 : BM * 4) + tp * 256;
      p.sk[j] = 0;
    } else {                       // sw rows 64 (t - 2) ..
      const int64_t n = min(n0 + (t - 2) * 64 + l, a.N - 1);
      p.so[j] = (uint32_t)(((n >> a.gn_shift) * a.sw_sn) * 4);
      p.sdst[j] = h * x2::HALF + L::SW_OFF + (t - 2) * 256;
      p.sk[j] = 1;
    }
  }
  return p;
}

// Loads K blocks kb0 and kb0 + 1 (clamped to the last block) into a double stage.
template <bool PACKED>
__device__ __forceinline__ void issue_double(uint8_t* st, const PlanX2& p, __amdgpu_buffer_rsrc_t rx,
                                             __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rm,
                                             __amdgpu_buffer_rsrc_t rsx, __amdgpu_buffer_rsrc_t rsw,
                                             const GemmArgs& a, int kb0, int KB, int wave) {
  using L = Stage<true>;
  const int kbh[2] = {min(kb0, KB - 1), min(kb0 + 1, KB - 1)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = j >> 1, slot = (8 * j + wave) & 15;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(st + h * x2::HALF + L::X_OFF + slot * 1024), 16,
                                             p.xo[j], kbh[h] * 128, 0, 0);
  }
  if (PACKED) {
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int q = 8 * j + wave, h = q / 20, slot = q % 20;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(st + h * x2::HALF + L::W_OFF + slot * 1024), 16,
                                               p.wo[j], kbh[h] * PK_CHUNK, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = j >> 1, slot = (8 * j + wave) & 15;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(st + h * x2::HALF + L::W_OFF + slot * 1024), 16,
                                               p.wo[j], kbh[h] * 64, 0, 0);
    }
    const int h = wave >> 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (lds_void*)(st + h * x2::HALF + L::M_OFF + (wave & 3) * 1024), 16,
                                             p.mo, kbh[h] * 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int h = (2 * wave + j) >> 3;
    if (p.sk[j] == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lds_void*)(st + p.sdst[j]), 4, p.so[j],
                                               (int)(kbh[h] * a.sx_sk * 4), 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)(st + p.sdst[j]), 4, p.so[j],
                                               (int)(kbh[h] * a.sw_sk * 4), 0, 0);
  }
}
#endif  // SG_DEVICE_PASS

#if SG_DEVICE_PASS
// One 256 x 128 output tile (n tile tn, m tile tm) of problem `a`.
template <bool I8, bool PACKED, int GRAN_N, bool OUT_BF16, bool OUT_T>
// db0, db1: the kernel's two double-stage LDS arrays (x2::DBL bytes each).
__device__ __forceinline__ void x2_tile(const GemmArgs& a, int tn, int tm, uint8_t* db0, uint8_t* db1) {
  const int64_t n0 = (int64_t)tn * BN, m0 = (int64_t)tm * BM;

  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = wave >> 2, w4 = wave & 3;
  const int wn = w4 & 1, wm = w4 >> 1;
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  const int NIT = (KB + 1) >> 1;

  const int64_t mrows = min((int64_t)BM, a.M - m0), nrows = min((int64_t)BN, a.N - n0);
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + m0 * a.ldx, (uint32_t)(mrows * a.ldx));
  // packed weights: the tile's row blocks are contiguous, KB * 1280 bytes each;
  // row blocks past N do not exist and read as zero
  const int64_t tile_rbs = min((int64_t)(BN / PK_ROWS), (a.N + PK_ROWS - 1) / PK_ROWS - (int64_t)tn * (BN / PK_ROWS));
  const __amdgpu_buffer_rsrc_t rw =
      PACKED ? rsrc(a.w + (int64_t)tn * (BN / PK_ROWS) * KB * PK_CHUNK, (uint32_t)(tile_rbs * KB * PK_CHUNK))
             : rsrc(a.w + n0 * a.ldw, (uint32_t)(nrows * a.ldw));
  const __amdgpu_buffer_rsrc_t rm = PACKED ? rw : rsrc(a.meta + n0 * a.ldm, (uint32_t)(nrows * a.ldm));
  const __amdgpu_buffer_rsrc_t rsx = rsrc(a.sx, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t rsw = rsrc(a.sw, 0xffffffffu);
  const PlanX2 plan = make_plan_x2<PACKED>(a, n0, m0, wave, l);
  const uint32_t msel = (g >> 1) ? 0x07060302u : 0x05040100u;
  const LaneOffsets lo = PACKED ? lane_offsets_packed(wn, wm, g, lr) : lane_offsets(wn, wm, g, lr);
  const uint32_t qoff = (uint32_t)q * x2::HALF;

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  issue_double<PACKED>(db0, plan, rx, rw, rm, rsx, rsw, a, 0, KB, wave);
  // The K loop: group q multiplies K block 2 it + q of double stage it.
  // SCALED: the rescaled-accumulator promotion (compute_stage_scaled).
  uint32_t clo = 0xffffffffu, chi = 0;
  auto kloop = [&](auto scaled_tag) {
    constexpr bool SCALED = decltype(scaled_tag)::value;
    float cprev[4] = {0.f, 0.f, 0.f, 0.f};   // scale product of the last K block multiplied (0: none yet)
    for (int it0 = 0; it0 < NIT; it0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = it0 + u;
        if (it < NIT) {
          wait_vmcnt<0>();
          __syncthreads();
          if (it + 1 < NIT)
            issue_double<PACKED>(u == 0 ? db1 : db0, plan, rx, rw, rm, rsx, rsw, a, 2 * (it + 1), KB, wave);
          if (2 * it + q < KB) {
            if constexpr (SCALED)
              compute_stage_scaled<PACKED>((u == 0 ? db0 : db1) + qoff, acc, lo, wn, g, msel, cprev, clo, chi);
            else
              compute_stage<GRAN_N, PACKED, I8>((u == 0 ? db0 : db1) + qoff, acc, lo, wn, g, msel);
          }
        }
      }
    }
    if constexpr (SCALED) {   // back to true values: acc * c_last
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] *= cprev[j];
    }
  };
  // FP8 codes with 128-row W scale blocks take the rescaled-accumulator
  // promotion; if any wave met a scale product that is not positive and
  // normal, or products more than 2^60 apart, the whole tile is computed
  // again with the zero-and-FMA promotion.  The last double stage issues no
  // loads, so nothing is in flight when the K loop ends.
  if constexpr (GRAN_N == 128 && !I8) {
    kloop(std::true_type{});
    const bool ok = chi < clo ||   // no K block of this wave
                    (clo >= 0x00800000u && chi <= 0x7f7fffffu && (chi >> 23) - (clo >> 23) <= 60u);
    if (__syncthreads_or(!ok)) {   // (also: every wave is done with both double stages)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      issue_double<PACKED>(db0, plan, rx, rw, rm, rsx, rsw, a, 0, KB, wave);
      kloop(std::false_type{});
    }
  } else {
    kloop(std::false_type{});
  }

  // Add the two groups' partial tiles: group 0 finishes sub-tile rows i < 4,
  // group 1 rows i >= 4; each hands the other half to its partner through LDS.
  // (Uniform branches with constant indices keep acc in registers.)
  __syncthreads();
  if (q == 0) {
    xchg_out<4>(reinterpret_cast<float4*>(db0), acc, w4, l);
  } else {
    xchg_out<0>(reinterpret_cast<float4*>(db1), acc, w4, l);
  }
  __syncthreads();
  // Scales constant along K: the second half of the last double stage holds
  // them (a landed K block, or the copy of the last one), above the bytes the
  // exchange and the staged tile use.
  constexpr int SCALE = GRAN_N == 0 ? (I8 ? 2 : 1) : 0;
  static_assert(x2::HALF + Stage<true>::SX_OFF >= 65536 &&
                x2::HALF + Stage<true>::SX_OFF >= OutTile<OUT_BF16, OUT_T, x2::DBL>::RPH *
                                                       OutTile<OUT_BF16, OUT_T, x2::DBL>::PITCH,
                "scales must survive the exchange and the staged tile");
  const uint8_t* const sst = ((NIT - 1) & 1 ? db1 : db0) + x2::HALF;
  const float* const sxp = reinterpret_cast<const float*>(sst + Stage<true>::SX_OFF) + wm * 64 + lr;
  const float* const swp = reinterpret_cast<const float*>(sst + Stage<true>::SW_OFF) + wn * 128 + 4 * g;
  const float* const bias = a.bias ? a.bias + n0 : nullptr;
  const int nlim = (int)nrows;
  if (q == 0)
    x2_finish<0, OUT_BF16, OUT_T, x2::DBL, SCALE>(db1, db0, db1, acc, w4, l, wn, wm, g, lr, sxp, swp, bias, nlim);
  else
    x2_finish<1, OUT_BF16, OUT_T, x2::DBL, SCALE>(db0, db0, db1, acc, w4, l, wn, wm, g, lr, sxp, swp, bias, nlim);
  __syncthreads();
  store_staged<OUT_BF16, OUT_T, x2::DBL>(a, db0, db1, m0, n0, t);
}
#endif  // SG_DEVICE_PASS

template <bool I8, bool PACKED, int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_sparse_x2(GemmArgs a, int tiles_m, int tiles_n) {
#if SG_DEVICE_PASS
  to_batch(a);
  int tn, tm;
  tile_coords(tiles_m, tiles_n, tn, tm);
  __shared__ __attribute__((aligned(1024))) uint8_t db0[x2::DBL];
  __shared__ __attribute__((aligned(1024))) uint8_t db1[x2::DBL];
  x2_tile<I8, PACKED, GRAN_N, OUT_BF16, OUT_T>(a, tn, tm, db0, db1);
#endif  // SG_DEVICE_PASS
}

// ============================= large-M 2:4 kernel, weight in registers
// Packed weights, FP8 codes.  Workgroup tile 256 W rows (n) x 128 X rows (m),
// 8 waves: two K groups of four.  Wave (q, wn) owns W rows 64 wn .. 64 wn + 63
// (four 16-row blocks) and all 128 X rows (eight 16-column sub-tiles) and
// multiplies the K blocks kb = q (mod 2).  No other wave needs its W rows, so
// it loads them from the packed weight straight into registers: a lane's
// 16-byte A operand and 4-byte index word of one row block are one dwordx4
// and one dword load, coalesced over the wave, issued one period (two K
// blocks) ahead.  X, which the four waves of a group share, goes through LDS:
// two arrays of four K blocks (per K block 16 KB of codes with 16-byte chunks
// swizzled by row, the 128 X scales and the 256 W-row scales), filled by
// buffer loads that write LDS.  While one array is multiplied the other
// one's loads are in flight, and one barrier per four K blocks joins the
// waves.  Against the 2 x 2 wave grid of k_gemm_sparse_x2 this halves the
// bytes written into LDS per K block and doubles the time an LDS load has
// to land.  At the end the two groups add their partial tiles through LDS
// (group q finishes sub-tile columns 4 q .. 4 q + 3) and the finished tile is
// staged for whole-row stores.
namespace wr {
constexpr int KPA = 4;                       // K blocks per LDS array
constexpr int XB = BM * 128;                 // X codes of one K block
constexpr int SX_OFF = XB;                   // 128 X scales
constexpr int SW_OFF = XB + BM * 4;          // 256 W-row scales
constexpr int SPARE_OFF = SW_OFF + BN * 4;   // spare slot for the scale loads of waves 6, 7
constexpr int KBYTES = SPARE_OFF + BM * 4;   // one K block
constexpr int ARR = KPA * KBYTES;            // one array
}  // namespace wr

#if SG_DEVICE_PASS
// A wave's W operands of one K block: row block rb = 4 wn + i, i = 0..3.
struct WrRegs {
  v4i v[4];
  int idx[4];
};

// Loads row block 4 wn + i of K block kb (clamped to the last block) into
// registers: two buffer loads.
__device__ __forceinline__ void wr_load_w1(WrRegs& w, int i, __amdgpu_buffer_rsrc_t rw, uint32_t voff_v,
                                           uint32_t voff_m, int wn, int kb, int KB) {
  const int so = ((4 * wn + i) * KB + min(kb, KB - 1)) * PK_CHUNK;
  w.v[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, voff_v, so, 0));
  w.idx[i] = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(rw, voff_m, so, 0));
}

// All four row blocks (exactly wr::NW loads).
__device__ __forceinline__ void wr_load_w(WrRegs& w, __amdgpu_buffer_rsrc_t rw, uint32_t voff_v, uint32_t voff_m,
                                          int wn, int kb, int KB) {
#pragma unroll
  for (int i = 0; i < 4; ++i) wr_load_w1(w, i, rw, voff_v, voff_m, wn, kb, KB);
}

// Issues the LDS loads of K blocks 4 P .. 4 P + 3 into an array: every wave
// two 1 KB slices of X codes per K block and one scale load (waves 0, 1: X
// scales; waves 2 .. 5: W-row scales; waves 6, 7: the X scales again, into a
// spare slot), so that every wave issues the same number of loads on every
// path (the compiler's and this kernel's load counting rely on it).  K
// blocks at or past KB go through descriptors of zero records: no memory
// access, zeros written.
struct WrPlan {
  uint32_t xo[2];   // X slice source offsets (K block 0)
  uint32_t so;      // scale source offset (K block 0), bytes
  uint32_t sdst;    // scale destination within a K block
  bool sw;          // the scale is a W-row scale (else an X scale)
};

__device__ __forceinline__ WrPlan wr_plan(const GemmArgs& a, int64_t n0, int64_t m0, int wave, int l) {
  WrPlan p;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = (8 * j + wave) * 64 + l;            // 16-byte position in the K block's X area
    const int r = s >> 3, c = (s & 7) ^ swz8(r);
    p.xo[j] = (uint32_t)(r * a.ldx + c * 16);
  }
  if (wave >= 2 && wave < 6) {
    const int64_t n = min(n0 + (wave - 2) * 64 + l, a.N - 1);
    p.so = (uint32_t)(((n >> a.gn_shift) * a.sw_sn) * 4);
    p.sdst = wr::SW_OFF + (wave - 2) * 256;
    p.sw = true;
  } else {
    const int h = wave & 1;
    const int64_t m = min(m0 + h * 64 + l, a.M - 1);
    p.so = (uint32_t)(((m >> a.gm_shift) * a.sx_sm) * 4);
    p.sdst = (wave < 2 ? wr::SX_OFF : wr::SPARE_OFF) + h * 256;
    p.sw = false;
  }
  return p;
}

// The loads of K block 4 P + k (three per wave).
__device__ __forceinline__ void wr_issue_x1(uint8_t* arr, const WrPlan& p, __amdgpu_buffer_rsrc_t rx,
                                            __amdgpu_buffer_rsrc_t rs, int64_t s_sk, int P, int k, int KB, int wave) {
  const __amdgpu_buffer_rsrc_t none = rsrc(nullptr, 0);
  const int kb = wr::KPA * P + k;
  const bool ok = kb < KB;
  const int kbc = ok ? kb : 0;
  uint8_t* st = arr + k * wr::KBYTES;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ok ? rx : none, (lds_void*)(st + (8 * j + wave) * 1024), 16, p.xo[j],
                                             kbc * 128, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ok ? rs : none, (lds_void*)(st + p.sdst), 4, p.so, (int)(kbc * s_sk * 4),
                                           0, 0);
}

__device__ __forceinline__ void wr_issue_x(uint8_t* arr, const WrPlan& p, __amdgpu_buffer_rsrc_t rx,
                                           __amdgpu_buffer_rsrc_t rs, int64_t s_sk, int P, int KB, int wave) {
#pragma unroll
  for (int k = 0; k < wr::KPA; ++k) wr_issue_x1(arr, p, rx, rs, s_sk, P, k, KB, wave);
}

// Multiplies one K block (stage st of an array, W operands w) into the
// wave's 4 x 8 sub-tiles; issue(j) is called before sub-tile column j.  SCALED: the rescaled-accumulator promotion of
// compute_stage_scaled; else GRAN_N = 128 promotes each partial from zero,
// and GRAN_N = 0 accumulates in the matrix core (scales applied at the end;
// int8 codes (I8) keep the exact int32 sum in the accumulator's registers).
template <int GRAN_N, bool SCALED, bool I8, typename Issue>
__device__ __forceinline__ void wr_compute(const uint8_t* st, const WrRegs& w, v4f (&acc)[4][8], uint32_t x0,
                                           uint32_t x1, uint32_t sxo, int wn, float (&cprev)[8], uint32_t& clo,
                                           uint32_t& chi, Issue&& issue) {
  float swv = 1.f;
  if (GRAN_N == 128) swv = lds_ld<float>(st, wr::SW_OFF + wn * 256);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    issue(j);   // a share of the loads for later K blocks, spread over the multiplies
    const uint4 lo = lds_ld<uint4>(st, x0 + j * 2048);
    const uint4 hi = lds_ld<uint4>(st, x1 + j * 2048);
    const v8i bx = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    if constexpr (GRAN_N == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mma_sparse_acc<I8>(w.v[i], bx, acc[i][j], w.idx[i]);
    } else {
      const float c = lds_ld<float>(st, sxo + j * 64) * swv;
      if constexpr (SCALED) {
        const float r = cprev[j] * __builtin_amdgcn_rcpf(c);
        cprev[j] = c;
        clo = min(clo, __float_as_uint(c));   // the range of the products seen, checked after the K loop
        chi = max(chi, __float_as_uint(c));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mma_sparse_acc<false>(w.v[i], bx, acc[i][j] * r, w.idx[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] += mma_sparse<I8>(w.v[i], bx, w.idx[i]) * c;
      }
    }
  }
}

// Group Q's half of the epilogue: adds the partner group's partials of
// sub-tile columns 4 Q .. 4 Q + 3 (in buffer src), applies scales constant
// along K (GRAN_N = 0) and the bias, and stages the values in t0 / t1.
template <int Q, int GRAN_N, bool OUT_BF16, bool OUT_T, bool I8>
__device__ __forceinline__ void wr_finish(const GemmArgs& a, const uint8_t* src, uint8_t* t0, uint8_t* t1,
                                          const v4f (&acc)[4][8], int wn, int l, int64_t m0, int64_t n0) {
  const int g = l >> 4, lr = l & 15;
  float4 part[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) part[k] = reinterpret_cast<const float4*>(src)[((wn * 16 + k) << 6) + l];
  float sxj[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (GRAN_N == 0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      sxj[jj] = a.sx[(min(m0 + 16 * (4 * Q + jj) + lr, a.M - 1) >> a.gm_shift) * a.sx_sm];
  }
  __syncthreads();   // every wave holds its partner's partials: the buffers may be overwritten
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nl = wn * 64 + 16 * i + 4 * g;
    float sw[4] = {1.f, 1.f, 1.f, 1.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = min(n0 + nl + e, a.N - 1);
      if (GRAN_N == 0) sw[e] = a.sw[(n >> a.gn_shift) * a.sw_sn];
      if (a.bias) bv[e] = a.bias[n];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float4 o = part[i * 4 + jj];
      const v4f av = acc[i][4 * Q + jj];
      float v[4] = {av[0] + o.x, av[1] + o.y, av[2] + o.z, av[3] + o.w};
      if constexpr (I8 && GRAN_N == 0) {   // the two K groups' exact int32 sums, added before the conversion
        const v4i ai = __builtin_bit_cast(v4i, av);
        const int4 oi = __builtin_bit_cast(int4, o);
        v[0] = (float)(ai[0] + oi.x); v[1] = (float)(ai[1] + oi.y);
        v[2] = (float)(ai[2] + oi.z); v[3] = (float)(ai[3] + oi.w);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = v[e] * (sw[e] * sxj[jj]) + bv[e];
      stage_quad<OUT_BF16, OUT_T, wr::ARR>(t0, t1, nl, 16 * (4 * Q + jj) + lr, v);
    }
  }
}

// Sends sub-tile columns 4 (1 - Q) .. of the wave's partials to the partner group.
template <int Q>
__device__ __forceinline__ void wr_send(float4* dst, const v4f (&acc)[4][8], int wn, int l) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const v4f v = acc[i][4 * (1 - Q) + jj];
      dst[((wn * 16 + i * 4 + jj) << 6) + l] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <int GRAN_N, bool OUT_BF16, bool OUT_T, bool I8 = false>
__device__ __forceinline__ void wr_tile(const GemmArgs& a, int tn, int tm, uint8_t* arr0, uint8_t* arr1) {
  const int64_t n0 = (int64_t)tn * BN, m0 = (int64_t)tm * BM;
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = wave >> 2, wn = wave & 3;
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  const int NP = (KB + wr::KPA - 1) / wr::KPA;

  const int64_t mrows = min((int64_t)BM, a.M - m0);
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + m0 * a.ldx, (uint32_t)(mrows * a.ldx));
  const int64_t tile_rbs = min((int64_t)(BN / PK_ROWS), (a.N + PK_ROWS - 1) / PK_ROWS - (int64_t)tn * (BN / PK_ROWS));
  const __amdgpu_buffer_rsrc_t rw =
      rsrc(a.w + (int64_t)tn * (BN / PK_ROWS) * KB * PK_CHUNK, (uint32_t)(tile_rbs * KB * PK_CHUNK));
  const WrPlan plan = wr_plan(a, n0, m0, wave, l);
  const __amdgpu_buffer_rsrc_t rs = plan.sw ? rsrc(a.sw, 0xffffffffu) : rsrc(a.sx, 0xffffffffu);
  const int64_t s_sk = plan.sw ? a.sw_sk : a.sx_sk;
  const uint32_t voff_v = (uint32_t)pk_val_off(lr, g), voff_m = (uint32_t)(PK_META + pk_meta_word(lr, g));
  const uint32_t x0 = lr * 128 + (((2 * g) ^ swz8(lr)) << 4), x1 = lr * 128 + (((2 * g + 1) ^ swz8(lr)) << 4);
  const uint32_t sxo = wr::SX_OFF + lr * 4;

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // W operands: wa / wc for the first K block of even / odd super-periods,
  // wb for the second.  A wave's loads complete in issue order, so every W
  // load is issued where nothing it must not wait for lies behind it: during
  // a super-period's first K block come, column by column, the W of its
  // second K block and the W of the next super-period's first K block (both
  // needed one and two K blocks later), then the next X array.
  WrRegs wa, wb, wc;
  auto start = [&]() {   // K blocks 0 and 1 of X, the first W, then K blocks 2 and 3 of X
    wr_issue_x1(arr0, plan, rx, rs, s_sk, 0, 0, KB, wave);
    wr_issue_x1(arr0, plan, rx, rs, s_sk, 0, 1, KB, wave);
    wr_load_w(wa, rw, voff_v, voff_m, wn, q, KB);
    wr_issue_x1(arr0, plan, rx, rs, s_sk, 0, 2, KB, wave);
    wr_issue_x1(arr0, plan, rx, rs, s_sk, 0, 3, KB, wave);
  };

  // Super-period P: K blocks 4 P .. 4 P + 3 in array P % 2; this wave
  // multiplies 4 P + q and 4 P + 2 + q.  clo / chi: bit patterns of the
  // smallest and largest scale product the scaled promotion met.
  uint32_t clo = 0xffffffffu, chi = 0;
  auto kloop = [&](auto scaled_tag) {
    constexpr bool SCALED = decltype(scaled_tag)::value;
    float cprev[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // The loads are spread over the multiplies of the first K block (issued
    // all at once, a wave stalls until the memory pipeline has taken them).
    auto period = [&](uint8_t* cur, uint8_t* nxt, WrRegs& w0, WrRegs& w0next, int P) {
      if (P == 0) wait_vmcnt<6>();   // the first super-period: X K blocks 2, 3 (6 loads) may still fly
      else wait_vmcnt<0>();
      lds_barrier();
      auto issue0 = [&](int j) {
        if (j < 4) wr_load_w1(wb, j, rw, voff_v, voff_m, wn, 4 * P + 2 + q, KB);
        else wr_issue_x1(nxt, plan, rx, rs, s_sk, P + 1, j - 4, KB, wave);   // past the last K block: zeros
      };
      auto issue1 = [&](int j) {
        if (j < 4) wr_load_w1(w0next, j, rw, voff_v, voff_m, wn, 4 * (P + 1) + q, KB);
      };
      if (4 * P + q < KB) {
        wr_compute<GRAN_N, SCALED, I8>(cur + q * wr::KBYTES, w0, acc, x0, x1, sxo, wn, cprev, clo, chi, issue0);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) issue0(j);
      }
      if (P == 0) {   // K blocks 2, 3 of X: issued before the 20 loads of the first K block's columns
        wait_vmcnt<20>();
        lds_barrier();
      }
      if (4 * P + 2 + q < KB) {
        wr_compute<GRAN_N, SCALED, I8>(cur + (2 + q) * wr::KBYTES, wb, acc, x0, x1, sxo, wn, cprev, clo, chi,
                                       issue1);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) issue1(j);
      }
    };
    for (int P = 0; P < NP; P += 2) {
      period(arr0, arr1, wa, wc, P);
      if (P + 1 < NP) period(arr1, arr0, wc, wa, P + 1);
    }
    if constexpr (SCALED) {   // back to true values: acc * c_last
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] *= cprev[j];
    }
  };
  start();
  if constexpr (GRAN_N == 128 && !I8) {
    // The rescaled promotion first; if any wave met a scale product that is
    // not positive and normal, or products more than 2^60 apart, the whole
    // tile is computed again with the zero-and-FMA promotion.
    kloop(std::true_type{});
    const bool ok = chi < clo ||   // no K block of this wave
                    (clo >= 0x00800000u && chi <= 0x7f7fffffu && (chi >> 23) - (clo >> 23) <= 60u);
    wait_vmcnt<0>();   // the last (unused) loads of every wave have landed before the barrier
    if (__syncthreads_or(!ok)) {   // (also: every wave is done with both arrays)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      start();
      kloop(std::false_type{});
      wait_vmcnt<0>();
      __syncthreads();
    }
  } else {
    kloop(std::false_type{});
    wait_vmcnt<0>();   // the last (unused) W loads
    __syncthreads();   // every wave is done with both arrays
  }
  if (q == 0) wr_send<0>(reinterpret_cast<float4*>(arr1), acc, wn, l);
  else wr_send<1>(reinterpret_cast<float4*>(arr0), acc, wn, l);
  __syncthreads();
  if (q == 0) wr_finish<0, GRAN_N, OUT_BF16, OUT_T, I8>(a, arr0, arr0, arr1, acc, wn, l, m0, n0);
  else wr_finish<1, GRAN_N, OUT_BF16, OUT_T, I8>(a, arr1, arr0, arr1, acc, wn, l, m0, n0);
  __syncthreads();
  store_staged<OUT_BF16, OUT_T, wr::ARR>(a, arr0, arr1, m0, n0, t);
}
#endif  // SG_DEVICE_PASS

template <int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_sparse_wr(GemmArgs a, int tiles_m, int tiles_n) {
#if SG_DEVICE_PASS
  to_batch(a);
  int tn, tm;
  tile_coords(tiles_m, tiles_n, tn, tm);
  __shared__ __attribute__((aligned(1024))) uint8_t arr0[wr::ARR];
  __shared__ __attribute__((aligned(1024))) uint8_t arr1[wr::ARR];
  wr_tile<GRAN_N, OUT_BF16, OUT_T>(a, tn, tm, arr0, arr1);
#endif  // SG_DEVICE_PASS
}

// The same tile on int8 x int8 codes (packed int8 weight): the zero-and-FMA
// promotion of exact int32 partials per K block, or, with scales constant
// along K, one exact int32 sum per output (the launcher takes
// k_gemm_sparse_x2 for that case, measured 0.7 us faster at 2048 x 4096 x 4096).
template <int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_sparse_wr_i8(GemmArgs a, int tiles_m, int tiles_n) {
#if SG_DEVICE_PASS
  to_batch(a);
  int tn, tm;
  tile_coords(tiles_m, tiles_n, tn, tm);
  __shared__ __attribute__((aligned(1024))) uint8_t arr0[wr::ARR];
  __shared__ __attribute__((aligned(1024))) uint8_t arr1[wr::ARR];
  wr_tile<GRAN_N, OUT_BF16, OUT_T, true>(a, tn, tm, arr0, arr1);
#endif  // SG_DEVICE_PASS
}

// Grouped problems (different M per group, one packed weight per group): the
// groups' rows follow each other in X, in the scales of X and in Y; a launch
// covers rows row_off[g] .. row_end[g] - 1 of group g (all of them, or the
// part its kernel takes), the large-M kernel as m tiles numbered from
// tile_start[g] (tiles_n n tiles per m tile).
constexpr int MAX_GROUPS = 64;
struct GroupTable {
  int G, tiles_n;
  int tile_start[MAX_GROUPS + 1];
  int64_t row_off[MAX_GROUPS + 1];
  int64_t row_end[MAX_GROUPS];
};

#if SG_DEVICE_PASS
// Points a at group g's part of a grouped problem: rows row_off[g] ..
// row_end[g] - 1 of X, its scales and Y (columns of Y^T), the group's packed
// weight, W scales and bias.
template <bool OUT_BF16, bool OUT_T>
__device__ __forceinline__ void group_args(GemmArgs& a, const GroupTable& gt, int g) {
  const int64_t r0 = gt.row_off[g];
  a.M = gt.row_end[g] - r0;
  a.x += r0 * a.ldx;
  a.sx += r0 * a.sx_sm;
  a.y = static_cast<uint8_t*>(a.y) + (OUT_T ? r0 : r0 * a.ldy) * (OUT_BF16 ? 2 : 4);
  a.w += g * a.bw;
  a.sw += g * a.bsw;
  if (a.bias) a.bias += g * a.bbs;
}

// Large tile b (in the XCD order over T tiles) of a grouped problem (packed
// FP8 weights): the register-weight tile for 128-row W scale blocks and for
// scales constant along K, else the two-operand LDS tile.  db0 / db1 hold at
// least x2::DBL bytes each (more than the register-weight tile's arrays).
template <int GRAN_N, bool OUT_BF16, bool OUT_T>
__device__ __forceinline__ void grouped_tile(GemmArgs a, const GroupTable& gt, int T, uint8_t* db0, uint8_t* db1) {
  static_assert(wr::ARR <= x2::DBL, "the register-weight tile's arrays fit the LDS tile's");
  const int b = xcd_order(blockIdx.x, T);
  int g = 0;
  while (g + 1 < gt.G && gt.tile_start[g + 1] <= b) ++g;   // uniform; empty groups are skipped
  const int tiles_m = (gt.tile_start[g + 1] - gt.tile_start[g]) / gt.tiles_n;
  int tn, tm;
  tile_of(b - gt.tile_start[g], tiles_m, gt.tiles_n, tn, tm);
  group_args<OUT_BF16, OUT_T>(a, gt, g);
  if constexpr (GRAN_N == 128 || GRAN_N == 0)
    wr_tile<GRAN_N, OUT_BF16, OUT_T>(a, tn, tm, db0, db1);
  else
    x2_tile<false, true, GRAN_N, OUT_BF16, OUT_T>(a, tn, tm, db0, db1);
}
#endif  // SG_DEVICE_PASS

template <int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_sparse_grouped(GemmArgs a, GroupTable gt) {
#if SG_DEVICE_PASS
  __shared__ __attribute__((aligned(1024))) uint8_t db0[x2::DBL];
  __shared__ __attribute__((aligned(1024))) uint8_t db1[x2::DBL];
  grouped_tile<GRAN_N, OUT_BF16, OUT_T>(a, gt, gt.tile_start[gt.G], db0, db1);
#endif  // SG_DEVICE_PASS
}

// ================================================= dense kernel, 2 waves / SIMD
// Workgroup tile 256 W rows (n) x 128 X rows (m), 8 waves in a 4 (n) x 2 (m)
// grid, each wave 64 n x 64 m = 4 x 4 sub-tiles of 16 x 16.  One 128-wide K
// block per stage (the single-stage layout above), three stages in LDS: while
// all waves multiply stage kb, stages kb + 1 and kb + 2 are in flight.  Every
// wave issues the same number of loads per stage (two 1 KB X slots, four
// 1 KB W slots, one 256-byte scale load), so a wave waits for a stage by
// counting its own loads.  The finished tile is staged in LDS and stored in
// whole rows.
namespace d8 {
constexpr int NST = 3;
constexpr int LOADS = 7;                       // buffer loads per wave per stage
constexpr int BYTES = Stage<false>::BYTES;
}  // namespace d8

#if SG_DEVICE_PASS
struct PlanD8 {
  uint32_t xo[2], wo[4], so, sdst;
  int sk;   // 0: sx, 1: sw
};

__device__ __forceinline__ PlanD8 make_plan_d8(const GemmArgs& a, int64_t n0, int64_t m0, int wave, int l) {
  using L = Stage<false>;
  PlanD8 p;
#pragma unroll
  for (int j = 0; j < 2; ++j) {               // X slot 8 j + wave: rows 8 slot .. 8 slot + 7
    const int s = (8 * j + wave) * 64 + l;
    const int r = s >> 3, c = (s & 7) ^ swz8(r);
    p.xo[j] = (uint32_t)(r * a.ldx + c * 16);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {               // W slot 8 j + wave
    const int s = (8 * j + wave) * 64 + l;
    const int r = s >> 3, c = (s & 7) ^ swz8(r);
    p.wo[j] = (uint32_t)(r * a.ldw + c * 16);
  }
  // waves 0, 1: sx rows 64 w ..; waves 2 - 5: sw rows 64 (w - 2) ..; waves 6, 7
  // load sx rows again into the dummy copy.  Rows past M / N are clamped.
  if (wave < 2 || wave >= 6) {
    const int tp = wave < 2 ? wave : wave - 6;
    const int64_t m = min(m0 + tp * 64 + l, a.M - 1);
    p.so = (uint32_t)(((m >> a.gm_shift) * a.sx_sm) * 4);
    p.sdst = L::SX_OFF + (wave < 2 ? 0 : BM * 4) + tp * 256;
    p.sk = 0;
  } else {
    const int64_t n = min(n0 + (wave - 2) * 64 + l, a.N - 1);
    p.so = (uint32_t)(((n >> a.gn_shift) * a.sw_sn) * 4);
    p.sdst = L::SW_OFF + (wave - 2) * 256;
    p.sk = 1;
  }
  return p;
}

// The dense ring issues its loads through inline assembly (the same two
// instructions the buffer-load-to-LDS builtin produces: M0 = LDS byte address,
// then the load).  The compiler then does not track them, so it adds no
// waits of its own before LDS reads of other stages (its tracking of three
// ring buffers across the unrolled loop is not precise and waited for every
// load in flight); the explicit per-stage load counts carry the ordering.
typedef int rsrc_v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_v rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return (rsrc_v){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, (int)RSRC_WORD3};
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}

__device__ __forceinline__ void dma16(const rsrc_v& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const rsrc_v& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}

__device__ __forceinline__ void issue_d8(uint8_t* st, const PlanD8& p, const rsrc_v& rx, const rsrc_v& rw,
                                         const rsrc_v& rsx, const rsrc_v& rsw, const GemmArgs& a, int kb,
                                         int wave) {
  using L = Stage<false>;
  const uint32_t base = lds_addr(st);
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(rx, base + L::X_OFF + (8 * j + wave) * 1024, p.xo[j], (uint32_t)kb * 128);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16(rw, base + L::W_OFF + (8 * j + wave) * 1024, p.wo[j], (uint32_t)kb * 128);
  if (p.sk == 0) dma4(rsx, base + p.sdst, p.so, (uint32_t)(kb * a.sx_sk * 4));
  else dma4(rsw, base + p.sdst, p.so, (uint32_t)(kb * a.sw_sk * 4));
}
#endif  // SG_DEVICE_PASS

// Lane-constant LDS offsets: X row wm*64 + lr and W row wn*64 + lr, the two
// 16-byte chunks of lane group g (sub-tiles are 2 KB apart), the X scale of
// the lane's row and the W scales of the wave's rows.
struct LaneD8 {
  uint32_t x0, x1, w0, w1, sx, sw;
};

__device__ __forceinline__ LaneD8 lane_d8(int wn, int wm, int g, int lr) {
  using L = Stage<false>;
  LaneD8 o;
  const int xr = wm * 64 + lr, wr = wn * 64 + lr;
  o.x0 = L::X_OFF + xr * 128 + (((2 * g) ^ swz8(lr)) << 4);
  o.x1 = L::X_OFF + xr * 128 + (((2 * g + 1) ^ swz8(lr)) << 4);
  o.w0 = L::W_OFF + wr * 128 + (((2 * g) ^ swz8(lr)) << 4);
  o.w1 = L::W_OFF + wr * 128 + (((2 * g + 1) ^ swz8(lr)) << 4);
  o.sx = L::SX_OFF + xr * 4;
  o.sw = L::SW_OFF + (wn * 64 + 4 * g) * 4;
  return o;
}

// One stage's operands of a wave in registers: the A (W) and B (X) fragments
// of its 4 x 4 sub-tiles and the scales.
struct FragD8 {
  v8i a[4], b[4];
  float sx[4];    // X scales of the lane's rows (per-row W scales), or
                  // sx * sw, the whole scale of sub-tile column j (128-row W scale blocks)
  float4 sw[4];   // W scales of rows 16 i + 4 g .. + 3 (per-row W scales only)
};

__device__ __forceinline__ v8i ld_frag(const uint8_t* st, uint32_t o0, uint32_t o1) {
  const uint4 lo = lds_ld<uint4>(st, o0);
  const uint4 hi = lds_ld<uint4>(st, o1);
  return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// X fragments and scales of a stage.
template <int GRAN_N>
__device__ __forceinline__ void read_b_d8(const uint8_t* st, const LaneD8& o, int wn, FragD8& f) {
  using L = Stage<false>;
  const float swv = GRAN_N == 128 ? lds_ld<float>(st, L::SW_OFF + wn * 256) : 1.f;   // the wave's 64 rows share it
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (GRAN_N != 0) f.sx[j] = lds_ld<float>(st, o.sx + j * 64) * swv;
    f.b[j] = ld_frag(st, o.x0 + j * 2048, o.x1 + j * 2048);
  }
}

// W fragment (and per-row W scales) of sub-tile row i of a stage.
template <int GRAN_N>
__device__ __forceinline__ void read_a_d8(const uint8_t* st, const LaneD8& o, int i, FragD8& f) {
  f.a[i] = ld_frag(st, o.w0 + i * 2048, o.w1 + i * 2048);
  if (GRAN_N == 1) f.sw[i] = lds_ld<float4>(st, o.sw + i * 64);
}

// Promotes sub-tile row i.  The empty asm pins each result at this point:
// otherwise the compiler sinks the promotions past the next barrier (they
// are register-only arithmetic), keeping 64 MFMA results alive across it and
// bunching two stages' promotions into one.
template <int GRAN_N>
__device__ __forceinline__ void promote_d8(v4f (&acc)[4], const v4f (&p)[4], const FragD8& f, int i) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (GRAN_N == 128) {
      acc[j] += p[j] * f.sx[j];
    } else {
      acc[j][0] = fmaf(p[j][0] * f.sw[i].x, f.sx[j], acc[j][0]);
      acc[j][1] = fmaf(p[j][1] * f.sw[i].y, f.sx[j], acc[j][1]);
      acc[j][2] = fmaf(p[j][2] * f.sw[i].z, f.sx[j], acc[j][2]);
      acc[j][3] = fmaf(p[j][3] * f.sw[i].w, f.sx[j], acc[j][3]);
    }
    asm volatile("" : "+v"(acc[j]));
  }
}

// Multiplies stage `cur` (in registers) into the wave's 4 x 4 sub-tiles and
// promotes (or, with scales constant along K, GRAN_N = 0, accumulates in the
// matrix core), while reading the next stage into `nxt`: its X fragments
// first, then the W fragment of row i once row i of `cur` is multiplied, so
// the two register sets can share the W registers.
template <int GRAN_N>
__device__ __forceinline__ void step_d8(const FragD8& cur, FragD8& nxt, const uint8_t* st_next, const LaneD8& o,
                                        int wn, v4f (&acc)[4][4]) {
  read_b_d8<GRAN_N>(st_next, o, wn, nxt);
  v4f p[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (GRAN_N == 0) acc[i][j] = mma_dense_acc(cur.a[i], cur.b[j], acc[i][j]);
      else p[i & 1][j] = mma_dense(cur.a[i], cur.b[j]);
    }
    if (GRAN_N != 0 && i > 0) promote_d8<GRAN_N>(acc[i - 1], p[(i - 1) & 1], cur, i - 1);
    read_a_d8<GRAN_N>(st_next, o, i, nxt);
  }
  if (GRAN_N != 0) promote_d8<GRAN_N>(acc[3], p[1], cur, 3);
}

// Multiplies one stage's fragments into the wave's 4 x 4 sub-tiles and promotes.
template <int GRAN_N>
__device__ __forceinline__ void mma_d8(const FragD8& f, v4f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f p = mma_dense(f.a[i], f.b[j]);
      if (GRAN_N == 128) {
        acc[i][j] += p * f.sx[j];
      } else {
        acc[i][j][0] = fmaf(p[0] * f.sw[i].x, f.sx[j], acc[i][j][0]);
        acc[i][j][1] = fmaf(p[1] * f.sw[i].y, f.sx[j], acc[i][j][1]);
        acc[i][j][2] = fmaf(p[2] * f.sw[i].z, f.sx[j], acc[i][j][2]);
        acc[i][j][3] = fmaf(p[3] * f.sw[i].w, f.sx[j], acc[i][j][3]);
      }
    }
}

template <int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_dense8(GemmArgs a, int tiles_m, int tiles_n) {
#if SG_DEVICE_PASS
  using namespace d8;
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sm2[BYTES];
  uint8_t* const buf[3] = {sm0, sm1, sm2};
  to_batch(a);

  int tn, tm;
  tile_coords(tiles_m, tiles_n, tn, tm);
  const int64_t n0 = (int64_t)tn * BN, m0 = (int64_t)tm * BM;

  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 3, wm = wave >> 2;
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);

  const int64_t mrows = min((int64_t)BM, a.M - m0), nrows = min((int64_t)BN, a.N - n0);
  const rsrc_v rx = rsrc_words(a.x + m0 * a.ldx, (uint32_t)(mrows * a.ldx));
  const rsrc_v rw = rsrc_words(a.w + n0 * a.ldw, (uint32_t)(nrows * a.ldw));
  const rsrc_v rsx = rsrc_words(a.sx, 0xffffffffu);
  const rsrc_v rsw = rsrc_words(a.sw, 0xffffffffu);
  const PlanD8 plan = make_plan_d8(a, n0, m0, wave, l);
  const LaneD8 lo = lane_d8(wn, wm, g, lr);

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  if constexpr (GRAN_N == 128 || GRAN_N == 0) {
    // Three LDS stages and two register sets.  Step kb waits for stage
    // kb + 1, issues stage kb + 3 into the buffer stage kb has left, reads
    // stage kb + 1 into the spare register set and multiplies stage kb (read
    // during the previous step), so the LDS reads of one stage overlap the
    // MFMAs of the one before.  Stages past the last K block reload the last
    // block (into buffers whose contents are read but not used), so every
    // step issues one stage, each wave has exactly two stages in flight
    // before its wait, and the loop has no branches.  The loads are not
    // tracked by the compiler (see dma16), so the buffers rotate at run time.
#pragma unroll
    for (int s = 0; s < NST; ++s) issue_d8(buf[s], plan, rx, rw, rsx, rsw, a, min(s, KB - 1), wave);
    uint8_t* b0 = sm0;   // stage kb
    uint8_t* b1 = sm1;   // stage kb + 1
    uint8_t* b2 = sm2;   // stage kb + 2
    FragD8 f0, f1;
    wait_vmcnt<2 * LOADS>();
    lds_barrier();
    read_b_d8<GRAN_N>(b0, lo, wn, f0);
#pragma unroll
    for (int i = 0; i < 4; ++i) read_a_d8<GRAN_N>(b0, lo, i, f0);

    auto step = [&](const FragD8& cur, FragD8& nxt, int kb) {
      wait_vmcnt<LOADS>();   // stage kb + 1 has landed; stage kb + 2 may stay in flight
      lds_barrier();         // every wave is done reading stage kb into registers
      issue_d8(b0, plan, rx, rw, rsx, rsw, a, min(kb + NST, KB - 1), wave);
      step_d8<GRAN_N>(cur, nxt, b1, lo, wn, acc);
      uint8_t* const t = b0;
      b0 = b1; b1 = b2; b2 = t;
    };
    int kb = 0;
    for (; kb + 2 <= KB; kb += 2) {
      step(f0, f1, kb);
      step(f1, f0, kb + 1);
    }
    if (kb < KB) step(f0, f1, kb);
  } else {
    // Per-row W scales need more registers per stage: one register set.
    // Step kb waits for stage kb, issues stage kb + 2 into the buffer stage
    // kb - 1 has left, then reads and multiplies stage kb.
#pragma unroll
    for (int s = 0; s < NST - 1; ++s) issue_d8(buf[s], plan, rx, rw, rsx, rsw, a, min(s, KB - 1), wave);
    uint8_t* bp = sm2;   // stage kb - 1
    uint8_t* b0 = sm0;   // stage kb
    uint8_t* b1 = sm1;   // stage kb + 1
    FragD8 f;
    for (int kb = 0; kb < KB; ++kb) {
      wait_vmcnt<LOADS>();   // stage kb has landed; stage kb + 1 may stay in flight
      lds_barrier();
      issue_d8(bp, plan, rx, rw, rsx, rsw, a, min(kb + NST - 1, KB - 1), wave);
      read_b_d8<GRAN_N>(b0, lo, wn, f);
#pragma unroll
      for (int i = 0; i < 4; ++i) read_a_d8<GRAN_N>(b0, lo, i, f);
      mma_d8<GRAN_N>(f, acc);
      uint8_t* const t = bp;
      bp = b0; b0 = b1; b1 = t;
    }
  }
  wait_vmcnt<0>();   // no load may still be writing LDS when the tile is staged there
  if constexpr (GRAN_N == 0) {   // every wave's loads of the stages have landed
    lds_barrier();
    rows_scale<false, 4>(sm2, acc, lo.sx, lo.sw);
  }

  if constexpr (OUT_BF16) {   // half of a bf16 tile fits one stage buffer
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f b = with_bias(a, n0 + wn * 64 + i * 16 + 4 * g, acc[i][j]);
        const float v[4] = {b[0], b[1], b[2], b[3]};
        stage_quad<OUT_BF16, OUT_T, BYTES>(sm0, sm1, wn * 64 + i * 16 + 4 * g, wm * 64 + j * 16 + lr, v);
      }
    __syncthreads();
    store_staged<OUT_BF16, OUT_T, BYTES>(a, sm0, sm1, m0, n0, t);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_quad<OUT_BF16, OUT_T>(a, m0 + wm * 64 + j * 16 + lr, n0 + wn * 64 + i * 16 + 4 * g,
                                    with_bias(a, n0 + wn * 64 + i * 16 + 4 * g, acc[i][j]));
  }
#endif  // SG_DEVICE_PASS
}

// ============================================================ decode kernel
// For M <= 64 (decode-sized batches).  A workgroup owns RB blocks of 16 W
// rows and all M columns (MT sub-tiles of 16); its 8 waves split the K blocks
// (wave w takes kb = w, w + 8, ...), read their operands straight from global
// memory into the matrix-core layout, and finally add their partial tiles
// through LDS.  The weight is streamed once from HBM; X is small and stays in
// L2, and each X fragment a wave reads serves RB row blocks (RB is chosen at
// launch so that the grid still covers the 256 CUs).  A wave issues the loads
// of DEC_U K blocks before it multiplies them; all loads are unconditional
// (buffer loads read zeros past the rows that exist), so nothing waits for a
// load until its K block is multiplied.  (Measured on MI355X: two K blocks in
// flight per wave stream fastest; deeper batches or double buffering are
// slower.)  Columns m >= M are zero-filled (the partial M tile).
constexpr int DEC_WAVES = 8, DEC_U = 2;

// Operands of one K block for one wave.
template <int RB, int MT>
struct DecOps {
  v4i asp[RB];    // sparse A operands (W rows n0 + 16 r .. + 15)
  v8i ad[RB];     // dense A operands
  int idx[RB];    // sparse index words
  v8i bx[MT];     // X columns 16 j + lr
  float sxv[MT];  // their scales
  float sw4[RB][4];  // W scales of this lane's 4 output rows in each row block
};

#if SG_DEVICE_PASS
// Buffer resources of a decode workgroup: reads past the rows that exist
// return zeros, so every load is unconditional (a conditional load would make
// the compiler wait for it where the branches join).
struct DecRes {
  __amdgpu_buffer_rsrc_t rx, rw, rm;
};

__device__ __forceinline__ v4i buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ v2i buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
__device__ __forceinline__ int buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}

template <bool SPARSE, bool PACKED, int RB, int MT, int GRAN_N>
__device__ __forceinline__ void dec_load(const GemmArgs& a, const DecRes& res, int64_t n0, int kb, int KB, int lr,
                                         int g, DecOps<RB, MT>& o) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t nb = n0 + 16 * rb;
    o.idx[rb] = 0;
    if (PACKED) {
      // chunk of (row block rb of this workgroup, K block kb)
      const uint32_t c = (uint32_t)(rb * KB) * PK_CHUNK;
      const v4i av = buf_ld16(res.rw, c + pk_val_off(lr, g), kb * PK_CHUNK);
      o.asp[rb] = av;
      o.idx[rb] = buf_ld4(res.rw, c + PK_META + pk_meta_word(lr, g), kb * PK_CHUNK);
    } else if (SPARSE) {
      const uint32_t row = (uint32_t)((16 * rb + lr) * a.ldw) + sp_a_off(g);
      const v2i lo = buf_ld8(res.rw, row, kb * 64), hi = buf_ld8(res.rw, row + 16, kb * 64);
      const v4i mw = buf_ld16(res.rm, (uint32_t)((16 * rb + lr) * a.ldm), kb * 16);
      o.asp[rb] = (v4i){lo[0], lo[1], hi[0], hi[1]};
      o.idx[rb] = sp_meta_word(make_uint4(mw[0], mw[1], mw[2], mw[3]), g);
    } else {
      const uint32_t row = (uint32_t)((16 * rb + lr) * a.ldw) + 32 * g;
      const v4i lo = buf_ld16(res.rw, row, kb * 128), hi = buf_ld16(res.rw, row + 16, kb * 128);
      o.ad[rb] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // W scale(s) of this K block (rows past N read the last row's scale; they are never stored)
    if (GRAN_N == 128) {
      const float v = a.sw[(min(nb, a.N - 1) >> 7) * a.sw_sn + kb * a.sw_sk];
      o.sw4[rb][0] = o.sw4[rb][1] = o.sw4[rb][2] = o.sw4[rb][3] = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o.sw4[rb][e] = a.sw[min(nb + 4 * g + e, a.N - 1) * a.sw_sn + kb * a.sw_sk];
    }
  }
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = j * 16 + lr;   // rows past M read as zero; their scale is the last row's
    const uint32_t xo = (uint32_t)(m * a.ldx) + 32 * g;
    const v4i lo = buf_ld16(res.rx, xo, kb * 128), hi = buf_ld16(res.rx, xo + 16, kb * 128);
    o.bx[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    o.sxv[j] = a.sx[(min((int64_t)m, a.M - 1) >> a.gm_shift) * a.sx_sm + kb * a.sx_sk];
  }
}
#endif  // SG_DEVICE_PASS

template <bool SPARSE, bool I8, int RB, int MT>
__device__ __forceinline__ void dec_compute(const DecOps<RB, MT>& o, v4f (&acc)[RB][MT]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const v4f p = SPARSE ? mma_sparse<I8>(o.asp[rb], o.bx[j], o.idx[rb]) : mma_dense(o.ad[rb], o.bx[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[rb][j][e] = fmaf(p[e] * o.sw4[rb][e], o.sxv[j], acc[rb][j][e]);
    }
}

// EVEN: the row blocks shared over the workgroups as in k_gemm_decode_dma
// (one problem; q = R / G and r = R % G from the host).
template <bool SPARSE, bool I8, bool PACKED, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool EVEN>
__global__ void __launch_bounds__(512) k_gemm_decode(GemmArgs a, int q, int r) {
#if SG_DEVICE_PASS
  constexpr int U = DEC_U;
  __shared__ __attribute__((aligned(16))) float red[DEC_WAVES][RB * MT][64][4];
  to_batch(a);
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = l >> 4, lr = l & 15;
  int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
  if constexpr (EVEN) {
    const int b = (int)blockIdx.x;
    const int rb0 = b * q + min(b, r), rb1 = rb0 + q + (b < r ? 1 : 0);
    n0 = 16 * (int64_t)rb0;
    a.N = min(a.N, 16 * (int64_t)rb1);   // the rows past this workgroup's are another's: not loaded, not stored
  }
  if (blockIdx.y > 0) {   // grid row y (one problem, M <= 64): X rows, X scales and outputs from 16 MT y on
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;
    a.x += m0 * a.ldx;
    a.sx += (m0 >> a.gm_shift) * a.sx_sm;
    a.M -= m0;
    a.y = static_cast<uint8_t*>(a.y) + (OUT_T ? m0 : m0 * a.ldy) * (OUT_BF16 ? 2 : 4);
  }
  const int KB = (int)(a.K >> 7);
  const int nt = (KB - wave + DEC_WAVES - 1) / DEC_WAVES;   // K blocks of this wave
  const int rows = (int)min((int64_t)(16 * RB), a.N - n0);  // W rows of this workgroup that exist
  DecRes res;
  res.rx = rsrc(a.x, (uint32_t)(a.M * a.ldx));
  if (SPARSE && PACKED) {
    const int rbs = (rows + PK_ROWS - 1) / PK_ROWS;
    res.rw = rsrc(a.w + (n0 / PK_ROWS) * KB * PK_CHUNK, (uint32_t)(rbs * KB * PK_CHUNK));
    res.rm = res.rw;
  } else {
    res.rw = rsrc(a.w + n0 * a.ldw, (uint32_t)(rows * a.ldw));
    res.rm = SPARSE ? rsrc(a.meta + n0 * a.ldm, (uint32_t)(rows * a.ldm)) : res.rw;
  }

  v4f acc[RB][MT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[rb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  DecOps<RB, MT> ops[U];
  // (K blocks past the wave's last are loaded as its last one and not multiplied)
  auto load_batch = [&](DecOps<RB, MT>(&o)[U], int t0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      dec_load<SPARSE, PACKED, RB, MT, GRAN_N>(a, res, n0, wave + DEC_WAVES * min(t0 + u, nt - 1), KB, lr, g, o[u]);
  };
  auto compute_batch = [&](const DecOps<RB, MT>(&o)[U], int t0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u < nt) dec_compute<SPARSE, I8, RB, MT>(o[u], acc);
  };
  for (int t0 = 0; t0 < nt; t0 += U) {
    load_batch(ops, t0);
    compute_batch(ops, t0);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j)
      *reinterpret_cast<float4*>(&red[wave][rb * MT + j][l][0]) =
          make_float4(acc[rb][j][0], acc[rb][j][1], acc[rb][j][2], acc[rb][j][3]);
  __syncthreads();
  // 512 threads: thread -> (row block rb, sub-tile j, lane ll); RB * MT * 64 lanes of 4 values
  for (int q = t; q < RB * MT * 64; q += 512) {
    const int s = q >> 6, ll = q & 63, rb = s / MT, j = s % MT;
    float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[w][s][ll][0]);
      v4.x += v.x; v4.y += v.y; v4.z += v.z; v4.w += v.w;
    }
    const v4f out = {v4.x, v4.y, v4.z, v4.w};
    store_quad<OUT_BF16, OUT_T>(a, (int64_t)j * 16 + (ll & 15), n0 + 16 * rb + 4 * (ll >> 4),
                                with_bias(a, n0 + 16 * rb + 4 * (ll >> 4), out));
  }
#endif  // SG_DEVICE_PASS
}

// ------------------------------------------- decode kernel, LDS-DMA streaming
// For packed 2:4 weights with 128-row W scales and M <= 64.  Same work split
// as k_gemm_decode, but each wave streams its K blocks into a private ring of
// LDS slots with buffer loads that write LDS directly: per K block the RB
// weight chunks (verbatim), the X slice when M <= 16 (16 rows x 128 B, 16-byte
// chunks swizzled by row against bank conflicts) and both scales.  A wave only waits
// for its own loads, so the loop has no barriers, and a load into LDS needs no
// registers while in flight (measured on MI355X: this streams faster than
// loads into registers, which stop gaining from more loads in flight early).
// Ring of two slots per wave (the compiler tracks the loads in flight into two
// LDS arrays separately, so that reading one slot does not wait for the
// other); a slot holds KPS K blocks.  With two or more 16-row sub-tiles the X
// slices would crowd 4 row blocks of weight out of the ring (2 KB per sub-tile
// and K block against 1.25 KB per row block): there each wave loads its X
// fragments into registers with the same K block's loads (loads return in
// order, so the per-slot count still covers them).  With fewer row blocks X
// outweighs the weight, and the ring streams it better than register loads
// (measured at M = 37, N = 4096, K = 14336: 16.8 against 23.0 us).
template <int RB, int MT>
struct DmaCfg {
  static constexpr bool XR = MT >= 2 && (RB >= 3 || MT == 4);   // X fragments in registers
  static constexpr int XOFF = RB * PK_CHUNK;                    // X slices (2 KB each) unless XR
  static constexpr int SXOFF = XOFF + (XR ? 0 : MT * 2048);     // X scales (256 B per sub-tile)
  static constexpr int SWOFF = SXOFF + MT * 256;                // W scales (256 B)
  static constexpr int KSZ = SWOFF + 256;                       // bytes per wave per K block
  static constexpr int KPS = 2 * 2 * DEC_WAVES * KSZ <= 150 * 1024 ? 2 : 1;   // K blocks per slot
  static constexpr int SLOT = KPS * KSZ;                        // bytes per wave per slot
  static constexpr int ARR = DEC_WAVES * SLOT;                  // one ring slot of all waves
  static constexpr int L = KPS * (2 * RB + 3 * MT + 1);         // LDS-DMA loads per slot
  static constexpr bool FITS = 2 * DEC_WAVES * KSZ <= 160 * 1024;  // two slots of one K block
};

#if SG_DEVICE_PASS
struct DmaOffs {
  uint32_t x[2];    // X slice chunk source offsets (K block 0)
  uint32_t sx[4];   // X scale source offsets per sub-tile (K block 0)
  uint32_t sw;      // W scale source offset (K block 0)
};

// Loads of one K block into its part of a slot.  Every load writes LDS
// directly (so that the compiler can neither merge nor drop any of them: the
// slot's count of L loads is exact).  A K block past the wave's last is still
// issued (so that every slot has exactly L loads in flight on every path), but
// its weight and X loads go through descriptors of zero records, out of range
// for every offset (no memory access, zeros), and its scales are those of a
// valid block.
template <int RB, int MT>
__device__ __forceinline__ void dma_issue(uint8_t* slot, const GemmArgs& a, __amdgpu_buffer_rsrc_t rw,
                                          __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rsx,
                                          __amdgpu_buffer_rsrc_t rsw, const DmaOffs& o, int kb, int KB, int l,
                                          bool valid, v8i (&xr)[MT]) {
  using C = DmaCfg<RB, MT>;
  const int ws = valid ? kb * PK_CHUNK : 0, xs = valid ? kb * 128 : 0;
  if (!valid) {
    rw = rsrc(a.w, 0);
    rx = rsrc(a.x, 0);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    uint8_t* c = slot + rb * PK_CHUNK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)c, 16, (uint32_t)(rb * KB) * PK_CHUNK + l * 16, ws, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(c + PK_META), 4,
                                             (uint32_t)(rb * KB) * PK_CHUNK + PK_META + l * 4, ws, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    if constexpr (C::XR) {   // row 16 j + (l & 15), bytes 32 (l >> 4) .. + 31 of the K block
      const uint32_t xo = (uint32_t)((16 * j + (l & 15)) * a.ldx) + 32 * (l >> 4);
      const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, xs, 0));
      const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16, xs, 0));
      xr[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      uint8_t* x = slot + C::XOFF + j * 2048;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)x, 16, o.x[0] + (uint32_t)(16 * j * a.ldx), xs, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(x + 1024), 16, o.x[1] + (uint32_t)(16 * j * a.ldx),
                                               xs, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lds_void*)(slot + C::SXOFF + j * 256), 4, o.sx[j],
                                             (int)(kb * a.sx_sk * 4), 0, 0);
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)(slot + C::SWOFF), 4, o.sw, (int)(kb * a.sw_sk * 4), 0, 0);
}
#endif

#if SG_DEVICE_PASS
// The end of a decode workgroup: the 8 waves' partial tiles (each wave summed
// its own K blocks) are added in wave order through LDS (r0, r1: two arrays of
// ARR bytes that no load is filling any more) and stored with the bias.
template <int RB, int MT, int ARR, bool OUT_BF16, bool OUT_T>
__device__ __forceinline__ void dec_reduce_store(const GemmArgs& a, const v4f (&acc)[RB][MT], uint8_t* r0,
                                                 uint8_t* r1, int64_t n0, int wave) {
  const int t = threadIdx.x, l = t & 63;
  if constexpr (DEC_WAVES * RB * MT * 64 * 16 <= ARR) {   // all partial tiles at once, in r0
    __syncthreads();
    float4* red = reinterpret_cast<float4*>(r0);    // [DEC_WAVES][RB * MT][64]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < MT; ++j)
        red[(wave * RB * MT + rb * MT + j) * 64 + l] =
            make_float4(acc[rb][j][0], acc[rb][j][1], acc[rb][j][2], acc[rb][j][3]);
    __syncthreads();
    for (int q = t; q < RB * MT * 64; q += 512) {
      const int s = q >> 6, ll = q & 63, rb = s / MT, j = s % MT;
      float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) {
        const float4 v = red[(w * RB * MT + s) * 64 + ll];
        v4.x += v.x; v4.y += v.y; v4.z += v.z; v4.w += v.w;
      }
      const v4f out = {v4.x, v4.y, v4.z, v4.w};
      store_quad<OUT_BF16, OUT_T>(a, (int64_t)j * 16 + (ll & 15), n0 + 16 * rb + 4 * (ll >> 4),
                                  with_bias(a, n0 + 16 * rb + 4 * (ll >> 4), out));
    }
    return;
  }
  // otherwise waves 0-3 hand their partial tiles over in r0, waves 4-7 in r1,
  // one sub-tile column j at a time: [4][RB][64] float4 each
  static_assert(4 * RB * 64 * 16 <= ARR, "LDS");
  float4* const mine = reinterpret_cast<float4*>(wave < 4 ? r0 : r1) + (wave & 3) * RB * 64;
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      mine[rb * 64 + l] = make_float4(acc[rb][j][0], acc[rb][j][1], acc[rb][j][2], acc[rb][j][3]);
    __syncthreads();
    for (int q = t; q < RB * 64; q += 512) {
      const int rb = q >> 6, ll = q & 63;
      float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) {
        const float4 v = reinterpret_cast<const float4*>(w < 4 ? r0 : r1)[((w & 3) * RB + rb) * 64 + ll];
        v4.x += v.x; v4.y += v.y; v4.z += v.z; v4.w += v.w;
      }
      const v4f out = {v4.x, v4.y, v4.z, v4.w};
      store_quad<OUT_BF16, OUT_T>(a, (int64_t)j * 16 + (ll & 15), n0 + 16 * rb + 4 * (ll >> 4),
                                  with_bias(a, n0 + 16 * rb + 4 * (ll >> 4), out));
    }
  }
}

// r0, r1: two LDS arrays of at least DmaCfg<RB, MT>::ARR bytes (the ring's
// slots); n0: the workgroup's first W row (a multiple of 16; it owns rows
// n0 .. min(n0 + 16 RB, a.N) - 1).
template <bool I8, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
__device__ __forceinline__ void decode_dma_body(const GemmArgs& a, uint8_t* r0, uint8_t* r1, int64_t n0) {
  using C = DmaCfg<RB, MT>;
  constexpr int KPS = C::KPS;
  static_assert(MT <= 4 && 2 * C::ARR <= 160 * 1024, "LDS");
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  const int nt = (KB - wave + DEC_WAVES - 1) / DEC_WAVES;    // K blocks of this wave
  const int ns = (nt + KPS - 1) / KPS;                         // slots of this wave
  const int rows = (int)min((int64_t)(16 * RB), a.N - n0);
  const int rbs = (rows + PK_ROWS - 1) / PK_ROWS;
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w + (n0 / PK_ROWS) * KB * PK_CHUNK, (uint32_t)(rbs * KB * PK_CHUNK));
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, (uint32_t)(a.M * a.ldx));
  const __amdgpu_buffer_rsrc_t rsx = rsrc(a.sx, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t rsw = rsrc(a.sw, 0xffffffffu);
  DmaOffs o;
  // X slice: instruction i, lane l -> LDS 16-byte position p = 64 i + l: row p >> 3, chunk (p & 7) ^ (row & 7)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 64 * i + l, r = p >> 3, c = (p & 7) ^ swz8(r);
    o.x[i] = (uint32_t)(r * a.ldx + c * 16);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = min((int64_t)(16 * j + (l & 15)), a.M - 1);
    o.sx[j] = (uint32_t)(((m >> a.gm_shift) * a.sx_sm) * 4);
  }
  o.sw = (uint32_t)(((min(n0 + 16 * (l % RB), a.N - 1) >> 7) * a.sw_sn) * 4);
  // lane-constant LDS offsets within a wave's slot
  const uint32_t wslot = (uint32_t)wave * C::SLOT;
  const uint32_t oa = wslot + pk_val_off(lr, g), om = wslot + PK_META + pk_meta_word(lr, g);
  const uint32_t ox0 = wslot + C::XOFF + lr * 128 + (((2 * g) ^ swz8(lr)) << 4);
  const uint32_t ox1 = wslot + C::XOFF + lr * 128 + (((2 * g + 1) ^ swz8(lr)) << 4);
  const uint32_t osx = wslot + C::SXOFF + lr * 4, osw = wslot + C::SWOFF;

  // X fragments of the K blocks of the slot in r0 / r1 (registers when XR)
  v8i xa[KPS][MT], xb[KPS][MT];
  auto issue = [&](uint8_t* arr, v8i (&xr)[KPS][MT], int s) {
#pragma unroll
    for (int k = 0; k < KPS; ++k) {
      const int tt = s * KPS + k;
      dma_issue<RB, MT>(arr + wslot + k * C::KSZ, a, rw, rx, rsx, rsw, o, wave + DEC_WAVES * min(tt, nt - 1), KB, l,
                        tt < nt, xr[k]);
    }
  };

  v4f acc[RB][MT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[rb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* sl, const v8i (&xr)[KPS][MT], int s) {
#pragma unroll
    for (int k = 0; k < KPS; ++k) {
      if (s * KPS + k < nt) {
        const uint32_t kk = k * C::KSZ;
        v8i bx[MT];
        float sxv[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          if constexpr (C::XR) {
            bx[j] = xr[k][j];
          } else {
            const uint4 lo = lds_ld<uint4>(sl, ox0 + kk + j * 2048), hi = lds_ld<uint4>(sl, ox1 + kk + j * 2048);
            bx[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
          sxv[j] = lds_ld<float>(sl, osx + kk + j * 256);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint4 av = lds_ld<uint4>(sl, oa + kk + rb * PK_CHUNK);
          const int idx = lds_ld<int>(sl, om + kk + rb * PK_CHUNK);
          const float swv = lds_ld<float>(sl, osw + kk + rb * 4);
          const v4i aa = {(int)av.x, (int)av.y, (int)av.z, (int)av.w};
#pragma unroll
          for (int j = 0; j < MT; ++j) {
            const v4f p = mma_sparse<I8>(aa, bx[j], idx);
            acc[rb][j] += p * (swv * sxv[j]);
          }
        }
      }
    }
  };

  // slot s lives in r0 for even s, r1 for odd s; slot s + 1 is loaded while
  // slot s is multiplied
  if (ns > 0) issue(r0, xa, 0);
  for (int s0 = 0; s0 < ns; s0 += 2) {
    issue(r1, xb, s0 + 1);
    wait_vmcnt<C::L>();
    compute(r0, xa, s0);
    if (s0 + 1 < ns) {
      issue(r0, xa, s0 + 2);
      wait_vmcnt<C::L>();
      compute(r1, xb, s0 + 1);
    }
  }
  wait_vmcnt<0>();
  dec_reduce_store<RB, MT, C::ARR, OUT_BF16, OUT_T>(a, acc, r0, r1, n0, wave);
}
#endif  // SG_DEVICE_PASS

// EVEN: the G workgroups share the R row blocks of 16 evenly, q = R / G and
// r = R % G: workgroup b owns the q + (b < r) row blocks from b q + min(b, r)
// on (at most RB), so that one workgroup per CU covers a weight whose row
// blocks are not a multiple of RB per CU; otherwise workgroup b owns row
// blocks RB b .. RB b + RB - 1 (q and r unused).  The quotient and remainder
// come from the host: a division here would be expanded into vector
// instructions, and the buffer descriptors computed from its result would
// then be vector values that cost a readfirstlane loop around every load.
template <bool I8, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool EVEN>
__global__ void __launch_bounds__(512) k_gemm_decode_dma(GemmArgs a, int q, int r) {
#if SG_DEVICE_PASS
  to_batch(a);
  __shared__ __attribute__((aligned(1024))) uint8_t r0[DmaCfg<RB, MT>::ARR];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[DmaCfg<RB, MT>::ARR];
  int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
  if constexpr (EVEN) {
    const int b = (int)blockIdx.x;
    const int rb0 = b * q + min(b, r), rb1 = rb0 + q + (b < r ? 1 : 0);
    n0 = 16 * (int64_t)rb0;
    a.N = min(a.N, 16 * (int64_t)rb1);   // the rows past this workgroup's are another's: not loaded, not stored
  }
  if (blockIdx.y > 0) {   // grid row y (one problem, M <= 64): X rows, X scales and outputs from 16 MT y on
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;
    a.x += m0 * a.ldx;
    a.sx += (m0 >> a.gm_shift) * a.sx_sm;
    a.M -= m0;
    a.y = static_cast<uint8_t*>(a.y) + (OUT_T ? m0 : m0 * a.ldy) * (OUT_BF16 ? 2 : 4);
  }
  decode_dma_body<I8, RB, MT, GRAN_N, OUT_BF16, OUT_T>(a, r0, r1, n0);
#endif
}

// Grouped problems of at most 16 MT rows each (grid y = group): group g's X
// rows, X scales (one row each), Y rows (columns of Y^T), packed weight, W
// scales and bias, as in k_gemm_sparse_grouped.  An empty group's
// workgroups return at once.
template <bool I8, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_decode_dma_grouped(GemmArgs a, GroupTable gt) {
#if SG_DEVICE_PASS
  group_args<OUT_BF16, OUT_T>(a, gt, blockIdx.y);
  if (a.M == 0) return;
  __shared__ __attribute__((aligned(1024))) uint8_t r0[DmaCfg<RB, MT>::ARR];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[DmaCfg<RB, MT>::ARR];
  decode_dma_body<I8, RB, MT, GRAN_N, OUT_BF16, OUT_T>(a, r0, r1, (int64_t)blockIdx.x * 16 * RB);
#endif
}

// Grouped problem with tails (group tables gt for the large tiles, gtail for
// each group's last <= 64 rows): workgroups 0 .. T - 1 run the large tiles,
// the rest each run one block of 4 row blocks of one group's tail with the
// LDS-streaming decode body (tail_gx of them per group).  The tiles are
// dispatched first, so the tails run on the CUs the tiles leave idle and
// after them, in the same launch; both bodies use the same two LDS arrays.
template <int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_grouped_tails(GemmArgs a, GroupTable gt, GroupTable gtail, int T,
                                                             int tail_gx) {
#if SG_DEVICE_PASS
  static_assert(DmaCfg<4, 1>::ARR <= x2::DBL && DmaCfg<4, 2>::ARR <= x2::DBL && DmaCfg<4, 3>::ARR <= x2::DBL &&
                    DmaCfg<4, 4>::ARR <= x2::DBL,
                "the decode rings fit the tile's LDS arrays");
  __shared__ __attribute__((aligned(1024))) uint8_t s0[x2::DBL];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[x2::DBL];
  if ((int)blockIdx.x < T) {
    grouped_tile<GRAN_N, OUT_BF16, OUT_T>(a, gt, T, s0, s1);
  } else {
    const int d = (int)blockIdx.x - T;
    group_args<OUT_BF16, OUT_T>(a, gtail, d / tail_gx);
    if (a.M == 0) return;
    // as many 16-row sub-tiles as this group's tail needs (uniform per workgroup)
    if (a.M <= 16) decode_dma_body<false, 4, 1, 128, OUT_BF16, OUT_T>(a, s0, s1, (int64_t)(d % tail_gx) * 64);
    else if (a.M <= 32) decode_dma_body<false, 4, 2, 128, OUT_BF16, OUT_T>(a, s0, s1, (int64_t)(d % tail_gx) * 64);
    else if (a.M <= 48) decode_dma_body<false, 4, 3, 128, OUT_BF16, OUT_T>(a, s0, s1, (int64_t)(d % tail_gx) * 64);
    else decode_dma_body<false, 4, 4, 128, OUT_BF16, OUT_T>(a, s0, s1, (int64_t)(d % tail_gx) * 64);
  }
#endif
}

// ------------------------------------------- decode kernel, activation quantised in the prologue
// torchao PR #3258 "Introduce new W8A8-FP-CSR quantization API", jcaip's
// review: the activation is scaled and cast to float8_e4m3fn on the way into
// the sparse FP8 GEMM.  Here that cast happens inside the GEMM: X arrives as
// fp32 or bf16 and every wave quantises the 1 x 128 blocks of the K blocks it
// multiplies (block amax over the four lanes that hold a row's 128 values, one
// IEEE divide per value, the e4m3 encoder of the quantiser kernels), so the
// codes and scales are exactly those sg_fp8_quant_groupwise(gr = 1, gc = 128)
// writes.  The work split, the K-block order of each wave, the promotion
// acc += p * (sw * sx) and the reduction over the waves are those of
// k_gemm_decode_dma, so every output is the same fp32 sum, term by term: the
// fused call returns bit for bit what quantise-then-GEMM returns.
//
// Per wave and K block: the weight chunks and W scales go to a two-slot LDS
// ring (LDS-DMA, as in k_gemm_decode_dma); the X values go to registers (32
// per lane and 16-row sub-tile: lane (lr, g) holds row lr, values 32 g ..
// 32 g + 31 of the block, exactly the bytes of the SMFMAC B fragment it
// needs).  X of K block t + 1 is requested right after block t is quantised,
// so its latency hides behind block t's multiplies and the wait for the
// weight.  Each workgroup quantises all of X, so this pays off only while X is
// small against the weight: the replicated quantisation costs about
// (workgroups x M x K) divides.
template <typename XT>
struct XVals;
template <>
struct XVals<float> {
  static constexpr int LOADS = 8;   // 16-byte loads per lane and sub-tile (32 values)
  __device__ static void unpack(const v4i (&r)[LOADS], float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = __int_as_float(r[i][e]);
  }
};
template <>
struct XVals<uint16_t> {
  static constexpr int LOADS = 4;
  __device__ static void unpack(const v4i (&r)[LOADS], float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = (uint32_t)r[i][e];
        v[8 * i + 2 * e] = __uint_as_float(u << 16);
        v[8 * i + 2 * e + 1] = __uint_as_float(u & 0xffff0000u);
      }
  }
};

template <int RB>
struct QCfg {
  static constexpr int SWOFF = RB * PK_CHUNK;    // W scales (256 B)
  static constexpr int KSZ = SWOFF + 256;        // bytes per wave per K block
  static constexpr int ARR = DEC_WAVES * KSZ;    // one ring slot of all waves
  static constexpr int L = 2 * RB + 1;           // LDS-DMA loads per K block
};

#if SG_DEVICE_PASS
// fl32(v / s) from y = fl32(1 / s) with two FMA corrections (Markstein, "Computation
// of elementary functions on the IBM RISC System/6000 processor", 1990: with y
// within half an ulp of 1 / s and q within one ulp of v / s, the residual
// r = v - s q is exact and fl(q + r y) is the correctly rounded quotient; the
// first correction brings q0 = fl(v y), which may be 1.5 ulp off, within one
// ulp).  It holds while nothing underflows: the caller takes it only for
// 2^-90 <= s < inf, where every quotient that is not far below e4m3's
// smallest code keeps its residual normal.  The sign is copied from v, so
// that -0 / s stays -0.
__device__ __forceinline__ float div_refined(float v, float s, float y) {
  const float q0 = v * y;
  const float q1 = fmaf(fmaf(-q0, s, v), y, q0);
  const float q2 = fmaf(fmaf(-q1, s, v), y, q1);
  return __uint_as_float((__float_as_uint(q2) & 0x7fffffffu) | (__float_as_uint(v) & 0x80000000u));
}

// One 16-row sub-tile's K block, as the lane's B fragment (32 codes) and its
// row's scale: the codes of fl32(v / s), as the quantiser kernels compute
// them with IEEE divides.
template <typename XT>
__device__ __forceinline__ void quantise_block(const v4i (&raw)[XVals<XT>::LOADS], v8i& codes, float& sc) {
  float v[32];
  XVals<XT>::unpack(raw, v);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = amax_fold(a, v[i]);
  uint32_t u = __float_as_uint(a);
  u = max(u, (uint32_t)__shfl_xor((int)u, 16, 64));
  u = max(u, (uint32_t)__shfl_xor((int)u, 32, 64));
  sc = block_scale(__uint_as_float(u), 448.0f);
  if (sc >= 0x1p-90f && sc < __builtin_inff()) {   // finite scale: every v is finite
    const float y = 1.0f / sc;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      codes[d] = (int)e4m3_pack4_finite(div_refined(v[4 * d], sc, y), div_refined(v[4 * d + 1], sc, y),
                                        div_refined(v[4 * d + 2], sc, y), div_refined(v[4 * d + 3], sc, y));
  } else {   // tiny, infinite or NaN scales: plain IEEE divides
#pragma unroll
    for (int d = 0; d < 8; ++d)
      codes[d] = (int)e4m3_pack4(v[4 * d] / sc, v[4 * d + 1] / sc, v[4 * d + 2] / sc, v[4 * d + 3] / sc);
  }
}

template <typename XT, int RB, int MT, bool OUT_BF16, bool OUT_T>
__device__ __forceinline__ void decode_q_body(const GemmArgs& a, uint8_t* r0, uint8_t* r1, int64_t n0) {
  using C = QCfg<RB>;
  constexpr int NL = XVals<XT>::LOADS;
  constexpr int ES = (int)sizeof(XT);
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  const int nt = (KB - wave + DEC_WAVES - 1) / DEC_WAVES;    // K blocks of this wave
  const int rows = (int)min((int64_t)(16 * RB), a.N - n0);
  const int rbs = (rows + PK_ROWS - 1) / PK_ROWS;
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w + (n0 / PK_ROWS) * KB * PK_CHUNK, (uint32_t)(rbs * KB * PK_CHUNK));
  const __amdgpu_buffer_rsrc_t rw0 = rsrc(a.w, 0);
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, (uint32_t)(a.M * a.ldx * ES));
  const __amdgpu_buffer_rsrc_t rx0 = rsrc(a.x, 0);
  const __amdgpu_buffer_rsrc_t rsw = rsrc(a.sw, 0xffffffffu);
  const uint32_t osw_src = (uint32_t)(((min(n0 + 16 * (l % RB), a.N - 1) >> 7) * a.sw_sn) * 4);
  const uint32_t wslot = (uint32_t)wave * C::KSZ;
  const uint32_t oa = wslot + pk_val_off(lr, g), om = wslot + PK_META + pk_meta_word(lr, g);
  const uint32_t osw = wslot + C::SWOFF;
  uint32_t xo[MT];   // row 16 j + lr, values 32 g .. of the K block (rows past M read zeros)
#pragma unroll
  for (int j = 0; j < MT; ++j) xo[j] = (uint32_t)((16 * j + lr) * a.ldx * ES + 32 * g * ES);

  // K block number tt of this wave (tt >= nt: no memory access, zeros, W
  // scales of the last block; issued anyway so every slot counts C::L loads)
  auto issue_w = [&](uint8_t* arr, int tt) {
    const bool valid = tt < nt;
    const int kb = wave + DEC_WAVES * min(tt, nt - 1);   // >= 0: only called while nt >= 1
    const __amdgpu_buffer_rsrc_t r = valid ? rw : rw0;
    const int ws = valid ? kb * PK_CHUNK : 0;
    uint8_t* slot = arr + wslot;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint8_t* c = slot + rb * PK_CHUNK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)c, 16, (uint32_t)(rb * KB) * PK_CHUNK + l * 16, ws, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(c + PK_META), 4,
                                               (uint32_t)(rb * KB) * PK_CHUNK + PK_META + l * 4, ws, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)(slot + C::SWOFF), 4, osw_src,
                                             (int)(kb * a.sw_sk * 4), 0, 0);
  };
  v4i raw[MT][NL];
  auto issue_x = [&](int tt) {
    const bool valid = tt < nt;
    const __amdgpu_buffer_rsrc_t r = valid ? rx : rx0;
    const int xs = valid ? (wave + DEC_WAVES * tt) * 128 * ES : 0;
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int i = 0; i < NL; ++i) raw[j][i] = buf_ld16(r, xo[j] + 16 * i, xs);
  };

  v4f acc[RB][MT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[rb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // K block tt: its weight is in `sl`, its X values in raw
  auto step = [&](const uint8_t* sl, int tt) {
    v8i bxq[MT];
    float sxv[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) quantise_block<XT>(raw[j], bxq[j], sxv[j]);
    issue_x(tt + 1);
    if (tt < nt) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const uint4 av = lds_ld<uint4>(sl, oa + rb * PK_CHUNK);
        const int idx = lds_ld<int>(sl, om + rb * PK_CHUNK);
        const float swv = lds_ld<float>(sl, osw + rb * 4);
        const v4i aa = {(int)av.x, (int)av.y, (int)av.z, (int)av.w};
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const v4f p = mma_sparse<false>(aa, bxq[j], idx);
          acc[rb][j] += p * (swv * sxv[j]);
        }
      }
    }
  };

  // block tt's weight lives in r0 for even tt, r1 for odd tt; the next block's
  // weight is requested before this block is waited for.  A wave without K
  // blocks (K < 8 * 128) issues nothing: its "last block" would not exist.
  if (nt > 0) {
    issue_w(r0, 0);
    issue_x(0);
  }
  for (int t0 = 0; t0 < nt; t0 += 2) {
    issue_w(r1, t0 + 1);
    wait_vmcnt<C::L>();
    step(r0, t0);
    if (t0 + 1 < nt) {
      issue_w(r0, t0 + 2);
      wait_vmcnt<C::L>();
      step(r1, t0 + 1);
    }
  }
  wait_vmcnt<0>();
  dec_reduce_store<RB, MT, C::ARR, OUT_BF16, OUT_T>(a, acc, r0, r1, n0, wave);
}
#endif  // SG_DEVICE_PASS

// EVEN: the row blocks shared over the workgroups as in k_gemm_decode_dma
// (q = R / G and r = R % G from the host).  Every workgroup quantises all of
// X, so fewer, taller workgroups also mean less repeated quantisation.
template <typename XT, int RB, int MT, bool OUT_BF16, bool OUT_T, bool EVEN>
__global__ void __launch_bounds__(512) k_gemm_decode_q(GemmArgs a, int q, int r) {
#if SG_DEVICE_PASS
  __shared__ __attribute__((aligned(1024))) uint8_t r0[QCfg<RB>::ARR];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[QCfg<RB>::ARR];
  int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
  if constexpr (EVEN) {
    const int b = (int)blockIdx.x;
    const int rb0 = b * q + min(b, r), rb1 = rb0 + q + (b < r ? 1 : 0);
    n0 = 16 * (int64_t)rb0;
    a.N = min(a.N, 16 * (int64_t)rb1);   // the rows past this workgroup's are another's: not loaded, not stored
  }
  if (blockIdx.y > 0) {   // grid row y (one problem, M <= 64): X rows and outputs from 16 MT y on
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;
    a.x += m0 * a.ldx * (int64_t)sizeof(XT);
    a.M -= m0;
    a.y = static_cast<uint8_t*>(a.y) + (OUT_T ? m0 : m0 * a.ldy) * (OUT_BF16 ? 2 : 4);
  }
  decode_q_body<XT, RB, MT, OUT_BF16, OUT_T>(a, r0, r1, n0);
#endif
}

// ------------------------------------------------------------------ dispatch

template <bool SPARSE, bool I8, bool PACKED, int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_large(const GemmArgs& a, hipStream_t st) {
  const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
  const dim3 grid((unsigned)(tm * tn), 1, (unsigned)a.L);
  if constexpr (SPARSE && PACKED && !I8 && (GRAN_N == 128 || GRAN_N == 0))
    k_gemm_sparse_wr<GRAN_N, OUT_BF16, OUT_T><<<grid, 512, 0, st>>>(a, tm, tn);
  else if constexpr (SPARSE && PACKED && I8 && GRAN_N == 128)   // (int8 with scales constant along K: x2)
    k_gemm_sparse_wr_i8<GRAN_N, OUT_BF16, OUT_T><<<grid, 512, 0, st>>>(a, tm, tn);
  else if (SPARSE)
    k_gemm_sparse_x2<I8, PACKED, GRAN_N, OUT_BF16, OUT_T><<<grid, 512, 0, st>>>(a, tm, tn);
  else
    k_gemm_dense8<GRAN_N, OUT_BF16, OUT_T><<<grid, 512, 0, st>>>(a, tm, tn);
}

static dim3 dec_grid(const GemmArgs& a, int64_t rows16, int rb) {
  return dim3((unsigned)cdiv(rows16, rb), 1, (unsigned)a.L);
}

// Launches the LDS-streaming decode kernel with RB row blocks per workgroup if
// its ring fits LDS and the grid keeps at least 224 workgroups (7/8 of the
// CUs busy; RB = 1 always qualifies).
template <bool I8, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
static bool try_decode_dma(const GemmArgs& a, hipStream_t st, int64_t rows16) {
  if constexpr (DmaCfg<RB, MT>::FITS) {
    if (RB == 1 || rows16 >= RB * 224) {
      k_gemm_decode_dma<I8, RB, MT, GRAN_N, OUT_BF16, OUT_T, false><<<dec_grid(a, rows16, RB), 512, 0, st>>>(a, 0, 0);
      return true;
    }
  }
  return false;
}

// Row blocks per workgroup: the largest of 4, 2, 1 that keeps at least 224
// workgroups and whose operands fit (LDS ring of the streaming kernel; for
// the registers of k_gemm_decode up to 4 with three X sub-tiles, 2 with
// four).  Packed 2:4 weights with
// 128-row W scales take the LDS-streaming kernel when one of its rings fits.
// One problem with more row blocks than CUs but too few for 224 workgroups of
// four: one workgroup per CU, each with ceil(R / CUs) or one fewer row blocks
// (the LDS-streaming kernel's even split).  Measured at M = 16, K = 4096:
// N = 12288 in 8.8 us against 10.2 us with 384 workgroups of two row blocks;
// at N = 14336 the 4-row-block workgroups set the time either way (9.9 us),
// so there the launcher keeps 224 workgroups of four.
template <bool I8, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
static bool try_decode_even(const GemmArgs& a, hipStream_t st, int64_t rows16, int cus) {
  if constexpr (DmaCfg<RB, MT>::FITS) {
    k_gemm_decode_dma<I8, RB, MT, GRAN_N, OUT_BF16, OUT_T, true><<<dim3((unsigned)cus, 1, 1), 512, 0, st>>>(
        a, (int)(rows16 / cus), (int)(rows16 % cus));
    return true;
  }
  return false;
}

template <bool I8, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
static bool launch_decode_even(const GemmArgs& a, hipStream_t st, int64_t rows16) {
  const int cus = cu_count();
  if (a.L != 1 || rows16 <= cus || rows16 >= 4 * 224 || rows16 > 4LL * cus) return false;
  switch (cdiv(rows16, cus)) {
    case 2: return try_decode_even<I8, 2, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16, cus);
    case 3: return try_decode_even<I8, 3, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16, cus);
    default: return try_decode_even<I8, 4, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16, cus);
  }
}

template <bool SPARSE, bool I8, bool PACKED, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_decode_mt(const GemmArgs& a, hipStream_t st) {
  const int64_t rows16 = cdiv(a.N, 16);
  if constexpr (SPARSE && PACKED && GRAN_N == 128 && MT >= 2) {
    // Two grid rows of ceil(MT / 2) sub-tiles: at M = 49..64 over no more row
    // blocks than CUs (the four-sub-tile ring keeps X in registers, and ran
    // slower), and at M = 17..48 over at most half as many row blocks as CUs
    // (the other half of the CUs would idle)
    constexpr int MH = (MT + 1) / 2;
    if (a.L == 1 && (MT == 4 ? rows16 <= cu_count() : 2 * rows16 <= cu_count())) {
      k_gemm_decode_dma<I8, 1, MH, GRAN_N, OUT_BF16, OUT_T, false>
          <<<dim3((unsigned)rows16, (unsigned)cdiv(a.M, 16 * MH), 1), 512, 0, st>>>(a, 0, 0);
      return;
    }
  }
  if constexpr (SPARSE && PACKED && GRAN_N == 128) {
    if (launch_decode_even<I8, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16) ||
        try_decode_dma<I8, 4, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16) ||
        try_decode_dma<I8, 2, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16) ||
        try_decode_dma<I8, 1, MT, GRAN_N, OUT_BF16, OUT_T>(a, st, rows16))
      return;
  }
  constexpr int RB4 = MT <= 3 ? 4 : 1, RB2 = 2;
  if constexpr (MT >= 2) {
    // over at most half as many row blocks as CUs: two grid rows of
    // ceil(MT / 2) sub-tiles (K = 4096, dense, M = 64: N = 1792 8.3 against
    // 12.6 us; at N = 4096, 256 row blocks, slower: 14.8 against 13.7 us)
    constexpr int MH = (MT + 1) / 2;
    if (a.L == 1 && 2 * rows16 <= cu_count()) {
      k_gemm_decode<SPARSE, I8, PACKED, 1, MH, GRAN_N, OUT_BF16, OUT_T, false>
          <<<dim3((unsigned)rows16, (unsigned)cdiv(a.M, 16 * MH), 1), 512, 0, st>>>(a, 0, 0);
      return;
    }
  }
  // one problem over more row blocks than CUs but too few for 224 workgroups
  // of the largest share: one workgroup per CU with an even share of up to 4
  // row blocks (2 with four X sub-tiles); at most 98 of the 256 registers a
  // lane may hold at this occupancy were in use with 4 row blocks and one
  // sub-tile, 86 with 2 and two
  constexpr int RBE = MT <= 3 ? 4 : 2;
  const int cus = cu_count();
  if (a.L == 1 && rows16 > cus && rows16 < (int64_t)RBE * 224 && rows16 <= (int64_t)RBE * cus) {
    const dim3 grid((unsigned)cus, 1, 1);
    const int q = (int)(rows16 / cus), r = (int)(rows16 % cus);
    const int64_t rb = cdiv(rows16, cus);
    if constexpr (RBE == 4) {
      if (rb == 3) {
        k_gemm_decode<SPARSE, I8, PACKED, 3, MT, GRAN_N, OUT_BF16, OUT_T, true><<<grid, 512, 0, st>>>(a, q, r);
        return;
      }
      if (rb == 4) {
        k_gemm_decode<SPARSE, I8, PACKED, 4, MT, GRAN_N, OUT_BF16, OUT_T, true><<<grid, 512, 0, st>>>(a, q, r);
        return;
      }
    }
    k_gemm_decode<SPARSE, I8, PACKED, 2, MT, GRAN_N, OUT_BF16, OUT_T, true><<<grid, 512, 0, st>>>(a, q, r);
    return;
  }
  if (RB4 == 4 && rows16 >= 4 * 224)
    k_gemm_decode<SPARSE, I8, PACKED, RB4, MT, GRAN_N, OUT_BF16, OUT_T, false>
        <<<dec_grid(a, rows16, RB4), 512, 0, st>>>(a, 0, 0);
  else if (RB2 == 2 && rows16 >= 2 * 224)
    k_gemm_decode<SPARSE, I8, PACKED, RB2, MT, GRAN_N, OUT_BF16, OUT_T, false>
        <<<dec_grid(a, rows16, RB2), 512, 0, st>>>(a, 0, 0);
  else
    k_gemm_decode<SPARSE, I8, PACKED, 1, MT, GRAN_N, OUT_BF16, OUT_T, false>
        <<<dec_grid(a, rows16, 1), 512, 0, st>>>(a, 0, 0);
}

// The fused-quantisation decode kernel: row blocks per workgroup as for the
// LDS-streaming decode kernel (an even share over one workgroup per CU
// between 256 and 895 row blocks, else 4, 2 or 1 keeping at least 224
// workgroups); gy grid rows of 16 MT X rows each.  Four fp32 sub-tiles would
// take one row block per workgroup (their X values fill the registers), so
// fp32 X beyond 48 rows runs as two grid rows of two sub-tiles (M = 64,
// N = 14336, K = 4096: 49.6 against 171 us).
template <typename XT, int MT, bool OUT_BF16, bool OUT_T>
static void launch_decode_q_mt(const GemmArgs& a, hipStream_t st, unsigned gy = 1) {
  const int64_t rows16 = cdiv(a.N, 16);
  const int cus = cu_count();
  if constexpr (!(MT == 4 && sizeof(XT) == 4)) {
    // more row blocks than CUs but under 224 workgroups of four: one
    // workgroup per CU with an even share (N = 11008, M = 16, K = 4096:
    // 15.0 us against 23.9 us for 344 workgroups of two row blocks)
    if (a.L == 1 && rows16 > cus && rows16 < 4 * 224 && rows16 <= 4LL * cus) {
      const dim3 grid((unsigned)cus, gy, 1);
      const int q = (int)(rows16 / cus), r = (int)(rows16 % cus);
      switch (cdiv(rows16, cus)) {
        case 2: k_gemm_decode_q<XT, 2, MT, OUT_BF16, OUT_T, true><<<grid, 512, 0, st>>>(a, q, r); return;
        case 3: k_gemm_decode_q<XT, 3, MT, OUT_BF16, OUT_T, true><<<grid, 512, 0, st>>>(a, q, r); return;
        default: k_gemm_decode_q<XT, 4, MT, OUT_BF16, OUT_T, true><<<grid, 512, 0, st>>>(a, q, r); return;
      }
    }
  }
  auto grid = [&](int rb) { return dim3((unsigned)cdiv(rows16, rb), gy, (unsigned)a.L); };
  if (MT == 4 && sizeof(XT) == 4)
    k_gemm_decode_q<XT, 1, MT, OUT_BF16, OUT_T, false><<<grid(1), 512, 0, st>>>(a, 0, 0);
  else if (rows16 >= 4 * 224)
    k_gemm_decode_q<XT, 4, MT, OUT_BF16, OUT_T, false><<<grid(4), 512, 0, st>>>(a, 0, 0);
  else if (rows16 >= 2 * 224)
    k_gemm_decode_q<XT, 2, MT, OUT_BF16, OUT_T, false><<<grid(2), 512, 0, st>>>(a, 0, 0);
  else
    k_gemm_decode_q<XT, 1, MT, OUT_BF16, OUT_T, false><<<grid(1), 512, 0, st>>>(a, 0, 0);
}

template <typename XT, bool OUT_BF16, bool OUT_T>
static void launch_decode_q(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 16) launch_decode_q_mt<XT, 1, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 32) launch_decode_q_mt<XT, 2, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 48) launch_decode_q_mt<XT, 3, OUT_BF16, OUT_T>(a, st);
  // four fp32 sub-tiles fill the registers at one row block per workgroup:
  // two grid rows of 32 X rows instead (each workgroup quantises half of X)
  else if (sizeof(XT) == 4 && a.L == 1) launch_decode_q_mt<XT, 2, OUT_BF16, OUT_T>(a, st, 2);
  else launch_decode_q_mt<XT, 4, OUT_BF16, OUT_T>(a, st);
}

template <bool SPARSE, bool I8, bool PACKED, int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_shape(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 16)
    launch_decode_mt<SPARSE, I8, PACKED, 1, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 32)
    launch_decode_mt<SPARSE, I8, PACKED, 2, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 48)
    launch_decode_mt<SPARSE, I8, PACKED, 3, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 64)
    launch_decode_mt<SPARSE, I8, PACKED, 4, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else
    launch_large<SPARSE, I8, PACKED, GRAN_N, OUT_BF16, OUT_T>(a, st);
}

// Scales constant along K (both K-block strides 0) take the large-M kernels'
// accumulate-then-scale form (GRAN_N = 0); decode-sized M keeps the
// per-block kernels, which read the repeated scales (it streams the weight
// and does not wait on the promotion).  int8 sums stay exact in int32 while
// K * 127^2 < 2^31.
template <bool SPARSE, bool PACKED, bool I8 = false>
static void launch_gemm(const GemmArgs& a, int gran_n, bool bf16, bool yt, hipStream_t st) {
  const bool rows = a.sx_sk == 0 && a.sw_sk == 0 && a.M > 64 && (!I8 || a.K <= (1LL << 17));
  if (rows) {
    if (bf16) {
      if (yt) launch_large<SPARSE, I8, PACKED, 0, true, true>(a, st);
      else launch_large<SPARSE, I8, PACKED, 0, true, false>(a, st);
    } else {
      if (yt) launch_large<SPARSE, I8, PACKED, 0, false, true>(a, st);
      else launch_large<SPARSE, I8, PACKED, 0, false, false>(a, st);
    }
  } else if (gran_n == 128) {
    if (bf16) {
      if (yt) launch_shape<SPARSE, I8, PACKED, 128, true, true>(a, st);
      else launch_shape<SPARSE, I8, PACKED, 128, true, false>(a, st);
    } else {
      if (yt) launch_shape<SPARSE, I8, PACKED, 128, false, true>(a, st);
      else launch_shape<SPARSE, I8, PACKED, 128, false, false>(a, st);
    }
  } else {
    if (bf16) {
      if (yt) launch_shape<SPARSE, I8, PACKED, 1, true, true>(a, st);
      else launch_shape<SPARSE, I8, PACKED, 1, true, false>(a, st);
    } else {
      if (yt) launch_shape<SPARSE, I8, PACKED, 1, false, true>(a, st);
      else launch_shape<SPARSE, I8, PACKED, 1, false, false>(a, st);
    }
  }
}

// Common argument checks of both GEMM entry points (host only, before any HIP call).
static sg_status check_common(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx,
                              const float* sx, int64_t sx_sm, int64_t sx_sk, int gran_m, const float* sw,
                              int64_t sw_sn, int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                              sg_form form) {
  if (!xq || !sx || !sw || !y) return SG_ERR_NULL;
  if ((gran_m != 1 && gran_m != 128) || (gran_n != 1 && gran_n != 128)) return SG_ERR_UNSUPPORTED;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldx < K) return SG_ERR_SHAPE;
  if (ldy < (form == SG_OUT_Y ? N : M)) return SG_ERR_SHAPE;
  if (cdiv(M, 128) * cdiv(N, 256) > 0x7fffffffLL || cdiv(N, 16) > 0x7fffffffLL) return SG_ERR_SHAPE;
  // The large-M kernel addresses tiles and scales with 32-bit buffer offsets.
  if (ldx > (1LL << 24) || sx_sm < 0 || sx_sk < 0 || sw_sn < 0 || sw_sk < 0) return SG_ERR_SHAPE;
  if (((cdiv(M, gran_m) - 1) * sx_sm + (K / 128 - 1) * sx_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (((cdiv(N, gran_n) - 1) * sw_sn + (K / 128 - 1) * sw_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (!aligned(xq, 16) || ldx % 16 || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  return SG_OK;
}

// Batched problems: count and per-operand batch strides (bytes for the codes
// and metadata, floats for the scales, elements for y).
struct Batch {
  int64_t L = 1, bx = 0, bw = 0, bm = 0, bsx = 0, bsw = 0, by = 0;
  const float* bias = nullptr;   // optional per-output-row bias [N] per problem
  int64_t bbs = 0;
};

static sg_status check_batch(const Batch& b) {
  if (b.L <= 0 || b.L > 65535) return SG_ERR_SHAPE;
  if (b.bx < 0 || b.bw < 0 || b.bm < 0 || b.bsx < 0 || b.bsw < 0 || b.by < 0) return SG_ERR_SHAPE;
  if (b.bbs < 0) return SG_ERR_SHAPE;
  if (b.bx % 16 || b.bw % 16 || b.bm % 16 || !aligned(b.bias, 4)) return SG_ERR_ALIGN;
  return SG_OK;
}

static GemmArgs make_args(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx,
                          const float* sx, int64_t sx_sm, int64_t sx_sk, int gran_m, const uint8_t* w,
                          int64_t ldw, const uint8_t* meta, int64_t ldm, const float* sw, int64_t sw_sn,
                          int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt, int64_t ldy, const Batch& b) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.x = xq; a.ldx = ldx;
  a.sx = sx; a.sx_sm = sx_sm; a.sx_sk = sx_sk; a.gm_shift = gran_m == 128 ? 7 : 0;
  a.w = w; a.ldw = ldw; a.meta = meta; a.ldm = ldm;
  a.sw = sw; a.sw_sn = sw_sn; a.sw_sk = sw_sk; a.gn_shift = gran_n == 128 ? 7 : 0;
  a.y = y; a.ldy = ldy;
  const int64_t es = (int64_t)dtype_size(y_dt);
  const size_t vb = 4 * es;
  a.vec_store = (ldy % 4 == 0) && aligned(y, vb) && (b.by * es) % (int64_t)vb == 0;
  a.vec16 = ((ldy * es) % 16 == 0) && aligned(y, 16) && (b.by * es) % 16 == 0;
  a.bx = b.bx; a.bw = b.bw; a.bm = b.bm; a.bsx = b.bsx; a.bsw = b.bsw; a.by = b.by * es;
  a.L = (int)b.L;
  a.bias = b.bias;
  a.bbs = b.bbs;
  return a;
}

}  // namespace sg

using namespace sg;

static sg_status dense_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx, const float* sx,
                            int64_t sx_sm, int64_t sx_sk, int gran_m, const uint8_t* wq, int64_t ldw,
                            const float* sw, int64_t sw_sn, int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt,
                            int64_t ldy, sg_form form, const Batch& b, hipStream_t stream) {
  sg_status st = check_common(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy, form);
  if (st != SG_OK) return st;
  if ((st = check_batch(b)) != SG_OK) return st;
  if (!wq) return SG_ERR_NULL;
  if (ldw < K || ldw >= (1LL << 24)) return SG_ERR_SHAPE;
  if (!aligned(wq, 16) || ldw % 16) return SG_ERR_ALIGN;
  const GemmArgs a = make_args(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wq, ldw, nullptr, 0, sw, sw_sn,
                               sw_sk, gran_n, y, y_dt, ldy, b);
  clear_hip_error();
  launch_gemm<false, false>(a, gran_n, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}

extern "C" sg_status sg_fp8_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                           int64_t ldx, const float* sx, int64_t sx_sm,
                                           int64_t sx_sk, int gran_m, const uint8_t* wq,
                                           int64_t ldw, const float* sw, int64_t sw_sn,
                                           int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt,
                                           int64_t ldy, sg_form form, hipStream_t stream) {
  return dense_gemm(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wq, ldw, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy,
                    form, Batch{}, stream);
}

extern "C" sg_status sg_fp8_gemm_groupwise_batched(int64_t L, int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                                   int64_t ldx, int64_t x_bs, const float* sx, int64_t sx_sm,
                                                   int64_t sx_sk, int64_t sx_bs, int gran_m, const uint8_t* wq,
                                                   int64_t ldw, int64_t w_bs, const float* sw, int64_t sw_sn,
                                                   int64_t sw_sk, int64_t sw_bs, int gran_n, const float* bias,
                                                   int64_t bias_bs, void* y, sg_dtype y_dt, int64_t ldy,
                                                   int64_t y_bs, sg_form form, hipStream_t stream) {
  Batch b;
  b.L = L; b.bx = x_bs; b.bw = w_bs; b.bsx = sx_bs; b.bsw = sw_bs; b.by = y_bs;
  b.bias = bias; b.bbs = bias_bs;
  return dense_gemm(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wq, ldw, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy,
                    form, b, stream);
}

// The 2:4 GEMM entry points: FP8 (e4m3) or int8 codes, canonical (values +
// metadata) or gfx950-packed weights.
template <bool I8>
static sg_status sparse24_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx, const float* sx,
                               int64_t sx_sm, int64_t sx_sk, int gran_m, const uint8_t* wv, int64_t ldwv,
                               const uint8_t* wmeta, int64_t ldwm, const float* sw, int64_t sw_sn, int64_t sw_sk,
                               int gran_n, void* y, sg_dtype y_dt, int64_t ldy, sg_form form, const Batch& b,
                               hipStream_t stream) {
  sg_status st = check_common(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy, form);
  if (st != SG_OK) return st;
  if ((st = check_batch(b)) != SG_OK) return st;
  if (!wv || !wmeta) return SG_ERR_NULL;
  if (ldwv < K / 2 || ldwm < K / 8 || ldwv >= (1LL << 24) || ldwm >= (1LL << 24)) return SG_ERR_SHAPE;
  if (!aligned(wv, 16) || !aligned(wmeta, 16) || ldwv % 16 || ldwm % 16) return SG_ERR_ALIGN;
  const GemmArgs a = make_args(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wv, ldwv, wmeta, ldwm, sw, sw_sn,
                               sw_sk, gran_n, y, y_dt, ldy, b);
  clear_hip_error();
  launch_gemm<true, false, I8>(a, gran_n, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}

template <bool I8>
static sg_status sparse24_gemm_packed(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx,
                                      const float* sx, int64_t sx_sm, int64_t sx_sk, int gran_m,
                                      const uint8_t* wpacked, const float* sw, int64_t sw_sn, int64_t sw_sk,
                                      int gran_n, void* y, sg_dtype y_dt, int64_t ldy, sg_form form,
                                      const Batch& b, hipStream_t stream) {
  sg_status st = check_common(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy, form);
  if (st != SG_OK) return st;
  if ((st = check_batch(b)) != SG_OK) return st;
  if (!wpacked) return SG_ERR_NULL;
  if (!aligned(wpacked, 16)) return SG_ERR_ALIGN;
  // the large-M kernel addresses a tile's 16 row blocks with 32-bit offsets
  if ((K / 128) * (int64_t)(BN / PK_ROWS) * PK_CHUNK > 0x7fffffffLL) return SG_ERR_SHAPE;
  const GemmArgs a = make_args(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wpacked, 0, nullptr, 0, sw, sw_sn,
                               sw_sk, gran_n, y, y_dt, ldy, b);
  clear_hip_error();
  launch_gemm<true, true, I8>(a, gran_n, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}

extern "C" sg_status sg_fp8_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                                    int64_t ldx, const float* sx, int64_t sx_sm,
                                                    int64_t sx_sk, int gran_m, const uint8_t* wv,
                                                    int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                                    const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                    int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                    sg_form form, hipStream_t stream) {
  return sparse24_gemm<false>(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wv, ldwv, wmeta, ldwm, sw, sw_sn, sw_sk,
                              gran_n, y, y_dt, ldy, form, Batch{}, stream);
}

// Activation quantisation fused into the packed 2:4 GEMM (decode sizes,
// M <= 64): X as fp32 or bf16, quantised per 1 x 128 block inside the kernel.
extern "C" sg_status sg_fp8_sparse24_gemm_packed_quant_x(int64_t M, int64_t N, int64_t K, const void* x,
                                                         sg_dtype x_dt, int64_t ldx, const uint8_t* wpacked,
                                                         const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                         int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                         sg_form form, hipStream_t stream) {
  if (!x || !wpacked || !sw || !y) return SG_ERR_NULL;
  if (x_dt != SG_F32 && x_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (gran_n != 128) return SG_ERR_UNSUPPORTED;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldx < K) return SG_ERR_SHAPE;
  if (M > 64) return SG_ERR_UNSUPPORTED;
  if (ldy < (form == SG_OUT_Y ? N : M) || cdiv(N, 16) > 0x7fffffffLL) return SG_ERR_SHAPE;
  const int64_t es = (int64_t)dtype_size(x_dt);
  // X rows and K-block offsets are 32-bit buffer offsets
  if (64 * ldx * es >= (1LL << 32) || K * es >= (1LL << 31) || sw_sn < 0 || sw_sk < 0) return SG_ERR_SHAPE;
  if (((cdiv(N, 128) - 1) * sw_sn + (K / 128 - 1) * sw_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if ((K / 128) * (int64_t)(BN / PK_ROWS) * PK_CHUNK > 0x7fffffffLL) return SG_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * es) % 16 || !aligned(wpacked, 16) || !aligned(sw, 4) ||
      !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  GemmArgs a = make_args(M, N, K, static_cast<const uint8_t*>(x), ldx, nullptr, 0, 0, 1, wpacked, 0, nullptr, 0, sw,
                         sw_sn, sw_sk, gran_n, y, y_dt, ldy, Batch{});
  const bool bf16 = y_dt == SG_BF16, yt = form == SG_OUT_YT;
  clear_hip_error();
  if (x_dt == SG_F32) {
    if (bf16) yt ? launch_decode_q<float, true, true>(a, stream) : launch_decode_q<float, true, false>(a, stream);
    else yt ? launch_decode_q<float, false, true>(a, stream) : launch_decode_q<float, false, false>(a, stream);
  } else {
    if (bf16) yt ? launch_decode_q<uint16_t, true, true>(a, stream) : launch_decode_q<uint16_t, true, false>(a, stream);
    else yt ? launch_decode_q<uint16_t, false, true>(a, stream) : launch_decode_q<uint16_t, false, false>(a, stream);
  }
  return launch_status();
}

extern "C" sg_status sg_fp8_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                                           int64_t ldx, const float* sx, int64_t sx_sm,
                                                           int64_t sx_sk, int gran_m, const uint8_t* wpacked,
                                                           const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                           int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                           sg_form form, hipStream_t stream) {
  return sparse24_gemm_packed<false>(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wpacked, sw, sw_sn, sw_sk, gran_n,
                                     y, y_dt, ldy, form, Batch{}, stream);
}

extern "C" sg_status sg_int8_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                                     int64_t ldx, const float* sx, int64_t sx_sm,
                                                     int64_t sx_sk, int gran_m, const int8_t* wv,
                                                     int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                                     const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                     int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                     sg_form form, hipStream_t stream) {
  return sparse24_gemm<true>(M, N, K, reinterpret_cast<const uint8_t*>(xq), ldx, sx, sx_sm, sx_sk, gran_m,
                             reinterpret_cast<const uint8_t*>(wv), ldwv, wmeta, ldwm, sw, sw_sn, sw_sk, gran_n, y,
                             y_dt, ldy, form, Batch{}, stream);
}

extern "C" sg_status sg_int8_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                                            int64_t ldx, const float* sx, int64_t sx_sm,
                                                            int64_t sx_sk, int gran_m, const uint8_t* wpacked,
                                                            const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                            int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                            sg_form form, hipStream_t stream) {
  return sparse24_gemm_packed<true>(M, N, K, reinterpret_cast<const uint8_t*>(xq), ldx, sx, sx_sm, sx_sk, gran_m,
                                    wpacked, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy, form, Batch{}, stream);
}

// Batched 2:4 GEMMs ("L" mode): L problems of one shape, each operand at its
// own batch stride.
extern "C" sg_status sg_fp8_sparse24_gemm_groupwise_batched(
    int64_t L, int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx, int64_t x_bs, const float* sx,
    int64_t sx_sm, int64_t sx_sk, int64_t sx_bs, int gran_m, const uint8_t* wv, int64_t ldwv, int64_t wv_bs,
    const uint8_t* wmeta, int64_t ldwm, int64_t wm_bs, const float* sw, int64_t sw_sn, int64_t sw_sk,
    int64_t sw_bs, int gran_n, const float* bias, int64_t bias_bs, void* y, sg_dtype y_dt, int64_t ldy,
    int64_t y_bs, sg_form form, hipStream_t stream) {
  Batch b;
  b.L = L; b.bx = x_bs; b.bw = wv_bs; b.bm = wm_bs; b.bsx = sx_bs; b.bsw = sw_bs; b.by = y_bs;
  b.bias = bias; b.bbs = bias_bs;
  return sparse24_gemm<false>(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wv, ldwv, wmeta, ldwm, sw, sw_sn, sw_sk,
                              gran_n, y, y_dt, ldy, form, b, stream);
}

extern "C" sg_status sg_fp8_sparse24_gemm_groupwise_packed_batched(
    int64_t L, int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx, int64_t x_bs, const float* sx,
    int64_t sx_sm, int64_t sx_sk, int64_t sx_bs, int gran_m, const uint8_t* wpacked, int64_t wp_bs,
    const float* sw, int64_t sw_sn, int64_t sw_sk, int64_t sw_bs, int gran_n, const float* bias,
    int64_t bias_bs, void* y, sg_dtype y_dt, int64_t ldy, int64_t y_bs, sg_form form, hipStream_t stream) {
  Batch b;
  b.L = L; b.bx = x_bs; b.bw = wp_bs; b.bsx = sx_bs; b.bsw = sw_bs; b.by = y_bs;
  b.bias = bias; b.bbs = bias_bs;
  return sparse24_gemm_packed<false>(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wpacked, sw, sw_sn, sw_sk, gran_n,
                                     y, y_dt, ldy, form, b, stream);
}

// Grouped 2:4 GEMM (one launch over every group's tiles; see GroupTable).
template <int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_grouped(const GemmArgs& a, const GroupTable& gt, hipStream_t st) {
  k_gemm_sparse_grouped<GRAN_N, OUT_BF16, OUT_T><<<(unsigned)gt.tile_start[gt.G], 512, 0, st>>>(a, gt);
}

template <int GRAN_N>
static void launch_grouped_form(const GemmArgs& a, const GroupTable& gt, bool bf16, bool yt, hipStream_t st) {
  if (bf16) {
    if (yt) launch_grouped<GRAN_N, true, true>(a, gt, st);
    else launch_grouped<GRAN_N, true, false>(a, gt, st);
  } else {
    if (yt) launch_grouped<GRAN_N, false, true>(a, gt, st);
    else launch_grouped<GRAN_N, false, false>(a, gt, st);
  }
}

// Decode-sized groups: RB row blocks per workgroup, the largest of 4, 2, 1
// whose ring fits LDS and that keeps at least 224 workgroups over all groups.
template <int RB, int MT, bool OUT_BF16, bool OUT_T>
static bool try_grouped_decode(const GemmArgs& a, const GroupTable& gt, hipStream_t st, int64_t rows16) {
  if constexpr (DmaCfg<RB, MT>::FITS) {
    if (RB == 1 || cdiv(rows16, RB) * gt.G >= 224) {
      k_gemm_decode_dma_grouped<false, RB, MT, 128, OUT_BF16, OUT_T>
          <<<dim3((unsigned)cdiv(rows16, RB), (unsigned)gt.G), 512, 0, st>>>(a, gt);
      return true;
    }
  }
  return false;
}

// False when no ring fits (nothing launched).
template <int MT, bool OUT_BF16, bool OUT_T>
static bool launch_grouped_decode_mt(const GemmArgs& a, const GroupTable& gt, hipStream_t st) {
  const int64_t rows16 = cdiv(a.N, 16);
  return try_grouped_decode<4, MT, OUT_BF16, OUT_T>(a, gt, st, rows16) ||
         try_grouped_decode<2, MT, OUT_BF16, OUT_T>(a, gt, st, rows16) ||
         try_grouped_decode<1, MT, OUT_BF16, OUT_T>(a, gt, st, rows16);
}

template <bool OUT_BF16, bool OUT_T>
static bool launch_grouped_decode(const GemmArgs& a, const GroupTable& gt, int64_t mmax, hipStream_t st) {
  if (mmax <= 16) return launch_grouped_decode_mt<1, OUT_BF16, OUT_T>(a, gt, st);
  if (mmax <= 32) return launch_grouped_decode_mt<2, OUT_BF16, OUT_T>(a, gt, st);
  if (mmax <= 48) return launch_grouped_decode_mt<3, OUT_BF16, OUT_T>(a, gt, st);
  return launch_grouped_decode_mt<4, OUT_BF16, OUT_T>(a, gt, st);
}

// Large tiles and tails in one launch (k_gemm_grouped_tails).
template <int GRAN_N>
static void launch_grouped_tails(const GemmArgs& a, const GroupTable& gt, const GroupTable& gtail, bool bf16,
                                 bool yt, hipStream_t st) {
  const int T = gt.tile_start[gt.G];
  const int tail_gx = (int)cdiv(cdiv(a.N, 16), 4);
  const unsigned blocks = (unsigned)(T + (int64_t)tail_gx * gt.G);
  if (bf16) {
    if (yt) k_gemm_grouped_tails<GRAN_N, true, true><<<blocks, 512, 0, st>>>(a, gt, gtail, T, tail_gx);
    else k_gemm_grouped_tails<GRAN_N, true, false><<<blocks, 512, 0, st>>>(a, gt, gtail, T, tail_gx);
  } else {
    if (yt) k_gemm_grouped_tails<GRAN_N, false, true><<<blocks, 512, 0, st>>>(a, gt, gtail, T, tail_gx);
    else k_gemm_grouped_tails<GRAN_N, false, false><<<blocks, 512, 0, st>>>(a, gt, gtail, T, tail_gx);
  }
}

extern "C" sg_status sg_fp8_sparse24_gemm_groupwise_packed_grouped(
    int64_t G, const int64_t* m_sizes, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx, const float* sx,
    int64_t sx_sm, int64_t sx_sk, const uint8_t* wpacked, int64_t wp_bs, const float* sw, int64_t sw_sn,
    int64_t sw_sk, int64_t sw_bs, int gran_n, const float* bias, int64_t bias_bs, void* y, sg_dtype y_dt,
    int64_t ldy, sg_form form, hipStream_t stream) {
  if (G <= 0 || G > MAX_GROUPS) return SG_ERR_SHAPE;
  if (!m_sizes) return SG_ERR_NULL;
  GroupTable gt;
  gt.G = (int)G;
  gt.row_off[0] = 0;
  for (int g = 0; g < G; ++g) {
    if (m_sizes[g] < 0) return SG_ERR_SHAPE;
    gt.row_off[g + 1] = gt.row_off[g] + m_sizes[g];
    gt.row_end[g] = gt.row_off[g + 1];
  }
  const int64_t M = gt.row_off[G];
  sg_status st = check_common(M, N, K, xq, ldx, sx, sx_sm, sx_sk, 1, sw, sw_sn, sw_sk, gran_n, y, y_dt, ldy, form);
  if (st != SG_OK) return st;
  Batch b;
  b.bw = wp_bs; b.bsw = sw_bs; b.bias = bias; b.bbs = bias_bs;
  if ((st = check_batch(b)) != SG_OK) return st;
  if (!wpacked) return SG_ERR_NULL;
  if (!aligned(wpacked, 16)) return SG_ERR_ALIGN;
  if ((K / 128) * (int64_t)(BN / PK_ROWS) * PK_CHUNK > 0x7fffffffLL) return SG_ERR_SHAPE;
  const int64_t tiles_n = cdiv(N, BN);
  gt.tiles_n = (int)tiles_n;
  gt.tile_start[0] = 0;
  for (int g = 0; g < G; ++g) {
    const int64_t t = gt.tile_start[g] + cdiv(m_sizes[g], BM) * tiles_n;
    if (t > 0x7fffffffLL) return SG_ERR_SHAPE;
    gt.tile_start[g + 1] = (int)t;
  }
  GemmArgs a = make_args(M, N, K, xq, ldx, sx, sx_sm, sx_sk, 1, wpacked, 0, nullptr, 0, sw, sw_sn, sw_sk, gran_n,
                         y, y_dt, ldy, b);
  // Y^T: a group's columns start at its row offset, so 16-byte stores need
  // every offset to keep 16-byte alignment.
  if (form == SG_OUT_YT)
    for (int g = 0; g < G; ++g)
      if ((gt.row_off[g] * (int64_t)dtype_size(y_dt)) % 16) a.vec16 = 0;
  clear_hip_error();
  const bool bf16 = y_dt == SG_BF16, yt = form == SG_OUT_YT;
  int64_t mmax = 0;
  for (int g = 0; g < G; ++g) mmax = std::max(mmax, m_sizes[g]);
  // decode-sized groups: the LDS-streaming decode kernel where one of its rings fits
  bool done = false;
  if (gran_n == 128 && mmax <= 64) {
    if (bf16) done = yt ? launch_grouped_decode<true, true>(a, gt, mmax, stream)
                        : launch_grouped_decode<true, false>(a, gt, mmax, stream);
    else done = yt ? launch_grouped_decode<false, true>(a, gt, mmax, stream)
                   : launch_grouped_decode<false, false>(a, gt, mmax, stream);
  }
  if (!done) {
    // Tails: a group's last rows past a multiple of 128, when there are at
    // most 64 of them, cost the large-M kernel a whole K loop per tile.  When
    // leaving them out saves the tiles a round over the CUs, the same launch
    // runs them with the LDS-streaming decode body instead (streaming their
    // group's weight once more), on the CUs the tiles leave idle.
    GroupTable gh = gt, gtail = gt;
    int64_t tail_max = 0;
    gh.tile_start[0] = 0;
    for (int g = 0; g < G; ++g) {
      const int64_t r = m_sizes[g] % BM, tail = (r > 0 && r <= 64) ? r : 0;
      tail_max = std::max(tail_max, tail);
      gh.row_end[g] = gt.row_off[g + 1] - tail;
      gh.tile_start[g + 1] = gh.tile_start[g] + (int)(cdiv(gh.row_end[g] - gt.row_off[g], BM) * tiles_n);
      gtail.row_off[g] = gt.row_off[g + 1] - tail;
    }
    const int cus = cu_count();
    const bool split = gran_n == 128 && tail_max > 0 && gh.tile_start[G] > 0 &&
                       cdiv(gh.tile_start[G], cus) < cdiv(gt.tile_start[G], cus);
    if (split) {
      if (sx_sk == 0 && sw_sk == 0) launch_grouped_tails<0>(a, gh, gtail, bf16, yt, stream);
      else launch_grouped_tails<128>(a, gh, gtail, bf16, yt, stream);
    } else if (sx_sk == 0 && sw_sk == 0) {
      launch_grouped_form<0>(a, gt, bf16, yt, stream);
    } else if (gran_n == 128) {
      launch_grouped_form<128>(a, gt, bf16, yt, stream);
    } else {
      launch_grouped_form<1>(a, gt, bf16, yt, stream);
    }
  }
  return launch_status();
}
