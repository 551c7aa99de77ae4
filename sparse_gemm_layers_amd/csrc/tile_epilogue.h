// Workgroup tile order and the staged epilogue shared by the 8-wave GEMM
// kernels (256 W rows x 128 X rows per workgroup, two K groups of 4 waves in
// a 2 x 2 grid, each wave 128 n x 64 m = 8 x 4 sub-tiles of 16 x 16).
#pragma once

#include "gemm_common.h"

namespace sg {

constexpr int TILE_N = 256, TILE_M = 128;

// Workgroups go to the 8 XCDs round-robin.  Renumber so that each XCD owns a
// contiguous range of tile ids, then walk tiles in groups of 4 n-tiles so that
// the tiles resident on one XCD share W rows and X rows in its L2.
__device__ __forceinline__ int xcd_order(int b, int T) {
  return (T & 7) == 0 ? (b & 7) * (T >> 3) + (b >> 3) : b;
}

// Tile b (in the XCD order) of a tiles_m x tiles_n grid.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tn, int& tm) {
  const int G = 4;
  const int group = b / (G * tiles_m);
  const int first_n = group * G;
  const int gsize = min(tiles_n - first_n, G);
  const int in_g = b - group * G * tiles_m;
  tn = first_n + in_g % gsize;
  tm = in_g / gsize;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tn, int& tm) {
  tile_of(xcd_order(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, tn, tm);
}

// Partial-tile exchange between the two K groups (rows I0 .. I0+3 of the
// wave's 8 x 4 sub-tiles).
template <int I0>
__device__ __forceinline__ void xchg_out(float4* dst, const v4f (&acc)[8][4], int w4, int l) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f v = acc[I0 + i][j];
      dst[((w4 * 16 + i * 4 + j) << 6) + l] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// The finished 256 x 128 tile is staged in LDS in the stored layout (rows of
// Y are m, rows of Y^T are n), 16 bytes of padding per row, the first half of
// the rows in one double-stage buffer and the second half in the other, so
// that the stores are whole, 16-byte aligned row segments.
template <bool OUT_BF16, bool OUT_T, int BUF>
struct OutTile {
  static constexpr int ES = OUT_BF16 ? 2 : 4;
  static constexpr int ROWS = OUT_T ? TILE_N : TILE_M;
  static constexpr int COLS = OUT_T ? TILE_M : TILE_N;
  static constexpr int PITCH = COLS * ES + 16;
  static constexpr int RPH = ROWS / 2;          // rows per buffer
  static constexpr int CPR = COLS * ES / 16;    // 16-byte chunks per row
  static_assert(RPH * PITCH <= BUF, "half of the output tile must fit one buffer");
};

// Group Q's finished rows (Q = 0: sub-tile rows i < 4, Q = 1: i >= 4): adds
// the partner group's partial tile (16 float4 per lane in buffer `src`) and
// writes the result into the staged output tile.  Lane holds
// D[n = wn*128 + 16 i + 4 g + e][m = wm*64 + 16 j + lr].
// Writes one lane's four results D[nl + e][ml] (e = 0..3, tile-local
// indices) into the staged output tile.
template <bool OUT_BF16, bool OUT_T, int BUF>
__device__ __forceinline__ void stage_quad(uint8_t* t0, uint8_t* t1, int nl, int ml, const float (&v)[4]) {
  using OT = OutTile<OUT_BF16, OUT_T, BUF>;
  if (!OUT_T) {
    uint8_t* row = (ml < OT::RPH ? t0 : t1) + (ml % OT::RPH) * OT::PITCH;
    if (OUT_BF16) {
      uint2 pk;
      pk.x = f32x2_to_bf16x2(v[0], v[1]);
      pk.y = f32x2_to_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(row + nl * 2) = pk;
    } else {
      *reinterpret_cast<float4*>(row + nl * 4) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint8_t* row = (nl + e < OT::RPH ? t0 : t1) + ((nl + e) % OT::RPH) * OT::PITCH;
      if (OUT_BF16) *reinterpret_cast<uint16_t*>(row + ml * 2) = (uint16_t)f32_to_bf16(v[e]);
      else *reinterpret_cast<float*>(row + ml * 4) = v[e];
    }
  }
}

// SCALE = 0: the sums are final.  SCALE = 1 (fp32 sums) or 2 (exact int32
// sums, added as integers): scales constant along K are applied here, once:
// sxp[16 j] is the X scale of the lane's column in sub-tile column j and
// swp[16 i' + e] the W scale of row 16 i' + e (i' = 4 Q + i) of the wave's
// rows; both live in LDS that the exchange and the staged tile leave alone.
// bias (NULL: none) points at the tile's first row's bias; tile rows at or
// past nlim read bias[nlim - 1] (they are not stored).
template <int Q, bool OUT_BF16, bool OUT_T, int BUF, int SCALE = 0>
__device__ __forceinline__ void x2_finish(const uint8_t* src, uint8_t* t0, uint8_t* t1, const v4f (&acc)[8][4],
                                          int w4, int l, int wn, int wm, int g, int lr,
                                          const float* sxp = nullptr, const float* swp = nullptr,
                                          const float* bias = nullptr, int nlim = 0) {
  float4 part[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) part[k] = reinterpret_cast<const float4*>(src)[((w4 * 16 + k) << 6) + l];
  __syncthreads();   // every wave has its partner's partials: the buffers may be overwritten
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 sw = make_float4(1.f, 1.f, 1.f, 1.f);
    if (SCALE) sw = *reinterpret_cast<const float4*>(swp + (4 * Q + i) * 16);
    const int nl = wn * 128 + (4 * Q + i) * 16 + 4 * g;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = bias[min(nl + e, nlim - 1)];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 o = part[i * 4 + j];
      const v4f av = acc[4 * Q + i][j];
      float v[4];
      if (SCALE == 2) {
        const v4i ai = __builtin_bit_cast(v4i, av);
        const int4 oi = __builtin_bit_cast(int4, o);
        v[0] = (float)(ai[0] + oi.x); v[1] = (float)(ai[1] + oi.y);
        v[2] = (float)(ai[2] + oi.z); v[3] = (float)(ai[3] + oi.w);
      } else {
        v[0] = av[0] + o.x; v[1] = av[1] + o.y; v[2] = av[2] + o.z; v[3] = av[3] + o.w;
      }
      if (SCALE) {
        const float sx = sxp[16 * j];
        v[0] *= sw.x * sx; v[1] *= sw.y * sx; v[2] *= sw.z * sx; v[3] *= sw.w * sx;
      }
      v[0] += bv[0]; v[1] += bv[1]; v[2] += bv[2]; v[3] += bv[3];
      stage_quad<OUT_BF16, OUT_T, BUF>(t0, t1, nl, wm * 64 + j * 16 + lr, v);
    }
  }
}

// Stores the staged tile: 16-byte chunks of whole rows, non-temporal (the
// output is not read again by this kernel).  Partial tiles and outputs
// without 16-byte rows store element by element with bounds checks.
template <bool OUT_BF16, bool OUT_T, int BUF, typename Args>
__device__ __forceinline__ void store_staged(const Args& a, const uint8_t* t0, const uint8_t* t1, int64_t m0,
                                             int64_t n0, int t) {
  using OT = OutTile<OUT_BF16, OUT_T, BUF>;
  const int64_t r0 = OUT_T ? n0 : m0, c0 = OUT_T ? m0 : n0;
  const int64_t rlim = OUT_T ? a.N : a.M, clim = OUT_T ? a.M : a.N;
  const bool full = r0 + OT::ROWS <= rlim && c0 + OT::COLS <= clim && a.vec16;
  constexpr int CHUNKS = OT::ROWS * OT::CPR;
#pragma unroll
  for (int u = 0; u < CHUNKS / 512; ++u) {
    const int c = u * 512 + t, row = c / OT::CPR, col = c % OT::CPR;
    const uint4 v = *reinterpret_cast<const uint4*>((row < OT::RPH ? t0 : t1) + (row % OT::RPH) * OT::PITCH + col * 16);
    uint8_t* const yp = reinterpret_cast<uint8_t*>(a.y) + ((r0 + row) * a.ldy + c0 + col * (16 / OT::ES)) * OT::ES;
    if (full) {
      typedef unsigned int u4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store((u4v){v.x, v.y, v.z, v.w}, reinterpret_cast<u4v*>(yp));
    } else if (r0 + row < rlim) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 16 / OT::ES; ++e) {
        if (c0 + col * (16 / OT::ES) + e < clim) {
          if (OUT_BF16) reinterpret_cast<uint16_t*>(yp)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          else reinterpret_cast<uint32_t*>(yp)[e] = w[e];
        }
      }
    }
  }
}

}  // namespace sg
