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
#include "gemm_common.h"

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
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ v4f mma_dense(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mma_sparse(const v4i& a, const v8i& b, int idx) {
  v4f p = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, p, idx, 0, 0);
}

// Lane group g's 32-bit SMFMAC index from one row's 16 metadata bytes of a K block.
__device__ __forceinline__ int sp_meta_word(uint4 w, int g) {
  const uint32_t a = (g & 1) ? w.z : w.x;
  const uint32_t b = (g & 1) ? w.w : w.y;
  return (int)((g >> 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                        : __builtin_amdgcn_perm(b, a, 0x05040100u));
}

__device__ __forceinline__ int sp_a_off(int g) { return 32 * (g & 1) + 8 * (g >> 1); }

// ============================================================ large-M kernel
// Workgroup tile: 256 W rows (n) x 128 X rows (m), 4 waves in a 2 x 2 grid,
// each wave 128 n x 64 m = 8 x 4 sub-tiles of 16 x 16.  One 128-wide K block
// per stage, two stages in LDS (register-staged double buffering: the global
// loads of block kb+1 are in flight while block kb is multiplied).
//
// LDS stage layout (bytes):
//   X    : 128 rows x 128 B; 16-byte chunk c of row r at chunk c ^ (r & 7)
//   W    : dense 256 rows x 128 B (same swizzle as X), or
//          sparse 256 rows x 64 B of values; 16-byte slot s holds lane group
//          s's operand bytes; slot s of row r at s ^ ((r >> 1) & 3)
//   meta : sparse only, 256 rows x 16 B, word g = lane group g's index
//   sx   : 128 floats (scale of X row r for this K block)
//   sw   : 256 floats (scale of W row r for this K block)
constexpr int BN = 256, BM = 128;
constexpr int X_BYTES = BM * 128;

template <bool SPARSE>
struct Stage {
  static constexpr int W_BYTES = SPARSE ? BN * 64 : BN * 128;
  static constexpr int M_BYTES = SPARSE ? BN * 16 : 0;
  static constexpr int X_OFF = 0;
  static constexpr int W_OFF = X_OFF + X_BYTES;
  static constexpr int M_OFF = W_OFF + W_BYTES;
  static constexpr int SX_OFF = M_OFF + M_BYTES;
  static constexpr int SW_OFF = SX_OFF + BM * 4;
  static constexpr int BYTES = SW_OFF + BN * 4;
};

template <bool SPARSE>
struct Staged {
  uint4 x[4];
  uint4 w[SPARSE ? 4 : 8];
  uint4 m;
  float sx, sw;
};

template <bool SPARSE>
__device__ __forceinline__ void stage_load(const GemmArgs& a, int64_t n0, int64_t m0, int kb, int t,
                                           Staged<SPARSE>& s) {
  const uint4 zero = {0u, 0u, 0u, 0u};
  // X: 1024 chunks of 16 B, 8 per row
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = t + 256 * j;
    const int r = i >> 3, c = i & 7;
    const int64_t m = m0 + r;
    s.x[j] = m < a.M ? *reinterpret_cast<const uint4*>(a.x + m * a.ldx + (int64_t)kb * 128 + c * 16) : zero;
  }
  if (SPARSE) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 2, c = i & 3;
      const int64_t n = n0 + r;
      s.w[j] = n < a.N ? *reinterpret_cast<const uint4*>(a.w + n * a.ldw + (int64_t)kb * 64 + c * 16) : zero;
    }
    const int64_t n = n0 + t;
    s.m = n < a.N ? *reinterpret_cast<const uint4*>(a.meta + n * a.ldm + (int64_t)kb * 16) : zero;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 3, c = i & 7;
      const int64_t n = n0 + r;
      s.w[j] = n < a.N ? *reinterpret_cast<const uint4*>(a.w + n * a.ldw + (int64_t)kb * 128 + c * 16) : zero;
    }
  }
  {
    const int64_t m = m0 + (t & 127);
    s.sx = (t < 128 && m < a.M) ? a.sx[(m >> a.gm_shift) * a.sx_sm + (int64_t)kb * a.sx_sk] : 0.f;
    const int64_t n = n0 + t;
    s.sw = n < a.N ? a.sw[(n >> a.gn_shift) * a.sw_sn + (int64_t)kb * a.sw_sk] : 0.f;
  }
}

template <bool SPARSE>
__device__ __forceinline__ void stage_store(uint8_t* st, int t, const Staged<SPARSE>& s) {
  using L = Stage<SPARSE>;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = t + 256 * j;
    const int r = i >> 3, c = i & 7;
    *reinterpret_cast<uint4*>(st + L::X_OFF + r * 128 + ((c ^ (r & 7)) << 4)) = s.x[j];
  }
  if (SPARSE) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 2, c = i & 3;
      const int sw = (r >> 1) & 3;
      // low 8 B = 8-byte chunk 2c -> slot c>>1; high 8 B = chunk 2c+1 -> slot 2 + (c>>1);
      // both in half (c & 1) of their slot
      uint8_t* row = st + L::W_OFF + r * 64 + ((c & 1) << 3);
      *reinterpret_cast<uint2*>(row + ((((c >> 1)) ^ sw) << 4)) = make_uint2(s.w[j].x, s.w[j].y);
      *reinterpret_cast<uint2*>(row + (((2 + (c >> 1)) ^ sw) << 4)) = make_uint2(s.w[j].z, s.w[j].w);
    }
    uint4 o;
    o.x = sp_meta_word(s.m, 0);
    o.y = sp_meta_word(s.m, 1);
    o.z = sp_meta_word(s.m, 2);
    o.w = sp_meta_word(s.m, 3);
    *reinterpret_cast<uint4*>(st + L::M_OFF + t * 16) = o;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t + 256 * j;
      const int r = i >> 3, c = i & 7;
      *reinterpret_cast<uint4*>(st + L::W_OFF + r * 128 + ((c ^ (r & 7)) << 4)) = s.w[j];
    }
  }
  if (t < 128) reinterpret_cast<float*>(st + L::SX_OFF)[t] = s.sx;
  reinterpret_cast<float*>(st + L::SW_OFF)[t] = s.sw;
}

template <bool SPARSE, int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(256, 1) k_gemm_large(GemmArgs a, int tiles_m, int tiles_n) {
  using L = Stage<SPARSE>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::BYTES];

  // Workgroups go to the 8 XCDs round-robin.  Renumber so that each XCD owns
  // a contiguous range of tile ids, then walk tiles in groups of 4 n-tiles so
  // that an XCD's tiles share W rows and X rows in its L2.
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
  const int KB = (int)(a.K >> 7);

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  Staged<SPARSE> stg;
  stage_load<SPARSE>(a, n0, m0, 0, t, stg);
  stage_store<SPARSE>(smem, t, stg);
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const uint8_t* st = smem + (kb & 1) * L::BYTES;
    if (kb + 1 < KB) stage_load<SPARSE>(a, n0, m0, kb + 1, t, stg);

    // scales of this K block
    const float* sxs = reinterpret_cast<const float*>(st + L::SX_OFF);
    const float* sws = reinterpret_cast<const float*>(st + L::SW_OFF);
    float sxj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sxj[j] = sxs[wm * 64 + j * 16 + lr];

    // X operands (B side) of the wave's 4 column sub-tiles
    v8i bx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wm * 64 + j * 16 + lr;
      const uint8_t* row = st + L::X_OFF + r * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(row + (((2 * g) ^ (r & 7)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(row + (((2 * g + 1) ^ (r & 7)) << 4));
      bx[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wn * 128 + i * 16 + lr;
      float s[4];
      if (GRAN_N == 128) {
        const float swv = sws[wn * 128];
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = sxj[j] * swv;
      }
      float4 swr;
      if (GRAN_N == 1) swr = *reinterpret_cast<const float4*>(sws + wn * 128 + i * 16 + 4 * g);
      if (SPARSE) {
        const int sl = g ^ ((r >> 1) & 3);
        const uint4 av = *reinterpret_cast<const uint4*>(st + L::W_OFF + r * 64 + (sl << 4));
        const int idx = *reinterpret_cast<const int*>(st + L::M_OFF + r * 16 + g * 4);
        const v4i aa = {(int)av.x, (int)av.y, (int)av.z, (int)av.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f p = mma_sparse(aa, bx[j], idx);
          if (GRAN_N == 128) {
            acc[i][j] += p * s[j];
          } else {
            acc[i][j][0] = fmaf(p[0] * swr.x, sxj[j], acc[i][j][0]);
            acc[i][j][1] = fmaf(p[1] * swr.y, sxj[j], acc[i][j][1]);
            acc[i][j][2] = fmaf(p[2] * swr.z, sxj[j], acc[i][j][2]);
            acc[i][j][3] = fmaf(p[3] * swr.w, sxj[j], acc[i][j][3]);
          }
        }
      } else {
        const uint8_t* row = st + L::W_OFF + r * 128;
        const uint4 lo = *reinterpret_cast<const uint4*>(row + (((2 * g) ^ (r & 7)) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(row + (((2 * g + 1) ^ (r & 7)) << 4));
        const v8i aa = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f p = mma_dense(aa, bx[j]);
          if (GRAN_N == 128) {
            acc[i][j] += p * s[j];
          } else {
            acc[i][j][0] = fmaf(p[0] * swr.x, sxj[j], acc[i][j][0]);
            acc[i][j][1] = fmaf(p[1] * swr.y, sxj[j], acc[i][j][1]);
            acc[i][j][2] = fmaf(p[2] * swr.z, sxj[j], acc[i][j][2]);
            acc[i][j][3] = fmaf(p[3] * swr.w, sxj[j], acc[i][j][3]);
          }
        }
      }
    }

    if (kb + 1 < KB) stage_store<SPARSE>(smem + ((kb + 1) & 1) * L::BYTES, t, stg);
    __syncthreads();
  }

  // Epilogue: lane holds D[n = n0 + wn*128 + 16 i + 4 g + e][m = m0 + wm*64 + 16 j + lr].
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_quad<OUT_BF16, OUT_T>(a, m0 + wm * 64 + j * 16 + lr, n0 + wn * 128 + i * 16 + 4 * g, acc[i][j]);
}

// ============================================================ decode kernel
// For M <= 64 (decode-sized batches).  A workgroup owns 16 W rows and all M
// columns (MT sub-tiles of 16); its 8 waves split the K blocks (wave w takes
// kb = w, w + 8, ...), read their operands straight from global memory into
// the matrix-core layout (the weight is streamed once from HBM; X is small
// and stays in L2), and finally add their partial tiles through LDS.
// Columns m >= M are zero-filled (the partial M tile).
constexpr int DEC_WAVES = 8;

template <bool SPARSE, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
__global__ void __launch_bounds__(512) k_gemm_decode(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) float red[DEC_WAVES][MT][64][4];
  const int t = threadIdx.x, l = t & 63, wave = t >> 6;
  const int g = l >> 4, lr = l & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + lr;            // this lane's W row (A operand)
  const bool n_ok = n < a.N;
  const int KB = (int)(a.K >> 7);

  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int kb = wave; kb < KB; kb += DEC_WAVES) {
    const int64_t k0 = (int64_t)kb * 128;
    // A operand (W rows n0..n0+15)
    v4i asp;
    v8i ad;
    int idx = 0;
    if (SPARSE) {
      uint2 lo = {0u, 0u}, hi = {0u, 0u};
      uint4 mw = {0u, 0u, 0u, 0u};
      if (n_ok) {
        const uint8_t* wr = a.w + n * a.ldw + k0 / 2 + sp_a_off(g);
        lo = *reinterpret_cast<const uint2*>(wr);
        hi = *reinterpret_cast<const uint2*>(wr + 16);
        mw = *reinterpret_cast<const uint4*>(a.meta + n * a.ldm + k0 / 8);
      }
      asp = (v4i){(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
      idx = sp_meta_word(mw, g);
    } else {
      uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (n_ok) {
        const uint8_t* wr = a.w + n * a.ldw + k0 + 32 * g;
        lo = *reinterpret_cast<const uint4*>(wr);
        hi = *reinterpret_cast<const uint4*>(wr + 16);
      }
      ad = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    // W scale(s) of this K block
    float sw4[4];
    if (GRAN_N == 128) {
      const float v = a.sw[(n0 >> 7) * a.sw_sn + kb * a.sw_sk];
      sw4[0] = sw4[1] = sw4[2] = sw4[3] = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ne = n0 + 4 * g + e;
        sw4[e] = ne < a.N ? a.sw[ne * a.sw_sn + kb * a.sw_sk] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int64_t m = j * 16 + lr;
      uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      float sxv = 0.f;
      if (m < a.M) {
        const uint8_t* xr = a.x + m * a.ldx + k0 + 32 * g;
        lo = *reinterpret_cast<const uint4*>(xr);
        hi = *reinterpret_cast<const uint4*>(xr + 16);
        sxv = a.sx[(m >> a.gm_shift) * a.sx_sm + kb * a.sx_sk];
      }
      const v8i bx = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const v4f p = SPARSE ? mma_sparse(asp, bx, idx) : mma_dense(ad, bx);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] = fmaf(p[e] * sw4[e], sxv, acc[j][e]);
    }
  }

#pragma unroll
  for (int j = 0; j < MT; ++j)
    *reinterpret_cast<float4*>(&red[wave][j][l][0]) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
  __syncthreads();
  // 512 threads: thread -> (sub-tile j, lane ll); MT * 64 lanes of 4 values
  for (int q = t; q < MT * 64; q += 512) {
    const int j = q >> 6, ll = q & 63;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[w][j][ll][0]);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const v4f out = {s.x, s.y, s.z, s.w};
    store_quad<OUT_BF16, OUT_T>(a, (int64_t)j * 16 + (ll & 15), n0 + 4 * (ll >> 4), out);
  }
}

// ------------------------------------------------------------------ dispatch

template <bool SPARSE, int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_large(const GemmArgs& a, hipStream_t st) {
  const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
  k_gemm_large<SPARSE, GRAN_N, OUT_BF16, OUT_T><<<tm * tn, 256, 0, st>>>(a, tm, tn);
}

template <bool SPARSE, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_decode_mt(const GemmArgs& a, hipStream_t st) {
  k_gemm_decode<SPARSE, MT, GRAN_N, OUT_BF16, OUT_T><<<(unsigned)cdiv(a.N, 16), 512, 0, st>>>(a);
}

template <bool SPARSE, int GRAN_N, bool OUT_BF16, bool OUT_T>
static void launch_shape(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 16)
    launch_decode_mt<SPARSE, 1, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 32)
    launch_decode_mt<SPARSE, 2, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 48)
    launch_decode_mt<SPARSE, 3, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else if (a.M <= 64)
    launch_decode_mt<SPARSE, 4, GRAN_N, OUT_BF16, OUT_T>(a, st);
  else
    launch_large<SPARSE, GRAN_N, OUT_BF16, OUT_T>(a, st);
}

template <bool SPARSE>
static void launch_gemm(const GemmArgs& a, int gran_n, bool bf16, bool yt, hipStream_t st) {
  if (gran_n == 128) {
    if (bf16) {
      if (yt) launch_shape<SPARSE, 128, true, true>(a, st); else launch_shape<SPARSE, 128, true, false>(a, st);
    } else {
      if (yt) launch_shape<SPARSE, 128, false, true>(a, st); else launch_shape<SPARSE, 128, false, false>(a, st);
    }
  } else {
    if (bf16) {
      if (yt) launch_shape<SPARSE, 1, true, true>(a, st); else launch_shape<SPARSE, 1, true, false>(a, st);
    } else {
      if (yt) launch_shape<SPARSE, 1, false, true>(a, st); else launch_shape<SPARSE, 1, false, false>(a, st);
    }
  }
}

// Common argument checks of both GEMM entry points (host only, before any HIP call).
static sg_status check_common(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx,
                              const float* sx, int gran_m, const float* sw, int gran_n, void* y,
                              sg_dtype y_dt, int64_t ldy, sg_form form) {
  if (!xq || !sx || !sw || !y) return SG_ERR_NULL;
  if ((gran_m != 1 && gran_m != 128) || (gran_n != 1 && gran_n != 128)) return SG_ERR_UNSUPPORTED;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K <= 0 || K % 128 != 0 || ldx < K) return SG_ERR_SHAPE;
  if (ldy < (form == SG_OUT_Y ? N : M)) return SG_ERR_SHAPE;
  if (cdiv(M, 128) * cdiv(N, 256) > 0x7fffffffLL || cdiv(N, 16) > 0x7fffffffLL) return SG_ERR_SHAPE;
  if (!aligned(xq, 16) || ldx % 16 || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  return SG_OK;
}

static GemmArgs make_args(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx,
                          const float* sx, int64_t sx_sm, int64_t sx_sk, int gran_m, const uint8_t* w,
                          int64_t ldw, const uint8_t* meta, int64_t ldm, const float* sw, int64_t sw_sn,
                          int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt, int64_t ldy) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.x = xq; a.ldx = ldx;
  a.sx = sx; a.sx_sm = sx_sm; a.sx_sk = sx_sk; a.gm_shift = gran_m == 128 ? 7 : 0;
  a.w = w; a.ldw = ldw; a.meta = meta; a.ldm = ldm;
  a.sw = sw; a.sw_sn = sw_sn; a.sw_sk = sw_sk; a.gn_shift = gran_n == 128 ? 7 : 0;
  a.y = y; a.ldy = ldy;
  const size_t vb = 4 * dtype_size(y_dt);
  a.vec_store = (ldy % 4 == 0) && aligned(y, vb);
  return a;
}

}  // namespace sg

using namespace sg;

extern "C" sg_status sg_fp8_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                           int64_t ldx, const float* sx, int64_t sx_sm,
                                           int64_t sx_sk, int gran_m, const uint8_t* wq,
                                           int64_t ldw, const float* sw, int64_t sw_sn,
                                           int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt,
                                           int64_t ldy, sg_form form, hipStream_t stream) {
  sg_status st = check_common(M, N, K, xq, ldx, sx, gran_m, sw, gran_n, y, y_dt, ldy, form);
  if (st != SG_OK) return st;
  if (!wq) return SG_ERR_NULL;
  if (ldw < K) return SG_ERR_SHAPE;
  if (!aligned(wq, 16) || ldw % 16) return SG_ERR_ALIGN;
  if (M == 0 || N == 0) return SG_OK;
  const GemmArgs a = make_args(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wq, ldw, nullptr, 0, sw, sw_sn,
                               sw_sk, gran_n, y, y_dt, ldy);
  clear_hip_error();
  launch_gemm<false>(a, gran_n, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}

extern "C" sg_status sg_fp8_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                                    int64_t ldx, const float* sx, int64_t sx_sm,
                                                    int64_t sx_sk, int gran_m, const uint8_t* wv,
                                                    int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                                    const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                    int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                    sg_form form, hipStream_t stream) {
  sg_status st = check_common(M, N, K, xq, ldx, sx, gran_m, sw, gran_n, y, y_dt, ldy, form);
  if (st != SG_OK) return st;
  if (!wv || !wmeta) return SG_ERR_NULL;
  if (ldwv < K / 2 || ldwm < K / 8) return SG_ERR_SHAPE;
  if (!aligned(wv, 16) || !aligned(wmeta, 16) || ldwv % 16 || ldwm % 16) return SG_ERR_ALIGN;
  if (M == 0 || N == 0) return SG_OK;
  const GemmArgs a = make_args(M, N, K, xq, ldx, sx, sx_sm, sx_sk, gran_m, wv, ldwv, wmeta, ldwm, sw, sw_sn,
                               sw_sk, gran_n, y, y_dt, ldy);
  clear_hip_error();
  launch_gemm<true>(a, gran_n, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}
