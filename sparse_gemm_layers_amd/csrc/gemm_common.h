// Epilogue helpers shared by the GEMM kernels: fp32 -> bf16/fp32 stores of
// one lane's 4 consecutive output rows, in the Y [M, N] or Y^T [N, M] layout,
// predicated on the partial M and N tiles.
#pragma once

#include "common.h"

namespace sg {

// LDS swizzles of operand rows: the 16-byte chunk c of row r is stored at
// chunk position c ^ swz(r).  Operand fragments are 16 rows read with
// ds_read_b128 (lane l reads row l % 16).  The functions below were chosen
// with gfx950's LDS bank-conflict counter: each makes its read pattern
// conflict-free, where the textbook c ^ (r & 7) on 128-byte rows costs four
// extra LDS cycles per read.  They depend on r mod 16 only.
//   swz8  - 128-byte rows, lane group g reads chunks 2 g and 2 g + 1 (fp8 operands)
//   swz8q - 128-byte rows, lane group g reads chunk 4 q + g (bf16 operands)
//   swz4  - 64-byte rows, lane group g reads chunk g
__device__ __host__ __forceinline__ int swz8(int r) { return (r & 6) ^ ((r >> 3) & 1); }
__device__ __host__ __forceinline__ int swz8q(int r) { return r & 6; }
__device__ __host__ __forceinline__ int swz4(int r) { return (r >> 1) & 3; }

// SMFMAC (v_smfmac_f32_16x16x128_fp8_fp8) A-operand layout: lane group g
// (lanes 16 g .. 16 g + 15) takes, from a row's 64 compressed bytes of a
// 128-wide K block, bytes [b, b + 8) and [b + 16, b + 24) with
// b = 32 (g & 1) + 8 (g >> 1); its 32-bit index holds the metadata nibbles of
// those 8 groups of 4, i.e. metadata bytes b/4, b/4 + 1, b/4 + 4, b/4 + 5 of
// the row's 16 metadata bytes, nibble order unchanged.
// Lane group g's 32-bit SMFMAC index from one row's 16 metadata bytes of a K block.
__device__ __forceinline__ int sp_meta_word(uint4 w, int g) {
  const uint32_t a = (g & 1) ? w.z : w.x;
  const uint32_t b = (g & 1) ? w.w : w.y;
  return (int)((g >> 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                        : __builtin_amdgcn_perm(b, a, 0x05040100u));
}

__device__ __forceinline__ int sp_a_off(int g) { return 32 * (g & 1) + 8 * (g >> 1); }

// gfx950 packed weight layout: one 1280-byte chunk per 16-row block R and
// 128-wide K block kb, at (R * KB + kb) * 1280, so that one row block's chunks
// follow each other along K.  Inside a chunk, local row lr's values for lane
// group g sit at pk_val_off(lr, g) and its index word at
// PK_META + pk_meta_word(lr, g).  The GEMM kernels' LDS image of a 256-row
// tile uses the same swizzle with the tile row r (it depends on r mod 16
// only): values at pk_val_off(r, g), index words at LDS_META + pk_meta_word(r, g).
constexpr int PK_ROWS = 16, PK_CHUNK = 1280, PK_META = 1024, LDS_META = 16384;
// Blocked int4 weight (the weight-only kernels' int4 form): one 768-byte chunk
// per 16-row block and K block at (R * KB + kb) * 768, the 16 rows' 32 code
// bytes row after row, then their 16 metadata bytes at PK4_META + lr * 16.
constexpr int PK4_CHUNK = 768, PK4_META = 512;
__device__ __host__ __forceinline__ int pk_val_off(int r, int g) { return r * 64 + 16 * (g ^ swz4(r)); }
__device__ __host__ __forceinline__ int pk_meta_word(int r, int g) { return r * 16 + 4 * ((g + 2 * ((r >> 3) & 1)) & 3); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS stage rings.  __syncthreads() also fences
// global memory, which makes the compiler wait for every load in flight,
// including the buffer loads that are filling later stages.  Here each wave
// first waits (vmcnt) for its own loads of the stage it is about to read;
// this barrier then waits for the wave's LDS reads to finish (so a stage read
// before the barrier may be refilled after it) and joins the waves.  The
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
        p.x = f32x2_to_bf16x2(v[0], v[1]);
        p.y = f32x2_to_bf16x2(v[2], v[3]);
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
