// Groupwise quantisers: fp32/bf16 -> e4m3 or int8 codes + one fp32 scale per
// block (1 x gc or 128 x gc), and fp32/bf16 -> packed int4 + one scale per
// (row, 128 columns).  Both are HBM-bound streaming kernels: every input
// byte is read once with 16- or 8-byte loads, codes are written once with
// 4- or 2-byte stores per lane, scales once per block.
//
// Block amax -> scale -> quantise follows CUTLASS PR #2095 "Improvements for:
// Groupwise scaling along M for FP8 gemm" (hwu36's comment on the
// ScaleGranularityM/N modes) and torchao PR #3258 "Introduce new W8A8-FP-CSR
// quantization API" (jcaip's review: positive scales, all-zero input allowed,
// scale then cast to float8_e4m3fn).  int8 (for the int8 x int8 2:4 GEMM the
// same torchao page names): s = amax / 127, codes rint-even clamped to +-127.
//
// Non-finite inputs (the pages say nothing of them): a block holding a NaN
// gets a NaN scale, a block holding an infinity (and no NaN) an infinite
// scale; codes are still the encoder applied to v / s, so finite values of
// such a block give zero codes and NaN quotients give 0x7F (e4m3) or 0 (int).
#include "common.h"

namespace sg {

enum QuantMode { Q_FP8 = 0, Q_INT8 = 2 };

// Integer code of v / sc, rounded half to even and clamped to +-qmax (an
// infinite quotient saturates); a NaN quotient gives code 0.
__device__ __forceinline__ int int_code(float v, float sc, float qmax) {
  const float t = __builtin_rintf(v / sc);                       // IEEE divide, half to even
  return t != t ? 0 : (int)fminf(fmaxf(t, -qmax), qmax);
}

// int8 code of v / sc as a byte (two's complement).
__device__ __forceinline__ uint32_t int8_encode(float v, float sc) { return (uint32_t)int_code(v, sc, 127.0f) & 0xffu; }

// ------------------------------------------------------------------ int4, 1 x 128
// LPB = GC/4 lanes share one block, 4 consecutive elements per lane (two
// codes per byte: 2-byte stores); a wave covers 64/LPB blocks per iteration
// of a grid-stride loop.
template <typename TIn, int GC>
__global__ void __launch_bounds__(256) k_quant_int4(const TIn* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                    float* __restrict__ s, int64_t ssr, int64_t ssc) {
  constexpr int LPB = GC / 4;
  constexpr int BPW = 64 / LPB;
  const int64_t nbc = cols / GC;
  const int64_t nblk = rows * nbc;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPB;
  const int li = lane % LPB;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t b0 = wave * BPW; b0 < nblk; b0 += nwaves * BPW) {
    const int64_t b = b0 + sub;
    const bool valid = b < nblk;
    const int64_t r = valid ? b / nbc : 0;
    const int64_t cb = valid ? b % nbc : 0;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) load4(x + r * ldx + cb * GC + li * 4, v);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) a = amax_fold(a, v[i]);
    a = group_max<LPB>(a);
    const float sc = block_scale(a, 7.0f);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= ((uint32_t)int_code(v[i], sc, 7.0f) & 0xfu) << (4 * i);
    if (valid) {
      *reinterpret_cast<uint16_t*>(q + r * ldq + cb * (GC / 2) + li * 2) = (uint16_t)packed;
      if (li == 0) s[r * ssr + cb * ssc] = sc;
    }
  }
}

// ------------------------------------------------------------------ 1 x GC, 16 per lane
// FP8 / int8 codes with one scale per (row, GC columns): each lane owns 16
// consecutive elements (four 16-byte fp32 loads or two bf16 loads in flight,
// one 16-byte code store), GC/16 lanes share a block, a wave covers
// 64 / (GC/16) blocks per iteration of a grid-stride loop.
template <typename TIn, int GC, int MODE>
__global__ void __launch_bounds__(256) k_quant_row16(const TIn* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                     float* __restrict__ s, int64_t ssr, int64_t ssc) {
  static_assert(MODE == Q_FP8 || MODE == Q_INT8, "byte codes only");
  constexpr int LPB = GC / 16;
  constexpr int BPW = 64 / LPB;
  const int64_t nbc = cols / GC;
  const int64_t nblk = rows * nbc;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPB, li = lane % LPB;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t b0 = wave * BPW; b0 < nblk; b0 += nwaves * BPW) {
    const int64_t b = b0 + sub;
    const bool valid = b < nblk;
    const int64_t r = valid ? b / nbc : 0;
    const int64_t cb = valid ? b % nbc : 0;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.f;
    if (valid) {
      const TIn* src = x + r * ldx + cb * GC + li * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) load4(src + 4 * i, v + 4 * i);
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = amax_fold(a, v[i]);
    a = group_max<LPB>(a);
    const float sc = block_scale(a, MODE == Q_FP8 ? 448.0f : 127.0f);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float* t = v + 4 * d;
      if (MODE == Q_FP8) {
        w[d] = e4m3_pack4(t[0] / sc, t[1] / sc, t[2] / sc, t[3] / sc);   // IEEE divides
      } else {
        w[d] = int8_encode(t[0], sc) | (int8_encode(t[1], sc) << 8) | (int8_encode(t[2], sc) << 16) |
               (int8_encode(t[3], sc) << 24);
      }
    }
    if (valid) {
      *reinterpret_cast<uint4*>(q + r * ldq + cb * GC + li * 16) = make_uint4(w[0], w[1], w[2], w[3]);
      if (li == 0) s[r * ssr + cb * ssc] = sc;
    }
  }
}

// ------------------------------------------------------------------ 128 x GC
// One 256-thread workgroup per block.  LPR = GC/4 lanes cover one row of the
// block; each thread keeps its STEPS x 4 inputs in registers between the amax
// reduction and the encode, so the block is read from HBM once.
template <typename TIn, int GC, int MODE>
__global__ void __launch_bounds__(256) k_quant_block128(const TIn* __restrict__ x, int64_t rows,
                                                        int64_t ldx, uint8_t* __restrict__ q,
                                                        int64_t ldq, float* __restrict__ s,
                                                        int64_t ssr, int64_t ssc) {
  constexpr int LPR = GC / 4;
  constexpr int RPS = 256 / LPR;
  constexpr int STEPS = 128 / RPS;
  __shared__ float red[4];
  const int64_t cb = blockIdx.x, rb = blockIdx.y;
  const int t = threadIdx.x;
  const int lr = t / LPR, li = t % LPR;
  float v[STEPS][4];
  float a = 0.f;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int64_t r = rb * 128 + st * RPS + lr;
    if (r < rows) {
      load4(x + r * ldx + cb * GC + li * 4, v[st]);
    } else {
      v[st][0] = v[st][1] = v[st][2] = v[st][3] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a = amax_fold(a, v[st][i]);
  }
  a = group_max<64>(a);
  if ((t & 63) == 0) red[t >> 6] = a;
  __syncthreads();
  a = amax_fold(amax_fold(amax_fold(red[0], red[1]), red[2]), red[3]);
  const float sc = block_scale(a, MODE == Q_FP8 ? 448.0f : 127.0f);
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int64_t r = rb * 128 + st * RPS + lr;
    const float* t = v[st];
    const uint32_t packed =
        MODE == Q_FP8 ? e4m3_pack4(t[0] / sc, t[1] / sc, t[2] / sc, t[3] / sc)
                      : (int8_encode(t[0], sc) | (int8_encode(t[1], sc) << 8) | (int8_encode(t[2], sc) << 16) |
                         (int8_encode(t[3], sc) << 24));
    if (r < rows) *reinterpret_cast<uint32_t*>(q + r * ldq + cb * GC + li * 4) = packed;
  }
  if (t == 0) s[rb * ssr + cb * ssc] = sc;
}

// ------------------------------------------------------------------ whole rows, whole tensor
// Scales constant along K: one scale per row (gc = cols) or one for the whole
// tensor (gr = rows, gc = cols).  Rows: one 256-thread workgroup per row, 16
// consecutive elements per thread and step; the first pass takes the row's
// amax, the second reads the row again (from L2) and encodes it.  Tensor: the
// amax comes first from k_amax_tensor (amax_in), and the encode pass reads it.
template <typename TIn>
__device__ __forceinline__ void load16(const TIn* p, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) load4(p + 4 * i, v + 4 * i);
}

template <typename TIn, int MODE>
__global__ void __launch_bounds__(256) k_quant_rowwide(const TIn* __restrict__ x, int64_t cols, int64_t ldx,
                                                       uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s,
                                                       int64_t ssr, const float* __restrict__ amax_in) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;
  const TIn* xr = x + r * ldx;
  float a;
  if (amax_in) {
    a = *amax_in;
  } else {
    a = 0.f;
    for (int64_t c = (int64_t)t * 16; c < cols; c += 256 * 16) {
      float v[16];
      load16(xr + c, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) a = amax_fold(a, v[i]);
    }
    a = group_max<64>(a);
    if ((t & 63) == 0) red[t >> 6] = a;
    __syncthreads();
    a = amax_fold(amax_fold(amax_fold(red[0], red[1]), red[2]), red[3]);
  }
  const float sc = block_scale(a, MODE == Q_FP8 ? 448.0f : 127.0f);
  for (int64_t c = (int64_t)t * 16; c < cols; c += 256 * 16) {
    float v[16];
    load16(xr + c, v);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float* e = v + 4 * d;
      w[d] = MODE == Q_FP8 ? e4m3_pack4(e[0] / sc, e[1] / sc, e[2] / sc, e[3] / sc)
                           : (int8_encode(e[0], sc) | (int8_encode(e[1], sc) << 8) |
                              (int8_encode(e[2], sc) << 16) | (int8_encode(e[3], sc) << 24));
    }
    *reinterpret_cast<uint4*>(q + r * ldq + c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (t == 0 && !amax_in) s[r * ssr] = sc;
}

// amax of the whole tensor into *slot (cleared first by k_fill1): each
// workgroup reduces its grid-stride share, then one atomic max per workgroup
// on the value's bits (non-negative floats order like their bit patterns);
// the grid is kept small so that few atomics meet at the one address.
template <typename TIn>
__global__ void __launch_bounds__(256) k_amax_tensor(const TIn* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t ldx, float* __restrict__ slot) {
  __shared__ float red[4];
  const int64_t per_row = cols / 16, items = rows * per_row;
  float a = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < items; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row, c = (i % per_row) * 16;
    float v[16];
    load16(x + r * ldx + c, v);
#pragma unroll
    for (int k = 0; k < 16; ++k) a = amax_fold(a, v[k]);
  }
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<unsigned int*>(slot),
              __float_as_uint(amax_fold(amax_fold(amax_fold(red[0], red[1]), red[2]), red[3])));
}

__global__ void k_fill1(float* p, float v) { *p = v; }

// The tensor's scale from its amax (in place).
template <int MODE>
__global__ void k_tensor_scale(float* s) {
  const float a = *s;
  *s = block_scale(a, MODE == Q_FP8 ? 448.0f : 127.0f);
}

template <typename TIn, int MODE>
static void launch_quant(const TIn* x, int64_t rows, int64_t cols, int64_t ldx, int gr, int gc,
                         uint8_t* q, int64_t ldq, float* s, int64_t ssr, int64_t ssc, hipStream_t st) {
  if ((gr != 1 && gr != 128) || (gc != 64 && gc != 128)) {
    // gc == cols: whole rows (gr == 1) or the whole tensor (gr == rows)
    if (gr == 1) {
      k_quant_rowwide<TIn, MODE><<<(unsigned)rows, 256, 0, st>>>(x, cols, ldx, q, ldq, s, ssr, nullptr);
    } else {
      k_fill1<<<1, 1, 0, st>>>(s, 0.f);
      k_amax_tensor<TIn><<<grid_for(rows * (cols / 16), 256, 512), 256, 0, st>>>(x, rows, cols, ldx, s);
      k_quant_rowwide<TIn, MODE><<<(unsigned)rows, 256, 0, st>>>(x, cols, ldx, q, ldq, nullptr, 0, s);
      k_tensor_scale<MODE><<<1, 1, 0, st>>>(s);
    }
  } else if (gr == 1) {
    const int64_t blocks = rows * (cols / gc);
    const int per_wg = 4 * (64 / (gc / 16));
    const unsigned g = grid_for(blocks, per_wg);
    if (gc == 128)
      k_quant_row16<TIn, 128, MODE><<<g, 256, 0, st>>>(x, rows, cols, ldx, q, ldq, s, ssr, ssc);
    else
      k_quant_row16<TIn, 64, MODE><<<g, 256, 0, st>>>(x, rows, cols, ldx, q, ldq, s, ssr, ssc);
  } else {
    const dim3 grid((unsigned)(cols / gc), (unsigned)cdiv(rows, 128));
    if (gc == 128)
      k_quant_block128<TIn, 128, MODE><<<grid, 256, 0, st>>>(x, rows, ldx, q, ldq, s, ssr, ssc);
    else
      k_quant_block128<TIn, 64, MODE><<<grid, 256, 0, st>>>(x, rows, ldx, q, ldq, s, ssr, ssc);
  }
}

}  // namespace sg

using namespace sg;

template <int MODE>
static sg_status quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx, int gr,
                                 int gc, uint8_t* q, int64_t ldq, float* s, int64_t s_stride_r, int64_t s_stride_c,
                                 hipStream_t stream) {
  if (!x || !q || !s) return SG_ERR_NULL;
  if (x_dt != SG_F32 && x_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  // 1 x {64, 128}, 128 x {64, 128}, one group per row (gr = 1, gc = cols) or
  // one for the tensor (gr = rows, gc = cols; cols a multiple of 16)
  const bool blocks = (gr == 1 || gr == 128) && (gc == 128 || gc == 64);
  const bool whole = gc == cols && (gr == 1 || gr == rows) && cols % 16 == 0 && cols > 0;
  if (!blocks && !whole) return SG_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || cols % gc != 0 || ldx < cols || ldq < cols) return SG_ERR_SHAPE;
  if (gr == 128 && cdiv(rows, gr) > 65535) return SG_ERR_SHAPE;
  if (!blocks && rows >= (1LL << 24)) return SG_ERR_SHAPE;   // one 256-thread workgroup per row
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4) || (ldx * (int64_t)dtype_size(x_dt)) % 16 ||
      ldq % 16)
    return SG_ERR_ALIGN;
  clear_hip_error();
  if (x_dt == SG_F32)
    launch_quant<float, MODE>((const float*)x, rows, cols, ldx, gr, gc, q, ldq, s, s_stride_r, s_stride_c, stream);
  else
    launch_quant<uint16_t, MODE>((const uint16_t*)x, rows, cols, ldx, gr, gc, q, ldq, s, s_stride_r, s_stride_c,
                                 stream);
  return launch_status();
}

extern "C" sg_status sg_fp8_quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows,
                                            int64_t cols, int64_t ldx, int gr, int gc, uint8_t* q,
                                            int64_t ldq, float* s, int64_t s_stride_r,
                                            int64_t s_stride_c, hipStream_t stream) {
  return quant_groupwise<Q_FP8>(x, x_dt, rows, cols, ldx, gr, gc, q, ldq, s, s_stride_r, s_stride_c, stream);
}

extern "C" sg_status sg_int8_quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows,
                                             int64_t cols, int64_t ldx, int gr, int gc, int8_t* q,
                                             int64_t ldq, float* s, int64_t s_stride_r,
                                             int64_t s_stride_c, hipStream_t stream) {
  return quant_groupwise<Q_INT8>(x, x_dt, rows, cols, ldx, gr, gc, reinterpret_cast<uint8_t*>(q), ldq, s,
                                 s_stride_r, s_stride_c, stream);
}

extern "C" sg_status sg_int4_quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows,
                                             int64_t cols, int64_t ldx, int gc, uint8_t* q, int64_t ldq,
                                             float* s, int64_t s_stride_r, int64_t s_stride_c,
                                             hipStream_t stream) {
  if (!x || !q || !s) return SG_ERR_NULL;
  if (x_dt != SG_F32 && x_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (gc != 128 && gc != 64) return SG_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || cols % gc != 0 || ldx < cols || ldq < cols / 2) return SG_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s, 4) || (ldx * (int64_t)dtype_size(x_dt)) % 16 ||
      ldq % 4)
    return SG_ERR_ALIGN;
  clear_hip_error();
  const int64_t blocks = rows * (cols / gc);
  const unsigned g = grid_for(blocks, 4 * (64 / (gc / 4)));
  if (x_dt == SG_F32) {
    if (gc == 128)
      k_quant_int4<float, 128><<<g, 256, 0, stream>>>((const float*)x, rows, cols, ldx, q, ldq, s, s_stride_r,
                                                       s_stride_c);
    else
      k_quant_int4<float, 64><<<g, 256, 0, stream>>>((const float*)x, rows, cols, ldx, q, ldq, s, s_stride_r,
                                                      s_stride_c);
  } else {
    if (gc == 128)
      k_quant_int4<uint16_t, 128><<<g, 256, 0, stream>>>((const uint16_t*)x, rows, cols, ldx, q, ldq, s,
                                                          s_stride_r, s_stride_c);
    else
      k_quant_int4<uint16_t, 64><<<g, 256, 0, stream>>>((const uint16_t*)x, rows, cols, ldx, q, ldq, s,
                                                         s_stride_r, s_stride_c);
  }
  return launch_status();
}
