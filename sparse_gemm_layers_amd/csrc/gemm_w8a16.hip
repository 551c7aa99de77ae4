// Weight-only 2:4 GEMMs (W8A16 and W4A16): Y = X . W^T with X in bf16
// (unquantised) and W as 2:4-compressed 8-bit codes (e4m3 or int8) or int4
// codes (two per byte) with groupwise scales.
//
// torchao PR #3258 "Introduce new W8A8-FP-CSR quantization API": jcaip's
// review says weight-only sparsity configs for int8 and float8 have no
// mixed-dtype kernel to run on; CUTLASS PR #2095 "Improvements for: Groupwise
// scaling along M for FP8 gemm" (hwu36's comment) fixes the scale blocks:
//   y[m, n] = sum_kb sw[n / gran_n, kb] * sum_{k in kb} x[m, k] * dec(w[n, k]).
//
// gfx950 has no matrix instruction that mixes 8-bit and bf16 operands, so the
// codes are widened to bf16 in registers (exact for both code types) and
// multiplied on the sparse bf16 matrix core (v_smfmac_f32_16x16x64_bf16),
// which reads the 2:4 metadata itself.  Its operand layout, measured on
// MI355X with one-hot operands: per 64-wide K slice, B lane (group g', column
// c) holds 16 values, virtual k = 16 g' + e; A lane group g holds the
// compressed pairs of the virtual groups of 4 {b, b+1, b+4, b+5},
// b = 8 (g & 1) + 2 (g >> 1), and nibble p of its index word (bits 4p..4p+3)
// places pair p inside its group.  The instruction sums over its K in any
// order, so virtual groups may stand for any aligned groups of the weight as
// long as A and B agree: here A lane group g of instruction h (K slice
// 64 h .. 64 h + 63 of a 128-wide K block) takes the four consecutive groups
// 16 h + 4 g .. + 3, i.e. 8 contiguous code bytes and 16 contiguous metadata
// bits (the index word as stored), and B lane group g' then holds
// x[k = 64 h + 8 g' .. + 7] and x[k = 64 h + 32 + 8 g' .. + 7].
//
// Three kernels share that arithmetic.  At decode sizes a workgroup owns RB
// blocks of 16 W rows and all (M <= 48, k_gemm_w8a16_dma: the weight streamed
// through per-wave LDS rings) or 64 (k_gemm_w8a16: operands loaded straight
// into registers) X rows; its 8 waves split the K blocks and add their
// partial tiles through LDS.  Large M (k_gemm_w8a16_tile) uses 256 x 128
// output tiles staged in LDS; the host picks it where it is the cheaper.
#include "tile_epilogue.h"
#include "sg.h"

namespace sg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));

struct W8Args {
  int64_t M, N, K;
  const uint16_t* x;     // bf16 [M, K]
  int64_t ldx;           // elements
  const uint8_t* w;      // codes [N, K/2]
  int64_t ldw;
  const uint8_t* meta;   // [N, K/8]
  int64_t ldm;
  const float* sw;
  int64_t sw_sn, sw_sk;
  int gn_shift;
  const float* bias;     // [N] or NULL
  void* y;
  int64_t ldy;
  int vec_store;
};

constexpr int W8_WAVES = 8, W8_U = 2;
enum W8Codes { C_E4M3 = 0, C_I8 = 1, C_I4 = 2 };

#if SG_DEVICE_PASS
__device__ __forceinline__ __amdgpu_buffer_rsrc_t w8_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v4i w8_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ int w8_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}

// bf16 bits of the two codes in the low (HI = false) or high half of w,
// first code in the low 16 bits.  Both conversions are exact: e4m3 goes
// through gfx950's scaled fp8 -> bf16 pair conversion with scale 1 (every
// e4m3 value, subnormals included, is a bf16 value).
template <bool I8, bool HI>
__device__ __forceinline__ uint32_t bf16_pair(uint32_t w) {
  if constexpr (I8) {
    const float f0 = (float)(int)(int8_t)(w >> (HI ? 16 : 0));
    const float f1 = (float)(int)(int8_t)(w >> (HI ? 24 : 8));
    // high halves of f0 (low 16 bits) and f1 (high 16 bits)
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
}

__device__ __forceinline__ v2i w8_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}

// bf16 A operand (8 values) of 8 consecutive codes: two dwords of bytes, or
// (int4) the 8 nibbles of w0, element 2j in the low nibble of byte j.
template <int CODES>
__device__ __forceinline__ v4i widen8(int w0, int w1) {
  if constexpr (CODES == C_I4) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // the builtin's result type is unsigned: convert it as the signed value it holds
      const float f0 = (float)(int)__builtin_amdgcn_sbfe(w0, 8 * q, 4);
      const float f1 = (float)(int)__builtin_amdgcn_sbfe(w0, 8 * q + 4, 4);
      d[q] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    }
    return (v4i){(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
  } else {
    constexpr bool I8 = CODES == C_I8;
    return (v4i){(int)bf16_pair<I8, false>((uint32_t)w0), (int)bf16_pair<I8, true>((uint32_t)w0),
                 (int)bf16_pair<I8, false>((uint32_t)w1), (int)bf16_pair<I8, true>((uint32_t)w1)};
  }
}

// Packed gfx950 weight (the FP8 kernels' layout: one 1280-byte chunk per 16
// rows and 128-wide K block, each row's 64 code bytes as 16-byte lane-group
// pieces and its 16 metadata bytes as lane-group index words).  The 8 code
// bytes that lane group g of K slice h multiplies here (row bytes
// 32 h + 8 g .. + 7) are half g >> 1 of the FP8 lane group 2 (g & 1) + h's
// piece, and their 16-bit index word (metadata bytes 8 h + 2 g, + 1) is half
// g >> 1 of that lane group's index word.  Offsets inside a chunk, local row r:
__device__ __forceinline__ int w8pk_code_off(int r, int g, int h) {
  return pk_val_off(r, 2 * (g & 1) + h) + 8 * (g >> 1);
}
__device__ __forceinline__ int w8pk_meta_off(int r, int g, int h) {
  return PK_META + pk_meta_word(r, 2 * (g & 1) + h) + 2 * (g >> 1);
}
// Bytes per (row block, K block) chunk of a packed weight: the gfx950 form of
// 8-bit codes, or the blocked int4 form (codes and metadata as stored).
template <int CODES>
constexpr int pk_chunk() {
  return CODES == C_I4 ? PK4_CHUNK : PK_CHUNK;
}

// The same index word from local row r's 16 packed metadata bytes m.
__device__ __forceinline__ int w8pk_meta_half(const v4i& m, int r, int g, int h) {
  const int q = (pk_meta_word(r, 2 * (g & 1) + h) - 16 * r) >> 2;
  const uint32_t d = (uint32_t)(q == 0 ? m[0] : q == 1 ? m[1] : q == 2 ? m[2] : m[3]);
  return (int)((d >> (16 * (g >> 1))) & 0xffffu);
}

template <int RB, int MT>
struct W8Ops {
  v4i cw[RB];       // code bytes of W row n0 + 16 rb + lr: 8 for K slice 0, 8 for slice 1
  v4i mw[RB];       // the row's 16 metadata bytes of the K block
  v4i bx[MT][4];    // X row m0 + 16 j + lr: k = 8 g + 32 q .. + 7 for q = 0..3
  float sw4[RB][4];
};

// PK: rw covers the workgroup's packed chunks (row block rb's chunk of K
// block kb at (rb KB + kb) pk_chunk<CODES>()); rm is unused.
template <int CODES, int RB, int MT, int GRAN_N, bool PK>
__device__ __forceinline__ void w8_load(const W8Args& a, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rm,
                                        __amdgpu_buffer_rsrc_t rx, int64_t n0, int kb, int lr, int g,
                                        W8Ops<RB, MT>& o) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t r = (uint32_t)(16 * rb + lr);
    if constexpr (PK && CODES == C_I4) {   // blocked: row lr's 32 code bytes at lr * 32
      constexpr int CH = PK4_CHUNK;
      const uint32_t c = (uint32_t)(rb * (int)(a.K >> 7) * CH);
      const int c0 = w8_ld4(rw, c + lr * 32 + 4 * g, kb * CH);
      const int c1 = w8_ld4(rw, c + lr * 32 + 16 + 4 * g, kb * CH);
      o.cw[rb] = (v4i){c0, 0, c1, 0};
      o.mw[rb] = w8_ld16(rw, c + PK4_META + 16 * lr, kb * CH);
    } else if constexpr (PK) {
      const uint32_t c = (uint32_t)(rb * (int)(a.K >> 7) * PK_CHUNK);
      const v2i c0 = w8_ld8(rw, c + w8pk_code_off(lr, g, 0), kb * PK_CHUNK);
      const v2i c1 = w8_ld8(rw, c + w8pk_code_off(lr, g, 1), kb * PK_CHUNK);
      o.cw[rb] = (v4i){c0[0], c0[1], c1[0], c1[1]};
      o.mw[rb] = w8_ld16(rw, c + PK_META + 16 * lr, kb * PK_CHUNK);
    } else if constexpr (CODES == C_I4) {   // 32 bytes per row and K block: 4 per lane and K slice
      const int c0 = w8_ld4(rw, r * (uint32_t)a.ldw + 4 * g, kb * 32);
      const int c1 = w8_ld4(rw, r * (uint32_t)a.ldw + 16 + 4 * g, kb * 32);
      o.cw[rb] = (v4i){c0, 0, c1, 0};
    } else {
      const v2i c0 = w8_ld8(rw, r * (uint32_t)a.ldw + 8 * g, kb * 64);
      const v2i c1 = w8_ld8(rw, r * (uint32_t)a.ldw + 32 + 8 * g, kb * 64);
      o.cw[rb] = (v4i){c0[0], c0[1], c1[0], c1[1]};
    }
    if constexpr (!PK) o.mw[rb] = w8_ld16(rm, r * (uint32_t)a.ldm, kb * 16);
    const int64_t nb = n0 + 16 * rb;   // rows past N read the last row's scale (never stored)
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
    const uint32_t xo = (uint32_t)((16 * j + lr) * a.ldx * 2) + 16 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q) o.bx[j][q] = w8_ld16(rx, xo + 64 * q, kb * 256);
  }
}

// 16-bit index word of metadata halfword hw of a row's 16 bytes.
__device__ __forceinline__ int meta_half(const v4i& m, int hw) {
  const uint32_t d = (uint32_t)((hw >> 1) == 0 ? m[0] : (hw >> 1) == 1 ? m[1] : (hw >> 1) == 2 ? m[2] : m[3]);
  return (int)((d >> (16 * (hw & 1))) & 0xffffu);
}

template <int CODES, int RB, int MT, bool PK>
__device__ __forceinline__ void w8_compute(const W8Ops<RB, MT>& o, int g, int lr, v4f (&acc)[RB][MT]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const v4i a0 = widen8<CODES>(o.cw[rb][0], o.cw[rb][1]);
    const v4i a1 = widen8<CODES>(o.cw[rb][2], o.cw[rb][3]);
    constexpr bool PKM = PK && CODES != C_I4;   // gfx950-packed index words (blocked int4: as stored)
    const int i0 = PKM ? w8pk_meta_half(o.mw[rb], lr, g, 0) : meta_half(o.mw[rb], g);
    const int i1 = PKM ? w8pk_meta_half(o.mw[rb], lr, g, 1) : meta_half(o.mw[rb], g + 4);
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const v8i b0 = {o.bx[j][0][0], o.bx[j][0][1], o.bx[j][0][2], o.bx[j][0][3],
                      o.bx[j][1][0], o.bx[j][1][1], o.bx[j][1][2], o.bx[j][1][3]};
      const v8i b1 = {o.bx[j][2][0], o.bx[j][2][1], o.bx[j][2][2], o.bx[j][2][3],
                      o.bx[j][3][0], o.bx[j][3][1], o.bx[j][3][2], o.bx[j][3][3]};
      v4f p = {0.f, 0.f, 0.f, 0.f};
      p = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v16bf, b0), p,
                                                    i0, 0, 0);
      p = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v16bf, b1), p,
                                                    i1, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[rb][j][e] = fmaf(p[e], o.sw4[rb][e], acc[rb][j][e]);
    }
  }
}
#endif  // SG_DEVICE_PASS

template <int CODES, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
__global__ void __launch_bounds__(512) k_gemm_w8a16(W8Args a) {
#if SG_DEVICE_PASS
  constexpr int U = W8_U;
  __shared__ __attribute__((aligned(16))) float red[W8_WAVES][RB * MT][64][4];
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
  const int64_t wrows = min((int64_t)(16 * RB), a.N - n0), xrows = min((int64_t)(16 * MT), a.M - m0);
  // rows past N or M read as zero (packed: the packer's zero rows)
  const __amdgpu_buffer_rsrc_t rw =
      PK ? w8_rsrc(a.w + (n0 / PK_ROWS) * KB * pk_chunk<CODES>(),
                   (uint32_t)(((wrows + PK_ROWS - 1) / PK_ROWS) * KB * pk_chunk<CODES>()))
         : w8_rsrc(a.w + n0 * a.ldw, (uint32_t)(wrows * a.ldw));
  const __amdgpu_buffer_rsrc_t rm = w8_rsrc(a.meta + n0 * a.ldm, (uint32_t)(wrows * a.ldm));
  const __amdgpu_buffer_rsrc_t rx = w8_rsrc(a.x + m0 * a.ldx, (uint32_t)(xrows * a.ldx * 2));

  v4f acc[RB][MT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[rb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // wave w multiplies K blocks w, w + 8, ...; U of them loaded before they are multiplied
  const int nt = (KB - wave + W8_WAVES - 1) / W8_WAVES;
  W8Ops<RB, MT> ops[U];
  for (int t0 = 0; t0 < nt; t0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      w8_load<CODES, RB, MT, GRAN_N, PK>(a, rw, rm, rx, n0, wave + W8_WAVES * min(t0 + u, nt - 1), lr, g, ops[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u < nt) w8_compute<CODES, RB, MT, PK>(ops[u], g, lr, acc);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j)
      *reinterpret_cast<float4*>(&red[wave][rb * MT + j][l][0]) =
          make_float4(acc[rb][j][0], acc[rb][j][1], acc[rb][j][2], acc[rb][j][3]);
  __syncthreads();
  for (int q = t; q < RB * MT * 64; q += 512) {
    const int s = q >> 6, ll = q & 63, rb = s / MT, j = s % MT;
    float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < W8_WAVES; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&red[w][s][ll][0]);
      v4.x += v.x; v4.y += v.y; v4.z += v.z; v4.w += v.w;
    }
    const int64_t n = n0 + 16 * rb + 4 * (ll >> 4);
    v4f out = {v4.x, v4.y, v4.z, v4.w};
    if (a.bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] += a.bias[min(n + e, a.N - 1)];
    }
    store_quad<OUT_BF16, OUT_T>(a, m0 + (int64_t)j * 16 + (ll & 15), n, out);
  }
#endif  // SG_DEVICE_PASS
}

// ------------------------------------------------------- M <= 48: LDS streaming
// The same arithmetic with the weight streamed into a private LDS ring of each
// wave by buffer loads that write LDS directly (no registers in flight, no
// barriers in the loop): per K block the RB row blocks' codes and metadata and
// the W scales.  X (bf16) takes 4 KB per 16 rows and K block: for one 16-row
// sub-tile it rides in the ring too (16-byte chunks XOR-swizzled by row); for
// two or three it would overflow LDS, so each wave loads its X fragments into
// registers with the same K block's loads (from L2: every workgroup reads all
// of X).  Two slots per wave; each wave waits only for its own loads, counted
// exactly (loads return in order, whether to LDS or to registers).
template <int CODES, int RB, int MT>
struct W8Dma {
  static constexpr int CB = CODES == C_I4 ? 512 : 1024;   // code bytes of 16 rows per K block
  static constexpr int MOFF = RB * CB;                       // metadata, 256 B per row block
  static constexpr int XOFF = MOFF + RB * 256;               // X (one sub-tile): 16 rows x 256 B
  static constexpr int SWOFF = XOFF + (MT == 1 ? 4096 : 0);  // W scales, 256 B
  static constexpr int KSZ = SWOFF + 256;                    // bytes per wave per K block
  static constexpr int ARR = W8_WAVES * KSZ;                 // one slot of every wave
  static constexpr int L = RB * (CODES == C_I4 ? 2 : 1) + RB + 4 * MT + 1;   // loads per K block
  static constexpr bool FITS = 2 * ARR <= 160 * 1024;
};

typedef __attribute__((address_space(3))) void w8_lds_t;

#if SG_DEVICE_PASS
__device__ __forceinline__ int xswz(int r) { return r & 7; }

template <typename T>
__device__ __forceinline__ T w8_lds(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

// X fragments of lane (g, lr) for MT sub-tiles: row 16 j + lr, 16-byte chunks
// g, g + 4, g + 8, g + 12 of the K block's 256 bytes
template <int MT>
struct W8X {
  v4i c[MT][4];
};

template <int CODES, int RB, int MT, int GRAN_N, bool PK>
__device__ __forceinline__ void w8_dma_issue(uint8_t* sl, const W8Args& a, __amdgpu_buffer_rsrc_t rw,
                                             __amdgpu_buffer_rsrc_t rm, __amdgpu_buffer_rsrc_t rx,
                                             __amdgpu_buffer_rsrc_t rsw, int64_t n0, int kb, int l, bool valid,
                                             W8X<MT>& xr) {
  using D = W8Dma<CODES, RB, MT>;
  constexpr int KBB = CODES == C_I4 ? 32 : 64;      // code bytes per row per K block
  // a K block past the wave's last reads through descriptors of zero records,
  // out of range for every offset: no memory access, zeros
  const int ws = valid ? kb * KBB : 0, ms = valid ? kb * 16 : 0, xs = valid ? kb * 256 : 0;
  if (!valid) {
    rw = w8_rsrc(a.w, 0);
    rm = w8_rsrc(a.meta, 0);
    rx = w8_rsrc(a.x, 0);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (PK) {   // the chunk as stored: codes, then metadata (int4: the canonical LDS image)
      constexpr int CH = pk_chunk<CODES>(), META = CODES == C_I4 ? PK4_META : PK_META;
      const uint32_t c = (uint32_t)(rb * (int)(a.K >> 7) * CH);
      const int cs = valid ? kb * CH : 0;
      if constexpr (CODES == C_I4) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(sl + rb * D::CB + e * 256), 4, c + 256 * e + 4 * l,
                                                   cs, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(sl + rb * D::CB), 16, c + 16 * l, cs, 0, 0);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(sl + D::MOFF + rb * 256), 4, c + META + 4 * l, cs, 0,
                                               0);
      continue;
    }
    if constexpr (CODES == C_I4) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (w8_lds_t*)(sl + rb * D::CB + e * 256), 4,
            (uint32_t)((16 * rb + 8 * e + (l >> 3)) * a.ldw + 4 * (l & 7)), ws, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(sl + rb * D::CB), 16,
                                               (uint32_t)((16 * rb + (l >> 2)) * a.ldw + 16 * (l & 3)), ws, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (w8_lds_t*)(sl + D::MOFF + rb * 256), 4,
                                             (uint32_t)((16 * rb + (l >> 2)) * a.ldm + 4 * (l & 3)), ms, 0, 0);
  }
  if constexpr (MT == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 64 * i + l, r = p >> 4, c = (p & 15) ^ xswz(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (w8_lds_t*)(sl + D::XOFF + i * 1024), 16,
                                               (uint32_t)(r * a.ldx * 2 + c * 16), xs, 0, 0);
    }
  } else {
    const int g = l >> 4, lr = l & 15;
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        xr.c[j][c] = w8_ld16(rx, (uint32_t)((16 * j + lr) * a.ldx * 2 + (g + 4 * c) * 16), xs);
  }
  // W scales of this K block: lane rb < RB (128-row blocks) or lane = row (per row)
  const int64_t n = GRAN_N == 128 ? (min(n0 + 16 * (l % RB), a.N - 1) >> 7) : min(n0 + l, a.N - 1);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (w8_lds_t*)(sl + D::SWOFF), 4, (uint32_t)(n * a.sw_sn * 4),
                                           (int)(kb * a.sw_sk * 4), 0, 0);
}
#endif  // SG_DEVICE_PASS

// EVEN: the G workgroups share the R row blocks of 16 evenly, q = R / G and
// r = R % G: workgroup b owns the q + (b < r) row blocks from b q + min(b, r)
// on (at most RB); otherwise workgroup b owns row blocks RB b .. RB b + RB - 1
// (q and r unused).  q and r come from the host, so that no division here
// turns the buffer descriptors into vector values.
// PK: the weight in its packed form (gfx950 chunks of 8-bit codes, blocked
// int4 chunks), each chunk copied into the ring as stored (codes at rb * CB,
// metadata at MOFF + rb * 256).
template <int CODES, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool EVEN, bool PK>
__global__ void __launch_bounds__(512) k_gemm_w8a16_dma(W8Args a, int q, int r) {
#if SG_DEVICE_PASS
  using D = W8Dma<CODES, RB, MT>;
  static_assert(D::FITS && 4 * RB * 64 * 16 <= D::ARR, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t r0[D::ARR];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[D::ARR];
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
  if constexpr (EVEN) {
    const int b = (int)blockIdx.x;
    const int rb0 = b * q + min(b, r), rb1 = rb0 + q + (b < r ? 1 : 0);
    n0 = 16 * (int64_t)rb0;
    a.N = min(a.N, 16 * (int64_t)rb1);   // the rows past this workgroup's are another's: not loaded, not stored
  }
  if (blockIdx.y > 0) {   // grid row y: X rows and output columns from 16 MT y on
    const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
    a.x += m0 * a.ldx;
    a.M -= m0;
    a.y = static_cast<uint8_t*>(a.y) + (OUT_T ? m0 : m0 * a.ldy) * (OUT_BF16 ? 2 : 4);
  }
  const int64_t wrows = min((int64_t)(16 * RB), a.N - n0);
  const __amdgpu_buffer_rsrc_t rw =
      PK ? w8_rsrc(a.w + (n0 / PK_ROWS) * KB * pk_chunk<CODES>(),
                   (uint32_t)(((wrows + PK_ROWS - 1) / PK_ROWS) * KB * pk_chunk<CODES>()))
         : w8_rsrc(a.w + n0 * a.ldw, (uint32_t)(wrows * a.ldw));
  const __amdgpu_buffer_rsrc_t rm = w8_rsrc(a.meta + n0 * a.ldm, (uint32_t)(wrows * a.ldm));
  const __amdgpu_buffer_rsrc_t rx = w8_rsrc(a.x, (uint32_t)(a.M * a.ldx * 2));   // rows past M read zero
  const __amdgpu_buffer_rsrc_t rsw = w8_rsrc(a.sw, 0xffffffffu);
  const int nt = (KB - wave + W8_WAVES - 1) / W8_WAVES;
  const uint32_t wslot = (uint32_t)wave * D::KSZ;

  v4f acc[RB][MT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[rb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  auto issue = [&](uint8_t* arr, W8X<MT>& xr, int tt) {
    w8_dma_issue<CODES, RB, MT, GRAN_N, PK>(arr + wslot, a, rw, rm, rx, rsw, n0, wave + W8_WAVES * min(tt, nt - 1), l,
                                        tt < nt, xr);
  };
  auto compute = [&](const uint8_t* arr, const W8X<MT>& xr) {
    const uint8_t* sl = arr + wslot;
    v8i b[MT][2];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      if constexpr (MT == 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 lo = w8_lds<uint4>(sl, D::XOFF + lr * 256 + (((g + 8 * h) ^ xswz(lr)) << 4));
          const uint4 hi = w8_lds<uint4>(sl, D::XOFF + lr * 256 + (((g + 8 * h + 4) ^ xswz(lr)) << 4));
          b[j][h] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v4i lo = xr.c[j][2 * h], hi = xr.c[j][2 * h + 1];
          b[j][h] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i cw;
      int i0, i1;
      if constexpr (PK && CODES != C_I4) {   // codes at rb * CB, metadata at MOFF + rb * 256
        const uint2 c0 = w8_lds<uint2>(sl, rb * D::CB + w8pk_code_off(lr, g, 0));
        const uint2 c1 = w8_lds<uint2>(sl, rb * D::CB + w8pk_code_off(lr, g, 1));
        cw = (v4i){(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
        i0 = w8_lds<uint16_t>(sl, D::MOFF + rb * 256 + w8pk_meta_off(lr, g, 0) - PK_META);
        i1 = w8_lds<uint16_t>(sl, D::MOFF + rb * 256 + w8pk_meta_off(lr, g, 1) - PK_META);
      } else {
        if constexpr (CODES == C_I4) {
          cw = (v4i){w8_lds<int>(sl, rb * D::CB + lr * 32 + 4 * g), 0,
                     w8_lds<int>(sl, rb * D::CB + lr * 32 + 16 + 4 * g), 0};
        } else {
          const uint2 c0 = w8_lds<uint2>(sl, rb * D::CB + lr * 64 + 8 * g);
          const uint2 c1 = w8_lds<uint2>(sl, rb * D::CB + lr * 64 + 32 + 8 * g);
          cw = (v4i){(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
        }
        // index words: halfwords g and g + 4 of the row's 16 metadata bytes
        i0 = w8_lds<uint16_t>(sl, D::MOFF + rb * 256 + lr * 16 + 2 * g);
        i1 = w8_lds<uint16_t>(sl, D::MOFF + rb * 256 + lr * 16 + 8 + 2 * g);
      }
      const v4i a0 = widen8<CODES>(cw[0], cw[1]);
      const v4i a1 = widen8<CODES>(cw[2], cw[3]);
      float4 sw;
      if (GRAN_N == 128) {
        const float v = w8_lds<float>(sl, D::SWOFF + rb * 4);
        sw = make_float4(v, v, v, v);
      } else {
        sw = w8_lds<float4>(sl, D::SWOFF + (16 * rb + 4 * g) * 4);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        v4f p = {0.f, 0.f, 0.f, 0.f};
        p = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v16bf, b[j][0]),
                                                      p, i0, 0, 0);
        p = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v16bf, b[j][1]),
                                                      p, i1, 0, 0);
        acc[rb][j][0] = fmaf(p[0], sw.x, acc[rb][j][0]);
        acc[rb][j][1] = fmaf(p[1], sw.y, acc[rb][j][1]);
        acc[rb][j][2] = fmaf(p[2], sw.z, acc[rb][j][2]);
        acc[rb][j][3] = fmaf(p[3], sw.w, acc[rb][j][3]);
      }
    }
  };

  // K block t of this wave lives in r0 / xa for even t, r1 / xb for odd t;
  // block t + 1 is loaded while block t is multiplied
  W8X<MT> xa, xb;
  if (nt > 0) issue(r0, xa, 0);
  for (int t0 = 0; t0 < nt; t0 += 2) {
    issue(r1, xb, t0 + 1);
    wait_vmcnt<D::L>();
    compute(r0, xa);
    if (t0 + 1 < nt) {
      issue(r0, xa, t0 + 2);
      wait_vmcnt<D::L>();
      compute(r1, xb);
    }
  }
  wait_vmcnt<0>();
  // waves 0-3 hand their partial tiles over in r0, waves 4-7 in r1, one
  // sub-tile column j at a time: [4][RB][64] float4 each
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
      for (int w = 0; w < W8_WAVES; ++w) {
        const float4 v = reinterpret_cast<const float4*>(w < 4 ? r0 : r1)[((w & 3) * RB + rb) * 64 + ll];
        v4.x += v.x; v4.y += v.y; v4.z += v.z; v4.w += v.w;
      }
      const int64_t n = n0 + 16 * rb + 4 * (ll >> 4);
      v4f out = {v4.x, v4.y, v4.z, v4.w};
      if (a.bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] += a.bias[min(n + e, a.N - 1)];
      }
      store_quad<OUT_BF16, OUT_T>(a, (int64_t)(16 * j + (ll & 15)), n, out);
    }
  }
#endif  // SG_DEVICE_PASS
}

// Launches the LDS-streaming kernel with RB row blocks per workgroup if its
// ring fits LDS and the grid keeps at least 224 workgroups (RB = 1 always
// qualifies).
template <int CODES, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
static bool try_w8_dma(const W8Args& a, hipStream_t st, int64_t rows16, unsigned gy = 1) {
  if constexpr (W8Dma<CODES, RB, MT>::FITS) {
    if (RB == 1 || rows16 >= RB * 224) {
      k_gemm_w8a16_dma<CODES, RB, MT, GRAN_N, OUT_BF16, OUT_T, false, PK>
          <<<dim3((unsigned)cdiv(rows16, RB), gy), 512, 0, st>>>(a, 0, 0);
      return true;
    }
  }
  return false;
}

// More 16-row blocks than CUs but too few for 224 workgroups of four: one
// workgroup per CU with an even share of ceil(R / CUs) or one fewer row
// blocks (as the FP8 decode kernel).
template <int CODES, int RB, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
static bool try_w8_even_rb(const W8Args& a, hipStream_t st, int64_t rows16, int cus, unsigned gy) {
  if constexpr (W8Dma<CODES, RB, MT>::FITS) {
    k_gemm_w8a16_dma<CODES, RB, MT, GRAN_N, OUT_BF16, OUT_T, true, PK>
        <<<dim3((unsigned)cus, gy), 512, 0, st>>>(a, (int)(rows16 / cus), (int)(rows16 % cus));
    return true;
  }
  return false;
}

template <int CODES, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
static bool try_w8_even(const W8Args& a, hipStream_t st, int64_t rows16, unsigned gy = 1) {
  const int cus = cu_count();
  if (rows16 <= cus || rows16 >= 4 * 224 || rows16 > 4LL * cus) return false;
  switch (cdiv(rows16, cus)) {
    case 2: return try_w8_even_rb<CODES, 2, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, cus, gy);
    case 3: return try_w8_even_rb<CODES, 3, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, cus, gy);
    default: return try_w8_even_rb<CODES, 4, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, cus, gy);
  }
}

// --------------------------------------------------------------- large M
// Workgroup tile 256 W rows (n) x 128 X rows (m), 8 waves in a 4 (n) x 2 (m)
// grid, each wave 64 x 64 = 4 x 4 sub-tiles, so every X fragment a wave reads
// serves four W row blocks and every widened W fragment four X sub-tiles.
// One 128-wide K block per LDS stage, two stages: all waves multiply stage kb
// while stage kb + 1 streams in through buffer loads that write LDS; one
// barrier per K block.  Stage layout (bytes; swizzles keep the fragment reads
// free of bank conflicts):
//   X    : 128 rows x 256 B (bf16); 16-byte chunk c of row r at chunk c ^ (r & 15)
//   W    : 256 rows x 64 B of codes (int4: 32 B); 16-byte unit u of row r at
//          u ^ ((r >> 2) & 3) (int4: u ^ ((r >> 3) & 1))
//   meta : 256 rows x 16 B
//   sw   : 256 floats, the scale of each W row for the K block (its 128-row
//          block's with 128-row scales); rows past N read row N - 1's
namespace w8t {
constexpr int BN = 256, BM = 128;
template <int CODES>
struct Lay {
  static constexpr int WROW = CODES == C_I4 ? 32 : 64;
  static constexpr int X_OFF = 0;
  static constexpr int W_OFF = BM * 256;
  static constexpr int M_OFF = W_OFF + BN * WROW;
  static constexpr int S_OFF = M_OFF + BN * 16;
  static constexpr int BYTES = S_OFF + BN * 4;
};
}  // namespace w8t

#if SG_DEVICE_PASS
// PK: W and metadata as the tile's 16 packed chunks, each copied as stored
// (codes of row block b at W_OFF + 1024 b, metadata at M_OFF + 256 b).
template <int CODES, int GRAN_N, bool PK>
__device__ __forceinline__ void w8t_issue(uint8_t* st, const W8Args& a, __amdgpu_buffer_rsrc_t rx,
                                          __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rm,
                                          __amdgpu_buffer_rsrc_t rsw, int64_t n0, int kb, int wave, int l) {
  using L = w8t::Lay<CODES>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // X: 2048 units of 16 B, unit p at LDS 16 p
    const int s = 8 * i + wave, p = 64 * s + l, r = p >> 4, c = (p & 15) ^ (r & 15);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (w8_lds_t*)(st + L::X_OFF + s * 1024), 16,
                                             (uint32_t)(r * a.ldx * 2 + c * 16), kb * 256, 0, 0);
  }
  if constexpr (PK && CODES == C_I4) {   // blocked: the canonical LDS image from row r's place in its chunk
    const int KB = (int)(a.K >> 7);
    const int p = 64 * wave + l, r = p >> 1, u = (p & 1) ^ ((r >> 3) & 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(st + L::W_OFF + wave * 1024), 16,
                                             (uint32_t)((r >> 4) * KB * PK4_CHUNK + (r & 15) * 32 + u * 16),
                                             kb * PK4_CHUNK, 0, 0);
    if (wave < 4) {
      const int rm4 = 64 * wave + l;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(st + L::M_OFF + wave * 1024), 16,
                                               (uint32_t)((rm4 >> 4) * KB * PK4_CHUNK + PK4_META + (rm4 & 15) * 16),
                                               kb * PK4_CHUNK, 0, 0);
    }
  } else if constexpr (PK) {   // 1024 code units (row block p >> 6), then 256 metadata units (row block p >> 4)
    const int KB = (int)(a.K >> 7);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = 8 * i + wave, p = 64 * s + l;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(st + L::W_OFF + s * 1024), 16,
                                               (uint32_t)((p >> 6) * KB * PK_CHUNK + 16 * (p & 63)), kb * PK_CHUNK,
                                               0, 0);
    }
    if (wave < 4) {
      const int p = 64 * wave + l;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(st + L::M_OFF + wave * 1024), 16,
                                               (uint32_t)((p >> 4) * KB * PK_CHUNK + PK_META + 16 * (p & 15)),
                                               kb * PK_CHUNK, 0, 0);
    }
  } else if constexpr (CODES == C_I4) {   // 512 units: row p >> 1, stored unit p & 1
    const int p = 64 * wave + l, r = p >> 1, u = (p & 1) ^ ((r >> 3) & 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(st + L::W_OFF + wave * 1024), 16,
                                             (uint32_t)(r * a.ldw + u * 16), kb * 32, 0, 0);
  } else {                         // 1024 units: row p >> 2, stored unit p & 3
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = 8 * i + wave, p = 64 * s + l, r = p >> 2, u = (p & 3) ^ ((r >> 2) & 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w8_lds_t*)(st + L::W_OFF + s * 1024), 16,
                                               (uint32_t)(r * a.ldw + u * 16), kb * 64, 0, 0);
    }
  }
  if (wave < 4) {   // metadata: row 64 wave + l
    if constexpr (!PK)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (w8_lds_t*)(st + L::M_OFF + wave * 1024), 16,
                                               (uint32_t)((64 * wave + l) * a.ldm), kb * 16, 0, 0);
  } else {          // W scales: row 64 (wave - 4) + l
    const int64_t n = min(n0 + 64 * (wave - 4) + l, a.N - 1);
    const int64_t row = GRAN_N == 128 ? (n >> 7) : n;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (w8_lds_t*)(st + L::S_OFF + (wave - 4) * 256), 4,
                                             (uint32_t)(row * a.sw_sn * 4), (int)(kb * a.sw_sk * 4), 0, 0);
  }
}

// Multiplies one stage into the wave's 4 x 4 sub-tiles and promotes each
// K block's partial with its W scale.
template <int CODES, int GRAN_N, bool PK>
__device__ __forceinline__ void w8t_compute(const uint8_t* st, int wn, int wm, int g, int lr, v4f (&acc)[4][4]) {
  using L = w8t::Lay<CODES>;
  v8i b0[4], b1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // X row wm * 64 + 16 j + lr: chunks g, g + 4 | g + 8, g + 12
    const uint32_t row = L::X_OFF + (uint32_t)(wm * 64 + 16 * j + lr) * 256;
    const uint4 c0 = w8_lds<uint4>(st, row + (((g) ^ lr) << 4));
    const uint4 c1 = w8_lds<uint4>(st, row + (((g + 4) ^ lr) << 4));
    const uint4 c2 = w8_lds<uint4>(st, row + (((g + 8) ^ lr) << 4));
    const uint4 c3 = w8_lds<uint4>(st, row + (((g + 12) ^ lr) << 4));
    b0[j] = (v8i){(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
    b1[j] = (v8i){(int)c2.x, (int)c2.y, (int)c2.z, (int)c2.w, (int)c3.x, (int)c3.y, (int)c3.z, (int)c3.w};
  }
  const float swv = GRAN_N == 128 ? w8_lds<float>(st, L::S_OFF + wn * 256) : 1.f;   // the wave's 64 rows share it
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wn * 64 + 16 * i + lr;   // W row in the tile
    v4i cw;
    int i0, i1;
    if constexpr (PK && CODES != C_I4) {   // row block wn * 4 + i of the tile, local row lr
      const uint32_t cb = L::W_OFF + (uint32_t)(wn * 4 + i) * 1024, mb = L::M_OFF + (uint32_t)(wn * 4 + i) * 256;
      const uint2 c0 = w8_lds<uint2>(st, cb + w8pk_code_off(lr, g, 0));
      const uint2 c1 = w8_lds<uint2>(st, cb + w8pk_code_off(lr, g, 1));
      cw = (v4i){(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
      i0 = w8_lds<uint16_t>(st, mb + w8pk_meta_off(lr, g, 0) - PK_META);
      i1 = w8_lds<uint16_t>(st, mb + w8pk_meta_off(lr, g, 1) - PK_META);
    } else if constexpr (CODES == C_I4) {
      const int f = (lr >> 3) & 1;
      cw = (v4i){w8_lds<int>(st, L::W_OFF + r * 32 + (f << 4) + 4 * g), 0,
                 w8_lds<int>(st, L::W_OFF + r * 32 + ((1 ^ f) << 4) + 4 * g), 0};
    } else {
      const int f = (lr >> 2) & 3;
      const uint2 c0 = w8_lds<uint2>(st, L::W_OFF + r * 64 + (((g >> 1) ^ f) << 4) + 8 * (g & 1));
      const uint2 c1 = w8_lds<uint2>(st, L::W_OFF + r * 64 + (((2 + (g >> 1)) ^ f) << 4) + 8 * (g & 1));
      cw = (v4i){(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
    }
    if constexpr (!PK || CODES == C_I4) {   // index words: halfwords g and g + 4 of the row's 16 metadata bytes
      i0 = w8_lds<uint16_t>(st, L::M_OFF + r * 16 + 2 * g);
      i1 = w8_lds<uint16_t>(st, L::M_OFF + r * 16 + 8 + 2 * g);
    }
    const v4i a0 = widen8<CODES>(cw[0], cw[1]);
    const v4i a1 = widen8<CODES>(cw[2], cw[3]);
    float4 sw;
    if (GRAN_N == 128) sw = make_float4(swv, swv, swv, swv);
    else sw = w8_lds<float4>(st, L::S_OFF + (wn * 64 + 16 * i + 4 * g) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4f p = {0.f, 0.f, 0.f, 0.f};
      p = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v16bf, b0[j]),
                                                    p, i0, 0, 0);
      p = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v16bf, b1[j]),
                                                    p, i1, 0, 0);
      acc[i][j][0] = fmaf(p[0], sw.x, acc[i][j][0]);
      acc[i][j][1] = fmaf(p[1], sw.y, acc[i][j][1]);
      acc[i][j][2] = fmaf(p[2], sw.z, acc[i][j][2]);
      acc[i][j][3] = fmaf(p[3], sw.w, acc[i][j][3]);
    }
  }
}
#endif  // SG_DEVICE_PASS

template <int CODES, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
__global__ void __launch_bounds__(512) k_gemm_w8a16_tile(W8Args a, int tiles_m, int tiles_n) {
#if SG_DEVICE_PASS
  using L = w8t::Lay<CODES>;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[L::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[L::BYTES];
  int tn, tm;
  tile_coords(tiles_m, tiles_n, tn, tm);
  const int64_t n0 = (int64_t)tn * w8t::BN, m0 = (int64_t)tm * w8t::BM;
  const int t = threadIdx.x, l = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 3, wm = wave >> 2;
  const int g = l >> 4, lr = l & 15;
  const int KB = (int)(a.K >> 7);
  // rows past M or N read as zero (resources sized to the rows that exist)
  const int64_t mrows = min((int64_t)w8t::BM, a.M - m0), nrows = min((int64_t)w8t::BN, a.N - n0);
  const __amdgpu_buffer_rsrc_t rx = w8_rsrc(a.x + m0 * a.ldx, (uint32_t)(mrows * a.ldx * 2));
  const __amdgpu_buffer_rsrc_t rw =
      PK ? w8_rsrc(a.w + (n0 / PK_ROWS) * KB * pk_chunk<CODES>(),
                   (uint32_t)(((nrows + PK_ROWS - 1) / PK_ROWS) * KB * pk_chunk<CODES>()))
         : w8_rsrc(a.w + n0 * a.ldw, (uint32_t)(nrows * a.ldw));
  const __amdgpu_buffer_rsrc_t rm = w8_rsrc(a.meta + n0 * a.ldm, (uint32_t)(nrows * a.ldm));
  const __amdgpu_buffer_rsrc_t rsw = w8_rsrc(a.sw, 0xffffffffu);

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // K block kb lives in s0 for even kb, s1 for odd kb; a wave's only loads in
  // flight at each wait are the next stage's, and the barrier after it also
  // tells every wave that the stage it is about to overwrite has been read
  w8t_issue<CODES, GRAN_N, PK>(s0, a, rx, rw, rm, rsw, n0, 0, wave, l);
  wait_vmcnt<0>();
  __syncthreads();
  for (int kb = 0; kb < KB; kb += 2) {
    if (kb + 1 < KB) w8t_issue<CODES, GRAN_N, PK>(s1, a, rx, rw, rm, rsw, n0, kb + 1, wave, l);
    w8t_compute<CODES, GRAN_N, PK>(s0, wn, wm, g, lr, acc);
    wait_vmcnt<0>();
    __syncthreads();
    if (kb + 1 < KB) {
      if (kb + 2 < KB) w8t_issue<CODES, GRAN_N, PK>(s0, a, rx, rw, rm, rsw, n0, kb + 2, wave, l);
      w8t_compute<CODES, GRAN_N, PK>(s1, wn, wm, g, lr, acc);
      wait_vmcnt<0>();
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + 16 * i + 4 * g;
      v4f out = acc[i][j];
      if (a.bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] += a.bias[min(n + e, a.N - 1)];
      }
      store_quad<OUT_BF16, OUT_T>(a, m0 + wm * 64 + 16 * j + lr, n, out);
    }
#endif  // SG_DEVICE_PASS
}

// The large-M tile kernel when it is the faster of the two and its 32-bit
// per-tile buffer offsets hold.  Measured on MI355X at K = 4096 (e4m3 codes):
// the tile kernel takes about 48 us per round of tiles over the CUs whatever
// M is, the decode-shaped kernel about 10.8 us per 64 rows of M and 4096 of N
// (N = 4096: 24 us at M = 128, 44 us at 256, 66 us at 384; the tile kernel
// 44-51 us for all three), so the tile kernel wins once
// ceil(M / 64) * N / 4096 exceeds 4.5 rounds.
template <int CODES, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
static bool try_w8_tile(const W8Args& a, hipStream_t st) {
  const int64_t tm = cdiv(a.M, w8t::BM), tn = cdiv(a.N, w8t::BN);
  if (tm * tn > 0x7fffffffLL || a.ldx >= (1LL << 22) || a.ldw >= (1LL << 23) || a.ldm >= (1LL << 23))
    return false;
  const int64_t rounds = cdiv(tm * tn, cu_count());
  if (2 * cdiv(a.M, 64) * a.N < 9 * 4096 * rounds) return false;
  k_gemm_w8a16_tile<CODES, GRAN_N, OUT_BF16, OUT_T, PK><<<(unsigned)(tm * tn), 512, 0, st>>>(a, (int)tm, (int)tn);
  return true;
}

// Row blocks per workgroup: with more 16-row blocks than CUs but under 896, an
// even share over one workgroup per CU; otherwise the largest of 4 (2 for
// MT > 2), 2, 1 that keeps at least 224 workgroups.  Every workgroup reads
// its X rows in full, so fewer, taller workgroups read X fewer times
// (measured at M = 37 and 64: 1.7x faster than one row block per workgroup).
// M <= 48 streams the weight through LDS; M = 49..64 does so in two grid
// rows when N is wide.
template <int CODES, int MT, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
static void launch_w8_mt(const W8Args& a, hipStream_t st) {
  const int64_t rows16 = cdiv(a.N, 16);
  const unsigned gy = (unsigned)cdiv(a.M, 16 * MT);
  if constexpr (MT >= 2 && MT <= 3) {
    // at most half as many row blocks as CUs: two grid rows of ceil(MT / 2)
    // sub-tiles, so that the other half of the CUs has work
    constexpr int MH = (MT + 1) / 2;
    if (2 * rows16 <= cu_count() &&
        try_w8_dma<CODES, 1, MH, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, (unsigned)cdiv(a.M, 16 * MH)))
      return;
  }
  if constexpr (MT <= 3) {   // LDS streaming, one workgroup per RB row blocks and all of M
    if (try_w8_even<CODES, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16) ||
        try_w8_dma<CODES, 4, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16) ||
        try_w8_dma<CODES, 2, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16) ||
        try_w8_dma<CODES, 1, MT, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16))
      return;
  } else if (a.M <= 64 && (rows16 > cu_count() || 2 * rows16 <= cu_count())) {
    // M = 49..64 over more row blocks than CUs, or at most half as many: two
    // grid rows of the LDS-streaming kernel, 32 X rows each (N = 14336,
    // K = 4096: 25.6 against 38.4 us packed on the register kernel; at
    // N = 4096 that kernel is the faster one)
    if (try_w8_even<CODES, 2, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, 2) ||
        try_w8_dma<CODES, 4, 2, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, 2) ||
        try_w8_dma<CODES, 2, 2, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, 2) ||
        try_w8_dma<CODES, 1, 2, GRAN_N, OUT_BF16, OUT_T, PK>(a, st, rows16, 2))
      return;
  }
  constexpr int RB4 = MT <= 2 ? 4 : 2, RB2 = 2;
  if (RB4 == 4 && rows16 * gy >= 4 * 224)
    k_gemm_w8a16<CODES, RB4, MT, GRAN_N, OUT_BF16, OUT_T, PK><<<dim3((unsigned)cdiv(rows16, RB4), gy), 512, 0, st>>>(a);
  else if (RB2 == 2 && rows16 * gy >= 2 * 224)
    k_gemm_w8a16<CODES, RB2, MT, GRAN_N, OUT_BF16, OUT_T, PK><<<dim3((unsigned)cdiv(rows16, RB2), gy), 512, 0, st>>>(a);
  else
    k_gemm_w8a16<CODES, 1, MT, GRAN_N, OUT_BF16, OUT_T, PK><<<dim3((unsigned)rows16, gy), 512, 0, st>>>(a);
}

template <int CODES, int GRAN_N, bool OUT_BF16, bool OUT_T, bool PK>
static void launch_w8_shape(const W8Args& a, hipStream_t st) {
  if (a.M > 64 && try_w8_tile<CODES, GRAN_N, OUT_BF16, OUT_T, PK>(a, st)) return;
  if (a.M <= 16) launch_w8_mt<CODES, 1, GRAN_N, OUT_BF16, OUT_T, PK>(a, st);
  else if (a.M <= 32) launch_w8_mt<CODES, 2, GRAN_N, OUT_BF16, OUT_T, PK>(a, st);
  else if (a.M <= 48) launch_w8_mt<CODES, 3, GRAN_N, OUT_BF16, OUT_T, PK>(a, st);
  else launch_w8_mt<CODES, 4, GRAN_N, OUT_BF16, OUT_T, PK>(a, st);
}

template <int CODES, int GRAN_N, bool PK = false>
static void launch_w8_form(const W8Args& a, bool bf16, bool yt, hipStream_t st) {
  if (bf16) {
    if (yt) launch_w8_shape<CODES, GRAN_N, true, true, PK>(a, st);
    else launch_w8_shape<CODES, GRAN_N, true, false, PK>(a, st);
  } else {
    if (yt) launch_w8_shape<CODES, GRAN_N, false, true, PK>(a, st);
    else launch_w8_shape<CODES, GRAN_N, false, false, PK>(a, st);
  }
}

}  // namespace sg

using namespace sg;

extern "C" sg_status sg_w8a16_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                                                      int64_t ldx, const uint8_t* wv, int64_t ldwv,
                                                      const uint8_t* wmeta, int64_t ldwm, sg_dtype w_dt,
                                                      const float* sw, int64_t sw_sn, int64_t sw_sk, int gran_n,
                                                      const float* bias, void* y, sg_dtype y_dt, int64_t ldy,
                                                      sg_form form, hipStream_t stream) {
  if (!x || !wv || !wmeta || !sw || !y) return SG_ERR_NULL;
  if (w_dt != SG_E4M3 && w_dt != SG_I8) return SG_ERR_UNSUPPORTED;
  if (gran_n != 1 && gran_n != 128) return SG_ERR_UNSUPPORTED;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldx < K || ldwv < K / 2 || ldwm < K / 8) return SG_ERR_SHAPE;
  if (ldy < (form == SG_OUT_Y ? N : M)) return SG_ERR_SHAPE;
  // 32-bit buffer offsets: 64 rows of each operand per workgroup
  if (ldx >= (1LL << 24) || ldwv >= (1LL << 24) || ldwm >= (1LL << 24) || sw_sn < 0 || sw_sk < 0) return SG_ERR_SHAPE;
  if (((cdiv(N, gran_n) - 1) * sw_sn + (K / 128 - 1) * sw_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (cdiv(N, 16) > 0x7fffffffLL || cdiv(M, 16) > 65535) return SG_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * 2) % 16 || !aligned(wv, 16) || ldwv % 16 || !aligned(wmeta, 16) || ldwm % 16 ||
      !aligned(sw, 4) || !aligned(bias, 4) || !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  W8Args a;
  a.M = M; a.N = N; a.K = K;
  a.x = x; a.ldx = ldx;
  a.w = wv; a.ldw = ldwv; a.meta = wmeta; a.ldm = ldwm;
  a.sw = sw; a.sw_sn = sw_sn; a.sw_sk = sw_sk; a.gn_shift = gran_n == 128 ? 7 : 0;
  a.bias = bias;
  a.y = y; a.ldy = ldy;
  a.vec_store = (ldy % 4 == 0) && aligned(y, 4 * dtype_size(y_dt));
  clear_hip_error();
  const bool bf16 = y_dt == SG_BF16, yt = form == SG_OUT_YT;
  if (w_dt == SG_I8) {
    if (gran_n == 128) launch_w8_form<C_I8, 128>(a, bf16, yt, stream);
    else launch_w8_form<C_I8, 1>(a, bf16, yt, stream);
  } else {
    if (gran_n == 128) launch_w8_form<C_E4M3, 128>(a, bf16, yt, stream);
    else launch_w8_form<C_E4M3, 1>(a, bf16, yt, stream);
  }
  return launch_status();
}

extern "C" sg_status sg_w8a16_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                                                             int64_t ldx, const uint8_t* wpacked, sg_dtype w_dt,
                                                             const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                             int gran_n, const float* bias, void* y, sg_dtype y_dt,
                                                             int64_t ldy, sg_form form, hipStream_t stream) {
  if (!x || !wpacked || !sw || !y) return SG_ERR_NULL;
  if (w_dt != SG_E4M3 && w_dt != SG_I8) return SG_ERR_UNSUPPORTED;
  if (gran_n != 1 && gran_n != 128) return SG_ERR_UNSUPPORTED;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldx < K) return SG_ERR_SHAPE;
  if (ldy < (form == SG_OUT_Y ? N : M)) return SG_ERR_SHAPE;
  // 32-bit buffer offsets: 64 X rows, and the 16 row blocks' chunks of a tile
  if (ldx >= (1LL << 24) || (K / 128) * 16 * PK_CHUNK >= (1LL << 31) || sw_sn < 0 || sw_sk < 0) return SG_ERR_SHAPE;
  if (((cdiv(N, gran_n) - 1) * sw_sn + (K / 128 - 1) * sw_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (cdiv(N, 16) > 0x7fffffffLL || cdiv(M, 16) > 65535) return SG_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * 2) % 16 || !aligned(wpacked, 16) || !aligned(sw, 4) || !aligned(bias, 4) ||
      !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  W8Args a;
  a.M = M; a.N = N; a.K = K;
  a.x = x; a.ldx = ldx;
  a.w = wpacked; a.ldw = 0; a.meta = wpacked; a.ldm = 0;
  a.sw = sw; a.sw_sn = sw_sn; a.sw_sk = sw_sk; a.gn_shift = gran_n == 128 ? 7 : 0;
  a.bias = bias;
  a.y = y; a.ldy = ldy;
  a.vec_store = (ldy % 4 == 0) && aligned(y, 4 * dtype_size(y_dt));
  clear_hip_error();
  const bool bf16 = y_dt == SG_BF16, yt = form == SG_OUT_YT;
  if (w_dt == SG_I8) {
    if (gran_n == 128) launch_w8_form<C_I8, 128, true>(a, bf16, yt, stream);
    else launch_w8_form<C_I8, 1, true>(a, bf16, yt, stream);
  } else {
    if (gran_n == 128) launch_w8_form<C_E4M3, 128, true>(a, bf16, yt, stream);
    else launch_w8_form<C_E4M3, 1, true>(a, bf16, yt, stream);
  }
  return launch_status();
}

extern "C" sg_status sg_w4a16_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                                                      int64_t ldx, const uint8_t* wv4, int64_t ldwv4,
                                                      const uint8_t* wmeta, int64_t ldwm, const float* sw,
                                                      int64_t sw_sn, int64_t sw_sk, const float* bias, void* y,
                                                      sg_dtype y_dt, int64_t ldy, sg_form form, hipStream_t stream) {
  if (!x || !wv4 || !wmeta || !sw || !y) return SG_ERR_NULL;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldx < K || ldwv4 < K / 4 || ldwm < K / 8) return SG_ERR_SHAPE;
  if (ldy < (form == SG_OUT_Y ? N : M)) return SG_ERR_SHAPE;
  if (ldx >= (1LL << 24) || ldwv4 >= (1LL << 24) || ldwm >= (1LL << 24) || sw_sn < 0 || sw_sk < 0) return SG_ERR_SHAPE;
  if (((N - 1) * sw_sn + (K / 128 - 1) * sw_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (cdiv(N, 16) > 0x7fffffffLL || cdiv(M, 16) > 65535) return SG_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * 2) % 16 || !aligned(wv4, 16) || ldwv4 % 16 || !aligned(wmeta, 16) || ldwm % 16 ||
      !aligned(sw, 4) || !aligned(bias, 4) || !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  W8Args a;
  a.M = M; a.N = N; a.K = K;
  a.x = x; a.ldx = ldx;
  a.w = wv4; a.ldw = ldwv4; a.meta = wmeta; a.ldm = ldwm;
  a.sw = sw; a.sw_sn = sw_sn; a.sw_sk = sw_sk; a.gn_shift = 0;
  a.bias = bias;
  a.y = y; a.ldy = ldy;
  a.vec_store = (ldy % 4 == 0) && aligned(y, 4 * dtype_size(y_dt));
  clear_hip_error();
  launch_w8_form<C_I4, 1>(a, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}

extern "C" sg_status sg_w4a16_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                                                             int64_t ldx, const uint8_t* wpacked, const float* sw,
                                                             int64_t sw_sn, int64_t sw_sk, const float* bias, void* y,
                                                             sg_dtype y_dt, int64_t ldy, sg_form form,
                                                             hipStream_t stream) {
  if (!x || !wpacked || !sw || !y) return SG_ERR_NULL;
  if (y_dt != SG_F32 && y_dt != SG_BF16) return SG_ERR_UNSUPPORTED;
  if (form != SG_OUT_Y && form != SG_OUT_YT) return SG_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || ldx < K) return SG_ERR_SHAPE;
  if (ldy < (form == SG_OUT_Y ? N : M)) return SG_ERR_SHAPE;
  // 32-bit buffer offsets: 64 X rows, and the 16 row blocks' chunks of a tile
  if (ldx >= (1LL << 24) || (K / 128) * 16 * PK4_CHUNK >= (1LL << 31) || sw_sn < 0 || sw_sk < 0) return SG_ERR_SHAPE;
  if (((N - 1) * sw_sn + (K / 128 - 1) * sw_sk) * 4 >= (1LL << 31)) return SG_ERR_SHAPE;
  if (cdiv(N, 16) > 0x7fffffffLL || cdiv(M, 16) > 65535) return SG_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * 2) % 16 || !aligned(wpacked, 16) || !aligned(sw, 4) || !aligned(bias, 4) ||
      !aligned(y, dtype_size(y_dt)))
    return SG_ERR_ALIGN;
  W8Args a;
  a.M = M; a.N = N; a.K = K;
  a.x = x; a.ldx = ldx;
  a.w = wpacked; a.ldw = 0; a.meta = wpacked; a.ldm = 0;
  a.sw = sw; a.sw_sn = sw_sn; a.sw_sk = sw_sk; a.gn_shift = 0;
  a.bias = bias;
  a.y = y; a.ldy = ldy;
  a.vec_store = (ldy % 4 == 0) && aligned(y, 4 * dtype_size(y_dt));
  clear_hip_error();
  launch_w8_form<C_I4, 1, true>(a, y_dt == SG_BF16, form == SG_OUT_YT, stream);
  return launch_status();
}
