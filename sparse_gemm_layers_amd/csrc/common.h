// Shared host/device helpers of the gfx950 kernels: vector types, the e4m3 and
// bf16 encoders, wave reductions and the host-side argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "sg.h"

// Device-only code (buffer resources and the kernel bodies that use them) is
// hidden from the host compilation pass, which only needs the kernel stubs.
#if defined(__HIP_DEVICE_COMPILE__)
#define SG_DEVICE_PASS 1
#else
#define SG_DEVICE_PASS 0
#endif

namespace sg {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- encoders

// fp32 -> OCP e4m3 ("e4m3fn") codes of four values, packed little-endian in
// a dword: round to nearest, ties to even, saturate at +-448 (infinities
// included), keep the sign (a negative value that rounds to zero gives 0x80),
// and give every NaN the one code 0x7F.  The values are clamped to +-448 first
// because the conversion instruction turns overflow into NaN; the clamp would
// turn NaN into -448, so NaN lanes are patched afterwards.  Over every finite
// fp32 input the codes equal those of an integer-only round-to-nearest-even
// encoder (checked exhaustively on MI355X, all 2^32 bit patterns).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  const uint32_t nan = (a != a ? 0xffu : 0u) | (b != b ? 0xff00u : 0u) | (c != c ? 0xff0000u : 0u) |
                       (d != d ? 0xff000000u : 0u);
  return ((uint32_t)w & ~nan) | (0x7f7f7f7fu & nan);
}

// e4m3_pack4 for values known not to be NaN (no NaN patch; infinities still
// saturate through the clamp).
__device__ __forceinline__ uint32_t e4m3_pack4_finite(float a, float b, float c, float d) {
  const auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}

// |v| folded into a running block maximum a (a >= 0).  Non-negative floats
// order like their bit patterns and every NaN pattern lies above +inf, so the
// maximum is taken on the bits: a block holding a NaN gets a NaN maximum
// (fmaxf would drop it).
__device__ __forceinline__ float amax_fold(float a, float v) {
  return __uint_as_float(max(__float_as_uint(a), __float_as_uint(v) & 0x7fffffffu));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits of two values (a in the low half): round to nearest even,
// NaN stays NaN (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16 bits of one value, as above.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return f32x2_to_bf16x2(f, 0.0f) & 0xffffu; }

// ---------------------------------------------------------------- loads

// Four consecutive inputs as fp32.  float: one 16-byte load; bf16: one 8-byte load.
__device__ __forceinline__ void load4(const float* p, float v[4]) {
  const float4 t = *reinterpret_cast<const float4*>(p);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(t.x << 16);
  v[1] = __uint_as_float(t.x & 0xffff0000u);
  v[2] = __uint_as_float(t.y << 16);
  v[3] = __uint_as_float(t.y & 0xffff0000u);
}

// Max of non-negative values (NaN patterns included, see amax_fold) over
// groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_max(float a) {
  uint32_t u = __float_as_uint(a);
#pragma unroll
  for (int o = WIDTH / 2; o >= 1; o >>= 1) u = max(u, (uint32_t)__shfl_xor((int)u, o, 64));
  return __uint_as_float(u);
}

// Scale of a block from its maximum magnitude a: a / qmax (an IEEE divide),
// 1 for an all-zero block; a NaN maximum gives a NaN scale and an infinite
// one an infinite scale.
__device__ __forceinline__ float block_scale(float a, float qmax) { return a == 0.0f ? 1.0f : a / qmax; }

// ---------------------------------------------------------------- host checks

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t dtype_size(sg_dtype d) { return d == SG_F32 ? 4 : d == SG_BF16 ? 2 : 1; }

// Clears any stale error of this host thread, so that the check after a
// launch reports the launch itself.
inline void clear_hip_error() { (void)hipGetLastError(); }

inline sg_status launch_status() { return hipGetLastError() == hipSuccess ? SG_OK : SG_ERR_HIP; }

// Workgroup count for grid-stride loops: enough to fill 256 CUs several times.
// Compute units of the current device (queried once per device).
inline int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

inline unsigned grid_for(int64_t items, int per_group, unsigned cap = 4096) {
  const int64_t g = cdiv(items, per_group);
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace sg
