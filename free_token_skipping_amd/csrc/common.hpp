// Shared device helpers for the SPTS gfx950 kernels: bf16 conversions, MFMA
// vector types, wave reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spts {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two fp32 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// RMSNorm pieces shared by every kernel that normalises a row, so that they all
// produce the same bf16 values: sum of squares of 8 bf16 values added to ss in
// a fixed order, and 1/sqrt(mean + eps) from a 256-thread block's four wave sums.
__device__ __forceinline__ float sumsq8(const u32x4& v, float ss) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a = lo_bf(v[w]), b = hi_bf(v[w]);
    ss += a * a + b * b;
  }
  return ss;
}
__device__ __forceinline__ float rms_inv(const float* red, int d, float eps) {
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  return 1.0f / sqrtf(tot / (float)d + eps);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// 16-byte global load/store through plain vector accesses.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace spts
