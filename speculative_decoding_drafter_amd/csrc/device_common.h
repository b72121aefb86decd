// Device helpers shared by the libspecopd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specopd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// bf16 <-> fp32.  A bf16 value is the high half of the fp32 with the same bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16 bits by the hardware conversion
// (v_cvt_pk_bf16_f32; NaN stays NaN).  An integer form of the rounding with
// its NaN test compiled to an exec-masked branch per value, which made
// writing a 256-row attention output take ~10,000 cycles.
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_cvt v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the transcendental unit (no denormal fix-up; results below the
// smallest normal flush to zero, far below anything these kernels sum).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Scalar element access for fp32 arrays and bf16 arrays (stored as uint16_t).
__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f32(uint16_t* p, float v) { *p = f32_to_bf16(v); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Running (max, sum of 2^((x - max) * log2 e)) pair merge, -inf aware.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float mm = fmaxf(m, m2);
  if (mm == kNegInf) { m = mm; s = 0.f; return; }
  s = s * fast_exp2((m - mm) * kLog2e) + s2 * fast_exp2((m2 - mm) * kLog2e);
  m = mm;
}

}  // namespace specopd
