// Device helpers shared by the HIP kernels: 16-byte vector types, bf16
// conversion (round-to-nearest-even on the bit pattern) and the gfx950 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, nearest-even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Activations of the fused gate|up epilogue, fp32 (act codes of the ABI:
// 0 gelu with the tanh approximation, 1 silu, 2 gelu with erf).  The tanh
// form is evaluated through 0.5 (1 + tanh u) = 1 / (1 + e^-2u), so
// gelu_tanh(x) = x / (1 + e^(-2u)) with the hardware exponential (relative
// error ~1e-6, far below the bf16 rounding of the result; it tends to 0 and
// to x at the two ends as the tanh form does).
__device__ __forceinline__ float activation(int act, float x) {
  if (act == 1) return x / (1.f + __expf(-x));
  if (act == 2) return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
  const float u = 0.79788456080286536f * (x + 0.044715f * x * x * x);
  return x / (1.f + __expf(-2.f * u));
}

// D += A * B for a 16x16 output tile over 32 k.  Lane l supplies A row (l & 15)
// and B column (l & 15), each as 8 bf16 at k-slots 8*(l >> 4) .. +7 (any
// k-permutation works as long as A and B use the same one); lane l receives
// D rows 4*(l >> 4) .. +3 of column (l & 15).
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

}  // namespace wl
