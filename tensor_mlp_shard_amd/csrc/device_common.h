// Device-side helpers shared by the HIP kernels of libtpmlp (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpm_internal.h"

namespace tpm {

// 8 bf16 = one 128-bit register quad, the per-lane operand of the bf16 MFMA.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

template <int EPI>
__device__ __forceinline__ float act_f(float s) {
  if constexpr (EPI == EPI_TANH) return tanhf(s);
  else return s;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// D = A(32x16) * B(16x32) + C on the matrix cores.  Lane l supplies
// A[l % 32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l % 32]; it receives
// D[8*(r/4) + 4*(l/32) + r%4][l % 32] in register r (0..15).
__device__ __forceinline__ f32x16_t mfma_32x32x16(const u32x4_t a, const u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C on the matrix cores.  Lane l supplies
// A[l % 16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l % 16]; it receives
// D[4*(l/16) + r][l % 16] in register r (0..3).  (Checked on MI355X with small
// integer operands.)
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Contraction index of element i (0..7) of lane half h in k-step s (fragment order).
__host__ __device__ __forceinline__ int kappa(int s, int h, int i) {
  return 32 * (s >> 1) + 16 * h + 8 * (s & 1) + i;
}

// Row (within the 32x32 output tile) held in accumulator register r by lane l.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace tpm
