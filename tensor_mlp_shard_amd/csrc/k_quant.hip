// Low-precision partials: FP8 transport with per-token scales, fp32 accumulation.
//
// Page "7.4 推理侧并行", section 7.4.2 (communication quantization): decode is
// bound by memory and communication, so the partials can travel in FP8 (half the
// bytes of FP16) with a per-token or per-channel scale, as long as the sum itself
// is done in high precision: dequantize to fp32 where the partials meet, add,
// and quantize again if the result travels on.  On one GPU the two halves are
// two kernels:
//
//  * k_quant_fp8: one workgroup per token row; the row's largest magnitude sets
//    the row scale s = amax / 448 (448 = largest finite E4M3 value), each element
//    is stored as the E4M3 code of x * (448 / amax), rounded to nearest, ties to
//    even, saturating at +-448 (the hardware FP8 conversion).  A zero row gets scale
//    1 and all-zero codes.
//  * k_reduce_fp8: element-wise, z = sum_i value(code_i) * s_i in rank order in
//    fp32; the codes are decoded by the hardware FP8 conversion, which reads OCP
//    E4M3 on gfx950.
//
// The pages name FP8 without fixing its layout; E4M3 here is the OCP 8-bit
// format the MI355X matrix cores use (1 sign, 4 exponent bits with bias 7, 3
// mantissa bits, subnormals, no infinities, 0x7f / 0xff NaN).  HBM-bound, 16-byte
// accesses; both divisions of the scale are correctly rounded, so the codes are
// a deterministic function of the fp32 input.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

// E4M3 codes of four fp32 values, packed little-endian into a word: the hardware
// conversion (v_cvt_pk_fp8_f32, OCP E4M3, round to nearest even).  On every finite
// value below 464 in magnitude it gives the code the definition asks for (checked on
// MI355X against a software rounding on the E4M3 grid for all 2^32 fp32 inputs: no
// difference below 464), and a finite row never produces more than 448 (1 + 2^-22).
// Clamping to +-448 first keeps the saturation of infinite products (a row whose amax
// is so small that 448 / amax overflows); NaN products take the NaN code 0x7f.
__device__ __forceinline__ uint32_t e4m3_x4(const float (&y)[4]) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(y[i], -448.0f), 448.0f);
  int t = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  t = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], t, true);
  uint32_t b = static_cast<uint32_t>(t);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (!(y[i] == y[i])) b = (b & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
  return b;
}

template <int IN>
__device__ __forceinline__ void load16(const void *p, int64_t c, float (&v)[16]) {
  if constexpr (IN == TPM_F32) {
    const f32x4_t *q = static_cast<const f32x4_t *>(p) + 4 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t x = q[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = x[i];
    }
  } else {
    const u32x4_t *q = static_cast<const u32x4_t *>(p) + 2 * c;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4_t x = q[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * j + 2 * i] = __uint_as_float(x[i] << 16);
        v[8 * j + 2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
      }
    }
  }
}

// One row per workgroup, NCH chunks of 16 columns per thread held in registers.
template <int IN, int NCH>
__global__ void __launch_bounds__(1024)
k_quant_fp8(const void *__restrict__ x, int cols16, u32x4_t *__restrict__ q,
            float *__restrict__ scale) {
  __shared__ float wmax[16];
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * cols16;
  float v[NCH][16];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * blockDim.x;
    if (c < cols16) {
      load16<IN>(x, row0 + c, v[j]);
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  if (tid == 0) {
    float t = wmax[0];
    for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) t = fmaxf(t, wmax[w]);
    wmax[0] = t;
  }
  __syncthreads();
  amax = wmax[0];
  const bool zero = !(amax > 0.0f);
  const float inv = zero ? 1.0f : __fdiv_rn(448.0f, amax);
  if (tid == 0) scale[blockIdx.x] = zero ? 1.0f : __fdiv_rn(amax, 448.0f);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * blockDim.x;
    if (c < cols16) {
      u32x4_t o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = __fmul_rn(v[j][4 * w + i], inv);
        o[w] = e4m3_x4(y);
      }
      q[row0 + c] = o;
    }
  }
}

constexpr int kMaxFp8Parts = 16;
struct Fp8Parts {
  const u32x4_t *q[kMaxFp8Parts];
  const float *s[kMaxFp8Parts];
};

template <int OUT>
__global__ void __launch_bounds__(256)
k_reduce_fp8(Fp8Parts pp, int k, int64_t n16, int cols16, void *__restrict__ out) {
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n16;
       c += gstride) {
    const int64_t row = c / cols16;
    float acc[16];
    for (int i0 = 0; i0 < k; i0 += 8) {
      u32x4_t t[8];
      float s[8];
#pragma unroll
      for (int p = 0; p < 8; ++p)
        if (i0 + p < k) {
          t[p] = pp.q[i0 + p][c];
          s[p] = pp.s[i0 + p][row];
        }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        if (i0 + p >= k) break;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // the matrix-core FP8 conversion of gfx950 reads OCP E4M3 (measured:
          // identical to the format's definition on all 256 codes); two codes per instruction
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(t[p][w]), false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(t[p][w]), true);
          const float d[4] = {lo[0] * s[p], lo[1] * s[p], hi[0] * s[p], hi[1] * s[p]};
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * w + i] = (i0 + p == 0) ? d[i] : acc[4 * w + i] + d[i];
        }
      }
    }
    if constexpr (OUT == TPM_F32) {
      f32x4_t *o = static_cast<f32x4_t *>(out) + 4 * c;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f32x4_t{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
    } else {
      u32x4_t *o = static_cast<u32x4_t *>(out) + 2 * c;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = static_cast<uint32_t>(f32_to_bf16(acc[8 * j + 2 * i])) |
                 (static_cast<uint32_t>(f32_to_bf16(acc[8 * j + 2 * i + 1])) << 16);
        o[j] = w;
      }
    }
  }
}

hipError_t launch_quant_fp8(const void *x, int64_t rows, int64_t cols, int in_dtype, void *q,
                            float *scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols % 16 || cols > kFp8MaxCols) return hipErrorInvalidValue;
  const int cols16 = static_cast<int>(cols / 16);
  const int bs = cols16 >= 1024 ? 1024 : ((cols16 + 63) / 64) * 64;
  const int nch = (cols16 + bs - 1) / bs;
  dim3 grid(static_cast<unsigned>(rows)), block(bs);
  u32x4_t *qq = static_cast<u32x4_t *>(q);
#define TPM_QUANT(IN, N) \
  hipLaunchKernelGGL((k_quant_fp8<IN, N>), grid, block, 0, s, x, cols16, qq, scale)
  if (in_dtype == TPM_F32) {
    if (nch == 1) TPM_QUANT(TPM_F32, 1);
    else TPM_QUANT(TPM_F32, 2);
  } else {
    if (nch == 1) TPM_QUANT(TPM_BF16, 1);
    else TPM_QUANT(TPM_BF16, 2);
  }
#undef TPM_QUANT
  return hipGetLastError();
}

hipError_t launch_reduce_fp8(const void *const *q, const float *const *scales, int k, int64_t rows,
                             int64_t cols, void *out, int out_dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols % 16 || k < 1 || k > kMaxFp8Parts) return hipErrorInvalidValue;
  Fp8Parts pp = {};
  for (int i = 0; i < k; ++i) {
    pp.q[i] = static_cast<const u32x4_t *>(q[i]);
    pp.s[i] = scales[i];
  }
  const int64_t n16 = rows * (cols / 16);
  // small blocks so that a decode-size sum (16 K chunks) still spreads over every CU
  const int bs = n16 >= (int64_t(1) << 18) ? 256 : 64;
  int64_t blocks = (n16 + bs - 1) / bs;
  if (blocks > 4096) blocks = 4096;
  const int cols16 = static_cast<int>(cols / 16);
  if (out_dtype == TPM_F32)
    hipLaunchKernelGGL((k_reduce_fp8<TPM_F32>), dim3(static_cast<unsigned>(blocks)), dim3(bs), 0,
                       s, pp, k, n16, cols16, out);
  else
    hipLaunchKernelGGL((k_reduce_fp8<TPM_BF16>), dim3(static_cast<unsigned>(blocks)), dim3(bs), 0,
                       s, pp, k, n16, cols16, out);
  return hipGetLastError();
}

}  // namespace tpm
