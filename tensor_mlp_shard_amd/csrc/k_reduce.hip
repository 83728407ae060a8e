// On-device sum of k rank partials held on one GPU.
//
// This is the arithmetic of the all-reduce that closes a tensor-parallel MLP
// (page "大模型推理系统揭秘（07）Multi-GPU", section 1.2.3: Z = Z_0 + Z_1 + Z_2 +
// Z_3), i.e. the local-sum half of a one-shot all-reduce once the peers' partials
// sit in this GPU's memory.  Partials are added in fp32 (page "7.4 推理侧并行",
// section 7.4.2: low-precision transport is fine but the sum is done in high
// precision), in rank order, by one thread per element, so the result does not
// depend on the launch shape and is bitwise reproducible.
//
// Purely HBM-bound: 16-byte loads and stores, 8 elements per thread per step, a
// grid-stride loop sized to fill the GPU, scalar handling of the last numel % 8.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

constexpr int kMaxParts = 16;
struct PartPtrs {
  const void *p[kMaxParts];
};

template <int IN>
__device__ __forceinline__ void load8(const void *p, int64_t c, float (&v)[8]) {
  if constexpr (IN == TPM_F32) {
    const f32x4_t *q = static_cast<const f32x4_t *>(p) + 2 * c;
    const f32x4_t x0 = q[0], x1 = q[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = x0[i]; v[4 + i] = x1[i]; }
  } else {
    const u32x4_t x = static_cast<const u32x4_t *>(p)[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(x[i] << 16);
      v[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  }
}

template <int OUT>
__device__ __forceinline__ void store8(void *p, int64_t c, const float (&v)[8]) {
  if constexpr (OUT == TPM_F32) {
    f32x4_t *q = static_cast<f32x4_t *>(p) + 2 * c;
    q[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    q[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  } else {
    u32x4_t x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    static_cast<u32x4_t *>(p)[c] = x;
  }
}

template <int IN>
__device__ __forceinline__ float load1(const void *p, int64_t e) {
  if constexpr (IN == TPM_F32) return static_cast<const float *>(p)[e];
  else return bf16_to_f32(static_cast<const uint16_t *>(p)[e]);
}

template <int IN, int OUT>
__global__ void __launch_bounds__(256)
k_reduce(PartPtrs pp, int k, int64_t numel, void *__restrict__ out) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t n8 = numel >> 3;
  for (int64_t c = gid; c < n8; c += gstride) {
    float acc[8];
    load8<IN>(pp.p[0], c, acc);
    for (int i = 1; i < k; ++i) {
      float t[8];
      load8<IN>(pp.p[i], c, t);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += t[j];
    }
    store8<OUT>(out, c, acc);
  }
  const int64_t e = (n8 << 3) + gid;
  if (e < numel) {
    float a = load1<IN>(pp.p[0], e);
    for (int i = 1; i < k; ++i) a += load1<IN>(pp.p[i], e);
    if constexpr (OUT == TPM_F32) static_cast<float *>(out)[e] = a;
    else static_cast<uint16_t *>(out)[e] = f32_to_bf16(a);
  }
}

hipError_t launch_reduce(const void *const *parts, int k, int64_t numel, int in_dtype, void *out,
                         int out_dtype, hipStream_t s) {
  if (numel == 0) return hipSuccess;
  PartPtrs pp = {};
  for (int i = 0; i < k; ++i) pp.p[i] = parts[i];
  const int64_t n8 = numel >> 3;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (in_dtype == TPM_F32 && out_dtype == TPM_F32)
    hipLaunchKernelGGL((k_reduce<TPM_F32, TPM_F32>), grid, block, 0, s, pp, k, numel, out);
  else if (in_dtype == TPM_F32)
    hipLaunchKernelGGL((k_reduce<TPM_F32, TPM_BF16>), grid, block, 0, s, pp, k, numel, out);
  else if (out_dtype == TPM_F32)
    hipLaunchKernelGGL((k_reduce<TPM_BF16, TPM_F32>), grid, block, 0, s, pp, k, numel, out);
  else
    hipLaunchKernelGGL((k_reduce<TPM_BF16, TPM_BF16>), grid, block, 0, s, pp, k, numel, out);
  return hipGetLastError();
}

}  // namespace tpm
