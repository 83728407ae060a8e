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

// acc = ((p_0 + p_1) + ...) + p_{k-1} for one chunk of 8 elements.  The loads of up
// to 8 partials are issued together (k is uniform, so the guards are scalar
// branches), so a chunk costs one memory round trip per 8 partials instead of one
// per partial.
template <int IN>
__device__ __forceinline__ void sum_parts8(const PartPtrs &pp, int k, int64_t c, float (&acc)[8]) {
  for (int i0 = 0; i0 < k; i0 += 8) {
    float t[8][8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (i0 + q < k) load8<IN>(pp.p[i0 + q], c, t[q]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (i0 + q >= k) break;
      if (i0 + q == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = t[0][j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += t[q][j];
      }
    }
  }
}

template <int IN, int OUT>
__global__ void __launch_bounds__(256)
k_reduce(PartPtrs pp, int k, int64_t numel, void *__restrict__ out) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t n8 = numel >> 3;
  for (int64_t c = gid; c < n8; c += gstride) {
    float acc[8];
    sum_parts8<IN>(pp, k, c, acc);
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
  // small blocks so that a decode-size sum (32 K chunks of 8) still spreads over every
  // compute unit: 512 workgroups of 64 threads rather than 128 of 256
  const int bs = n8 >= (int64_t(1) << 18) ? 256 : 64;
  int64_t blocks = (n8 + bs - 1) / bs;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  dim3 grid(static_cast<unsigned>(blocks)), block(bs);
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

// ---------------------------------------------------------------------------
// The step after the all-reduce, fused with it (page "7.4 推理侧并行", section
// 7.4.2, the kernel-fusion remedy: the residual add and RMSNorm that follow the
// all-reduce run in the same kernel, saving a round trip through device memory).
// Per row: z = sum of the k partials (rank order, fp32), h = residual + z,
// residual_out = h, y = h / sqrt(mean(h^2) + eps) * gamma.  RMSNorm is not defined
// on the pages; this is its textbook form, computed from the fp32 h.
//
// One workgroup per row: each thread owns NCH chunks of 8 columns, keeps their h in
// registers between the two passes, and the row's sum of squares meets in LDS in
// a fixed order, so results are bitwise reproducible.  HBM-bound: the partials and
// the residual are read once, both outputs written once.
template <int IN, int RES, int OUT, int NCH>
__global__ void __launch_bounds__(1024)
k_reduce_norm(PartPtrs pp, int k, int cols8, const void *__restrict__ res_in,
              void *__restrict__ res_out, const void *__restrict__ gamma, float eps, float inv_cols,
              void *__restrict__ y) {
  __shared__ float wsum[16];
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * cols8;  // first chunk of the row
  // gamma is loaded with the inputs when one chunk per thread leaves the registers
  // for it (the common case, cols <= 8192), else after the row reduction
  constexpr bool kEarlyGamma = NCH == 1;
  float h[NCH][8], g[NCH][8];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * blockDim.x;
    if (c < cols8) {
      float r[8];
      if constexpr (kEarlyGamma) load8<RES>(gamma, c, g[j]);
      load8<RES>(res_in, row0 + c, r);
      sum_parts8<IN>(pp, k, row0 + c, h[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[j][e] = r[e] + h[j][e];
        ss += h[j][e] * h[j][e];
      }
      store8<RES>(res_out, row0 + c, h[j]);
    }
  }
  // Row sum of squares: wave reduction, then the waves in order.
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float t = wsum[0];
    for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) t += wsum[w];
    wsum[0] = t;
  }
  __syncthreads();
  const float inv = 1.0f / sqrtf(wsum[0] * inv_cols + eps);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * blockDim.x;
    if (c < cols8) {
      float o[8];
      if constexpr (!kEarlyGamma) load8<RES>(gamma, c, g[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = h[j][e] * inv * g[j][e];
      store8<OUT>(y, row0 + c, o);
    }
  }
}

template <int IN, int RES, int OUT>
static hipError_t launch_norm3(const PartPtrs &pp, int k, int64_t rows, int cols8,
                               const void *res_in, void *res_out, const void *gamma, float eps,
                               void *y, hipStream_t s) {
  const int bs = cols8 >= 1024 ? 1024 : ((cols8 + 63) / 64) * 64;
  const int nch = (cols8 + bs - 1) / bs;
  const float inv_cols = 1.0f / static_cast<float>(8 * cols8);
  dim3 grid(static_cast<unsigned>(rows)), block(bs);
  if (nch == 1)
    hipLaunchKernelGGL((k_reduce_norm<IN, RES, OUT, 1>), grid, block, 0, s, pp, k, cols8, res_in,
                       res_out, gamma, eps, inv_cols, y);
  else if (nch == 2)
    hipLaunchKernelGGL((k_reduce_norm<IN, RES, OUT, 2>), grid, block, 0, s, pp, k, cols8, res_in,
                       res_out, gamma, eps, inv_cols, y);
  else if (nch <= 4)
    hipLaunchKernelGGL((k_reduce_norm<IN, RES, OUT, 4>), grid, block, 0, s, pp, k, cols8, res_in,
                       res_out, gamma, eps, inv_cols, y);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int IN, int RES>
static hipError_t launch_norm2(const PartPtrs &pp, int k, int64_t rows, int cols8,
                               const void *res_in, void *res_out, const void *gamma, float eps,
                               void *y, int out_dtype, hipStream_t s) {
  return out_dtype == TPM_F32
             ? launch_norm3<IN, RES, TPM_F32>(pp, k, rows, cols8, res_in, res_out, gamma, eps, y, s)
             : launch_norm3<IN, RES, TPM_BF16>(pp, k, rows, cols8, res_in, res_out, gamma, eps, y, s);
}

hipError_t launch_reduce_norm(const void *const *parts, int k, int64_t rows, int64_t cols,
                              int in_dtype, const void *res_in, void *res_out, int res_dtype,
                              const void *gamma, float eps, void *y, int out_dtype,
                              hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols % 8 || cols > kNormMaxCols) return hipErrorInvalidValue;
  PartPtrs pp = {};
  for (int i = 0; i < k; ++i) pp.p[i] = parts[i];
  const int cols8 = static_cast<int>(cols / 8);
  if (in_dtype == TPM_F32)
    return res_dtype == TPM_F32
               ? launch_norm2<TPM_F32, TPM_F32>(pp, k, rows, cols8, res_in, res_out, gamma, eps, y, out_dtype, s)
               : launch_norm2<TPM_F32, TPM_BF16>(pp, k, rows, cols8, res_in, res_out, gamma, eps, y, out_dtype, s);
  return res_dtype == TPM_F32
             ? launch_norm2<TPM_BF16, TPM_F32>(pp, k, rows, cols8, res_in, res_out, gamma, eps, y, out_dtype, s)
             : launch_norm2<TPM_BF16, TPM_BF16>(pp, k, rows, cols8, res_in, res_out, gamma, eps, y, out_dtype, s);
}

// ---------------------------------------------------------------------------
// Merge of k attention partials held on one GPU (page "LLM 推理并行化：先找瓶颈，再决定
// 怎么切", section 三.4, decode context parallelism: each rank attends over its own
// part of the KV history and reports its local score maximum m_i, its sum of
// exponentials s_i and its exponential-weighted value sum v_i, all relative to
// m_i).  Per row: g = max_i m_i, c_i = exp(m_i - g), out = (sum_i c_i v_i) /
// (sum_i c_i s_i), sums in rank order in fp32.  A rank without keys (m_i = -inf)
// has c_i = 0; a row without keys on any rank gives 0.  Optionally the merged
// statistics (g, sum_i c_i s_i) are written, so that a merged result can be merged
// again.
//
// One thread per 8 values of a row: it reads the row's 2k statistics (cache hits
// for all but the first thread of the row), then the k value chunks, 8 ranks' loads
// in flight at a time.  HBM-bound.
struct StatPtrs {
  const float *p[kMaxParts];
};

template <int IN, int OUT>
__global__ void __launch_bounds__(256)
k_attn_merge(PartPtrs vp, StatPtrs mp, StatPtrs sp, int k, int64_t rows, int dim8,
             void *__restrict__ out, float *__restrict__ m_out, float *__restrict__ s_out) {
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t n = rows * dim8;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n;
       c += gstride) {
    const int64_t r = c / dim8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.0f, g = -INFINITY;
    // Rescaled sums of ranks [i0, i0 + 8) in rank order (the statistics and value
    // chunks already in registers).
    auto add8 = [&](int i0, const float (&mi)[8], const float (&si)[8], const float (&v)[8][8]) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (i0 + q >= k) break;
        const float ci = mi[q] == -INFINITY ? 0.0f : expf(mi[q] - g);
        den += ci * si[q];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += ci * v[q][j];
      }
    };
    // The loads of up to 8 ranks are issued together (k is uniform, so the guards
    // are scalar branches).
    auto load_ranks = [&](int i0, float (&mi)[8], float (&si)[8], float (&v)[8][8]) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        mi[q] = -INFINITY;
        if (i0 + q < k) {
          mi[q] = mp.p[i0 + q][r];
          si[q] = sp.p[i0 + q][r];
          load8<IN>(vp.p[i0 + q], c, v[q]);
        }
      }
    };
    float mi[8], si[8], v[8][8];
    if (k <= 8) {
      // One round of loads: maxima, sums and values together.
      load_ranks(0, mi, si, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) g = fmaxf(g, mi[q]);
      if (g != -INFINITY) add8(0, mi, si, v);
    } else {
      // The global maximum first, then the ranks 8 at a time.
      for (int i0 = 0; i0 < k; i0 += 8) {
        float t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = i0 + q < k ? mp.p[i0 + q][r] : -INFINITY;
#pragma unroll
        for (int q = 0; q < 8; ++q) g = fmaxf(g, t[q]);
      }
      if (g != -INFINITY) {
        for (int i0 = 0; i0 < k; i0 += 8) {
          load_ranks(i0, mi, si, v);
          add8(i0, mi, si, v);
        }
      }
    }
    if (g != -INFINITY) {
      const float d = den != 0.0f ? den : 1.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = acc[j] / d;
    }
    store8<OUT>(out, c, acc);
    if (m_out && c - r * dim8 == 0) {
      m_out[r] = g;
      s_out[r] = den;
    }
  }
}

hipError_t launch_attn_merge(const void *const *values, const float *const *maxima,
                             const float *const *expsums, int k, int64_t rows, int64_t dim,
                             int in_dtype, void *out, int out_dtype, float *max_out,
                             float *expsum_out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (k < 1 || k > kMaxParts || dim % 8 || dim < 8 || dim / 8 > 0x7fffffff)
    return hipErrorInvalidValue;
  PartPtrs vp = {};
  StatPtrs mp = {}, sp = {};
  for (int i = 0; i < k; ++i) {
    vp.p[i] = values[i];
    mp.p[i] = maxima[i];
    sp.p[i] = expsums[i];
  }
  const int dim8 = static_cast<int>(dim / 8);
  const int64_t n = rows * dim8;
  constexpr int kThreads = 64;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if (in_dtype == TPM_F32 && out_dtype == TPM_F32)
    hipLaunchKernelGGL((k_attn_merge<TPM_F32, TPM_F32>), grid, block, 0, s, vp, mp, sp, k, rows, dim8, out, max_out, expsum_out);
  else if (in_dtype == TPM_F32)
    hipLaunchKernelGGL((k_attn_merge<TPM_F32, TPM_BF16>), grid, block, 0, s, vp, mp, sp, k, rows, dim8, out, max_out, expsum_out);
  else if (out_dtype == TPM_F32)
    hipLaunchKernelGGL((k_attn_merge<TPM_BF16, TPM_F32>), grid, block, 0, s, vp, mp, sp, k, rows, dim8, out, max_out, expsum_out);
  else
    hipLaunchKernelGGL((k_attn_merge<TPM_BF16, TPM_BF16>), grid, block, 0, s, vp, mp, sp, k, rows, dim8, out, max_out, expsum_out);
  return hipGetLastError();
}

}  // namespace tpm
