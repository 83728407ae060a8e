// fp32 projection with fused activation, for fp32 inputs (small shapes).
//
// fp32 weights have no matrix-core fast path here worth the complexity: this is a
// plain 16 x 16 LDS-tiled vector-ALU product with any M, K, N (bounds-checked),
// used for fp32 shards such as the two-rank toy MLP.  Each thread owns one output
// and, for SiLU-gate, accumulates the gate and the up column side by side.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

constexpr int kF32Tile = 16;

// out[m][n] = epi( sum_k A[m][k] * B[k][n] )  (SiLU-gate: up column = n + up_off)
template <int EPI>
__global__ void __launch_bounds__(kF32Tile * kF32Tile)
k_f32(const float *__restrict__ A, int64_t lda, int M, int K, const float *__restrict__ B,
      int64_t ldb, int N, int64_t up_off, void *__restrict__ out, int64_t ldo) {
  __shared__ float as[kF32Tile][kF32Tile + 1];
  __shared__ float bg[kF32Tile][kF32Tile + 1];
  __shared__ float bu[kF32Tile][kF32Tile + 1];
  const int tx = threadIdx.x, ty = threadIdx.y;
  const int row = blockIdx.y * kF32Tile + ty;
  const int col = blockIdx.x * kF32Tile + tx;
  float g = 0.0f, u = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kF32Tile) {
    as[ty][tx] = (row < M && k0 + tx < K) ? A[static_cast<int64_t>(row) * lda + k0 + tx] : 0.0f;
    const bool bk = (k0 + ty < K) && col < N;
    bg[ty][tx] = bk ? B[static_cast<int64_t>(k0 + ty) * ldb + col] : 0.0f;
    if constexpr (EPI == EPI_SILU_GATE)
      bu[ty][tx] = bk ? B[static_cast<int64_t>(k0 + ty) * ldb + up_off + col] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32Tile; ++kk) {
      g = fmaf(as[ty][kk], bg[kk][tx], g);
      if constexpr (EPI == EPI_SILU_GATE) u = fmaf(as[ty][kk], bu[kk][tx], u);
    }
    __syncthreads();
  }
  if (row >= M || col >= N) return;
  const int64_t o = static_cast<int64_t>(row) * ldo + col;
  if constexpr (EPI == EPI_SILU_GATE) static_cast<float *>(out)[o] = silu_f(g) * u;
  else if constexpr (EPI == EPI_TANH || EPI == EPI_IDENTITY) static_cast<float *>(out)[o] = act_f<EPI>(g);
  else if constexpr (EPI == EPI_OUT_F32) static_cast<float *>(out)[o] = g;
  else static_cast<uint16_t *>(out)[o] = f32_to_bf16(g);
}

template <int EPI>
static hipError_t launch_f32_one(const float *A, int64_t lda, int64_t M, int64_t K, const float *B,
                                 int64_t ldb, int64_t N, int64_t up_off, void *out, int64_t ldo,
                                 hipStream_t s, const Timing &t) {
  dim3 grid(static_cast<unsigned>((N + kF32Tile - 1) / kF32Tile),
            static_cast<unsigned>((M + kF32Tile - 1) / kF32Tile));
  hipExtLaunchKernelGGL((k_f32<EPI>), grid, dim3(kF32Tile, kF32Tile), 0, s, t.start, t.stop, 0, A, lda,
                     static_cast<int>(M), static_cast<int>(K), B, ldb, static_cast<int>(N), up_off,
                     out, ldo);
  return hipGetLastError();
}

hipError_t launch_f32_gemm(int epi, const float *A, int64_t lda, int64_t M, int64_t K,
                           const float *B, int64_t ldb, int64_t N, int64_t up_off, void *out,
                           int64_t ldo, hipStream_t s, const Timing &t) {
  switch (epi) {
    case EPI_SILU_GATE: return launch_f32_one<EPI_SILU_GATE>(A, lda, M, K, B, ldb, N, up_off, out, ldo, s, t);
    case EPI_TANH: return launch_f32_one<EPI_TANH>(A, lda, M, K, B, ldb, N, up_off, out, ldo, s, t);
    case EPI_IDENTITY: return launch_f32_one<EPI_IDENTITY>(A, lda, M, K, B, ldb, N, up_off, out, ldo, s, t);
    case EPI_OUT_F32: return launch_f32_one<EPI_OUT_F32>(A, lda, M, K, B, ldb, N, up_off, out, ldo, s, t);
    case EPI_OUT_BF16: return launch_f32_one<EPI_OUT_BF16>(A, lda, M, K, B, ldb, N, up_off, out, ldo, s, t);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpm
