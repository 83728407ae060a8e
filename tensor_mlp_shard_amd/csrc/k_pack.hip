// Weight repacking at handle creation: row-major bf16 weight -> fragment order.
//
// Runs once per shard (create), so it is written for clarity, not speed: each
// thread builds one 16-byte chunk (8 contraction indices of one column) by
// gathering from the row-major source.  The layout is described in
// tpm_internal.h.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

// src: row-major [K x ld] bf16.  dst: ks * n_cb * 64 chunks, k-step major.
// pairs = false: column c = 32*cb + lane%32 is source column c (zero if
//                c >= ncols_src).
// pairs = true:  block cb holds, for hidden features j = 16*cb + (lane%32)%16, the
//                gate weight (lane%32 < 16, source column j) or the up weight
//                (lane%32 >= 16, source column F + j); zero if j >= F.
// Contraction indices k >= K are zero.
__global__ void __launch_bounds__(256)
k_pack_bf16(const uint16_t *__restrict__ src, int64_t ld, int64_t K, int64_t ncols_src,
            int pairs, int64_t F, int64_t n_cb, int64_t ks, u32x4_t *__restrict__ dst) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = n_cb * ks * 64;
  if (idx >= total) return;
  const int lane = static_cast<int>(idx & 63);
  const int s = static_cast<int>((idx >> 6) / n_cb);
  const int64_t cb = (idx >> 6) % n_cb;
  const int c = lane & 31;
  int64_t col;
  bool valid;
  if (pairs) {
    const int64_t j = cb * 16 + (c & 15);
    valid = j < F;
    col = (c < 16 ? 0 : F) + j;
  } else {
    col = cb * kFragN + c;
    valid = col < ncols_src;
  }
  const int h = lane >> 5;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t ka = kappa(s, h, 2 * q), kb = ka + 1;
    const uint32_t lo = (valid && ka < K) ? src[ka * ld + col] : 0u;
    const uint32_t hi = (valid && kb < K) ? src[kb * ld + col] : 0u;
    w[q] = lo | (hi << 16);
  }
  u32x4_t v = {w[0], w[1], w[2], w[3]};
  dst[idx] = v;
}

hipError_t launch_pack_bf16(const void *src, int64_t ld, int64_t K, int64_t ncols_src,
                            bool pairs, int64_t F, int64_t n_cb, int64_t ks, void *dst,
                            hipStream_t s) {
  const int64_t total = n_cb * ks * 64;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_pack_bf16, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint16_t *>(src), ld, K, ncols_src, pairs ? 1 : 0, F,
                     n_cb, ks, static_cast<u32x4_t *>(dst));
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) k_zero_i32(int *__restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_i32(int *p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_i32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p,
                     n);
  return hipGetLastError();
}

}  // namespace tpm
