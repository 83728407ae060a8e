// Weight repacking at handle creation: row-major bf16 weight -> fragment tiles.
//
// Runs once per shard (create), so it is written for clarity, not speed: each
// thread builds one 16-byte chunk (8 consecutive k of one column) by gathering
// from the row-major source.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

// src: row-major [K x ld] bf16.  dst: n_cb * k_blocks * 64 chunks.
// pairs = false: packed column c = 32*cb + lane%32 is source column c (zero if
//                c >= ncols_src).
// pairs = true:  block cb = 2p + half holds hidden features j = 32p + lane%32 of the
//                gate (half 0, source column j) or up (half 1, source column F + j)
//                branch; zero if j >= F.
// Rows k >= K are zero.
__global__ void __launch_bounds__(256)
k_pack_bf16(const uint16_t *__restrict__ src, int64_t ld, int64_t K, int64_t ncols_src,
            int pairs, int64_t F, int64_t n_cb, int64_t k_blocks, u32x4_t *__restrict__ dst) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = n_cb * k_blocks * 64;
  if (idx >= total) return;
  const int lane = static_cast<int>(idx & 63);
  const int64_t kb = (idx >> 6) % k_blocks;
  const int64_t cb = (idx >> 6) / k_blocks;
  int64_t col;
  bool valid;
  if (pairs) {
    const int64_t j = (cb >> 1) * kFragN + (lane & 31);
    valid = j < F;
    col = (cb & 1) * F + j;
  } else {
    col = cb * kFragN + (lane & 31);
    valid = col < ncols_src;
  }
  const int64_t k0 = kb * kFragK + 8 * (lane >> 5);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ka = k0 + 2 * i, kb2 = ka + 1;
    const uint32_t lo = (valid && ka < K) ? src[ka * ld + col] : 0u;
    const uint32_t hi = (valid && kb2 < K) ? src[kb2 * ld + col] : 0u;
    w[i] = lo | (hi << 16);
  }
  u32x4_t v = {w[0], w[1], w[2], w[3]};
  dst[idx] = v;
}

hipError_t launch_pack_bf16(const void *src, int64_t ld, int64_t K, int64_t ncols_src,
                            bool pairs, int64_t F, int64_t n_cb, int64_t k_blocks, void *dst,
                            hipStream_t s) {
  const int64_t total = n_cb * k_blocks * 64;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_pack_bf16, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint16_t *>(src), ld, K, ncols_src, pairs ? 1 : 0, F,
                     n_cb, k_blocks, static_cast<u32x4_t *>(dst));
  return hipGetLastError();
}

}  // namespace tpm
