// Host-side internals of libtpmlp: the shard handle and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tp_mlp_shard.h"

namespace tpm {

// Epilogue kinds.  The first three produce the hidden activations (bf16 or fp32),
// the last two write the rank partial.
enum Epi : int {
  EPI_SILU_GATE = 0,  // h = SiLU(gate) * up; gate and up accumulate side by side
  EPI_TANH = 1,       // h = tanh(s)
  EPI_IDENTITY = 2,   // h = s
  EPI_OUT_F32 = 3,    // partial stored as fp32
  EPI_OUT_BF16 = 4,   // partial stored as bf16
};


// Packed weight layout ("fragment tiles").  A logical weight W [K x N] (K rows =
// the contraction index) is stored as 16-byte chunks indexed
//   ((cb * nKb + kb) * 64 + lane),   cb = column block of 32, kb = k block of 16,
// where chunk (cb, kb, lane) holds W[16*kb + 8*(lane/32) + i][32*cb + lane%32],
// i = 0..7, as 8 bf16.  That is exactly the B operand of one 32x32x16 bf16 MFMA for
// a wave, so one wave-wide 1 KiB load is one operand and the bytes of a column
// block are contiguous along K.  K is zero-padded to a multiple of 64 and N to a
// multiple of 256.
//
// For the SiLU-gate first weight the column blocks alternate gate / up over the
// same hidden indices: block 2p holds gate features [32p, 32p+32), block 2p+1 the
// up features with the same indices, so one tile always owns matching pairs.
constexpr int kFragK = 16;       // k per MFMA fragment
constexpr int kFragN = 32;       // columns per fragment
constexpr int kTileM = 256;      // tiled (prefill) kernel: rows per block
constexpr int kTileN = 256;      // tiled kernel: columns per block
constexpr int kTileK = 64;       // tiled kernel: k per LDS stage
constexpr int kStreamMaxTokens = 64;  // AUTO: streaming kernels for M <= this

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct StreamCfg {
  int mt;      // 32-row token tiles per wave (1 or 2)
  int ksplit;  // workgroups sharing one column unit along K
  int units;   // column units (one or two 32-column blocks each)
  int zgroups; // token groups of 32*mt rows (grid z)
};

struct Shard {
  tpm_desc desc;
  int device;
  int64_t ffn_pad;   // F padded (bf16 path)
  int64_t n1;        // packed columns of the first weight
  int64_t n2;        // packed columns of the second weight (d padded to 256)
  int64_t k1_blocks; // d / 16
  int64_t k2_blocks; // ffn_pad / 16
  void *w1;          // packed first weight (bf16) or a copy (fp32)
  void *w2;          // packed second weight (bf16) or a copy (fp32)
  void *hidden;      // [max_tokens x ffn_pad] bf16, or [max_tokens x F] fp32
  float *splitk;     // split-K partial sums (stream path)
  int *counters;     // split-K arrival counters, zero between calls
  int64_t splitk_floats;
  int64_t n_counters;
  void *alloc_base;  // single device allocation holding everything above
  int64_t alloc_bytes;
  hipEvent_t events[8];
  int n_events;
};

struct Sizes {
  int64_t ffn_pad, n1, n2, w1_bytes, w2_bytes, hidden_bytes, splitk_floats, n_counters;
};

// Sizes of the handle's buffers for a validated descriptor.
Sizes compute_sizes(const tpm_desc &d);

// Stream-path launch shape for a GEMM with `units` column units and `k_blocks` k
// blocks at M tokens.
StreamCfg stream_config(int64_t M, int64_t units, int64_t k_blocks);

// ---- launchers (all asynchronous on `s`) ----
hipError_t launch_pack_bf16(const void *src, int64_t ld, int64_t K, int64_t ncols_src,
                            bool pairs, int64_t F, int64_t n_cb, int64_t k_blocks, void *dst,
                            hipStream_t s);

hipError_t launch_stream_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t k_blocks,
                              const void *W, const StreamCfg &cfg, void *out, int64_t ldo,
                              int64_t n_store, float *splitk, int *counters, hipStream_t s);

hipError_t launch_tiled_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t K,
                             const void *W, int64_t n_packed, void *out, int64_t ldo,
                             int64_t n_store, hipStream_t s);

hipError_t launch_f32_gemm(int epi, const float *A, int64_t lda, int64_t M, int64_t K,
                           const float *B, int64_t ldb, int64_t N, int64_t up_offset, void *out,
                           int64_t ldo, hipStream_t s);

hipError_t launch_reduce(const void *const *parts, int k, int64_t numel, int in_dtype, void *out,
                         int out_dtype, hipStream_t s);

}  // namespace tpm
