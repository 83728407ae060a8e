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
  // A single projection Y = X W: row-major tokens in (as the first product),
  // row-major Y out (as the partial store)
  EPI_PROJ_F32 = 5,
  EPI_PROJ_BF16 = 6,
};

// Token operand of a product: row-major X (first product, single projections) or
// the packed hidden buffer (second product).
constexpr bool tokens_row_major(int epi) {
  return epi == EPI_SILU_GATE || epi == EPI_TANH || epi == EPI_IDENTITY || epi == EPI_PROJ_F32 ||
         epi == EPI_PROJ_BF16;
}
// Output: the packed hidden buffer (first product) or row-major rows.
constexpr bool writes_hidden(int epi) {
  return epi == EPI_SILU_GATE || epi == EPI_TANH || epi == EPI_IDENTITY;
}
// Row-major output stored as fp32 (else bf16).
constexpr bool stores_f32(int epi) { return epi == EPI_OUT_F32 || epi == EPI_PROJ_F32; }

// ---------------------------------------------------------------------------
// Operand layout on the matrix cores ("fragment order").
//
// Every product runs on v_mfma_f32_32x32x16_bf16: per k-step of 16, lane l of a
// wave supplies 8 bf16 of the A operand (row l % 32) and 8 bf16 of the B operand
// (column l % 32), for the 8 contraction indices selected by the lane half
// h = l / 32.  The contraction may take the indices of a k-step in any order as
// long as both operands agree, so the library fixes one order that makes row-
// major token loads wide: within each group of 32 contraction indices,
//
//   k-step s (0-based), lane half h, element i (0..7)  ->  index
//   kappa(s, h, i) = 32 * (s / 2) + 16 * h + 8 * (s % 2) + i.
//
// A lane thus reads the 16 consecutive indices 32*(s/2) + 16h .. +15 of its token
// row over the two k-steps of a pair, and the two lane halves together read 64
// contiguous bytes of the row.
//
// Packed weight W [K x N] (K = contraction, rows of the logical weight): 16-byte
// chunks at index ((s * NCB + cb) * 64 + lane), NCB = N_pad / 32 column blocks,
// each holding W[kappa(s, lane/32, i)][column(cb, lane % 32)], i = 0..7.  One
// 1 KiB wave load is one B operand.  The layout is k-step major: the fragments of
// one k-step for all column blocks are adjacent, so workgroups that stream
// different column blocks at the same pace read neighbouring memory at any moment
// (measured on MI355X: 10% more HBM bandwidth than block-major streams), and a
// tile's column blocks at one k-step form one contiguous run.  K is zero-padded to
// a multiple of 64 and the columns to a multiple of 256.
//
// SiLU-gate first weight: column block cb holds 16 gate columns then the 16 up
// columns of the same hidden features [16 cb, 16 cb + 16), so one 32x32 tile
// computes both branches of 16 features and the epilogue pairs lane c with lane
// c + 16.  tanh / identity first weight and the second weight: column block cb is
// columns [32 cb, 32 cb + 32).
//
// Packed hidden activations H [rows x F_pad] (the A operand of the second
// product): chunks at index ((mt * KS2 + s) * 64 + lane), KS2 = F_pad / 16, each
// holding H[32 mt + lane % 32][kappa(s, lane/32, i)], i = 0..7.  The first
// product writes H in this order, so the second reads it with 1 KiB contiguous
// wave loads.  Rows are padded to a multiple of 256 and every padded row holds
// finite values.
// ---------------------------------------------------------------------------
constexpr int kFragK = 16;            // k per MFMA step
constexpr int kFragN = 32;            // columns per fragment
constexpr int kTileM = 256;           // tiled (prefill) kernel: rows per block
constexpr int kTileN = 256;           // tiled kernel: columns per block
constexpr int kTileK = 64;            // tiled kernel: k per LDS stage
constexpr int kHiddenRowPad = 256;    // rows of the packed hidden buffer are padded to this
constexpr int kStreamMaxTokens = 64;  // AUTO: streaming kernels for M <= this
constexpr int kStreamMaxSlices = 16;  // streaming kernels: most contraction slices per block

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Shard {
  tpm_desc desc;
  int device;
  int64_t ffn_pad;    // F padded (bf16 path)
  int64_t n1;         // packed columns of the first weight
  int64_t n2;         // packed columns of the second weight (d padded to 256)
  int64_t ks1;        // k-steps of the first product (d / 16)
  int64_t ks2;        // k-steps of the second product (ffn_pad / 16)
  void *w1;           // packed first weight (bf16) or a copy (fp32)
  void *w2;           // packed second weight (bf16) or a copy (fp32)
  void *hidden;       // packed H (bf16 path) or [max_tokens x F] fp32
  float *scratch;     // streaming path: per-slice partial sums
  int *counters;      // arrival counters (streaming slices, tiled halves), zero between calls
  int64_t scratch_floats;  // room in scratch
  int64_t n_counters;      // room in counters
  int n_cu;           // compute units of the device
  int split_tiles;    // tiled path: split tiles the scratch holds
  void *alloc_base;   // single device allocation holding everything above
  int64_t alloc_bytes;
  hipEvent_t events[8];
  int n_events;
};

struct Sizes {
  int64_t ffn_pad, n1, n2, w1_bytes, w2_bytes, hidden_bytes, scratch_floats, n_counters;
  int64_t split_tiles;  // tiled path: room for this many split tiles in scratch / counters
};

// Launch shape of one streaming product: token tiles per workgroup (mt), column
// blocks per workgroup (c) and contraction slices (s).
struct StreamPlan {
  int mt, c, s;
  int atom = 0;  // s == 2 contraction halves added atomically into a zeroed fp32 output
};

// A clear of `n` fp32 outputs (a multiple of 4, 16-byte aligned) done as a side job
// by a launch, for the next launch on the stream to add into.
struct StreamZero {
  float *out = nullptr;
  int64_t n = 0;
};

// Waves per workgroup of the atomic-halves second product.
constexpr int kStreamAtomWaves = 4;

// The streaming shape the library uses for M tokens against n_cb column blocks
// and ks k-steps.  Contraction slices (s > 1) only come with one token group
// (M <= 64).
StreamPlan stream_plan(int64_t M, int64_t n_cb, int64_t ks);

// The shape of a second product (packed hidden tokens) with M tokens: stream_plan's,
// or, for an fp32 output that stream_plan does not slice, two column blocks per
// workgroup over two atomic contraction halves (the output must then be zeroed
// before the launch, e.g. by the first product's StreamZero).
StreamPlan stream_plan_out(int64_t M, int64_t n_cb, int64_t ks, bool out_f32);

// Workspace of the streaming contraction slices: sums parked by the slices
// (`floats` of room) and the per-unit arrival counters (`n_counters` of room,
// zero between calls).
struct StreamScratch {
  float *buf = nullptr;
  int *cnt = nullptr;
  int64_t floats = 0;
  int64_t n_counters = 0;
};

// Optional timing of one launch: the events ride on the kernel's own dispatch
// (start and end of its execution), so timing adds no work to the stream.
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Sizes of the handle's buffers for a validated descriptor.
Sizes compute_sizes(const tpm_desc &d);

// ---- launchers (all asynchronous on `s`) ----

// Repack a row-major bf16 weight into fragment order (see above).
//   pairs = true: SiLU-gate first weight with F gate then F up columns per row.
hipError_t launch_pack_bf16(const void *src, int64_t ld, int64_t K, int64_t ncols_src,
                            bool pairs, int64_t F, int64_t n_cb, int64_t ks, void *dst,
                            hipStream_t s);

// Decode-path products (any M; tuned for M <= 64).
//   First product (epi = SILU_GATE / TANH / IDENTITY): A = X row-major [M x lda],
//   out = packed H with ks_out k-steps.  Second product (epi = OUT_*): A = packed H
//   with ks k-steps, out = row-major partial [M x ldo], columns < n_store stored.
//   plan.s > 1 needs groups * n_cb * plan.s * plan.mt * 1024 floats of scratch and
//   groups * n_cb / plan.c zeroed counters (groups = token groups of 32 plan.mt
//   rows); a launch that would not fit `ws` is refused.
hipError_t launch_stream_gemm(int epi, const StreamPlan &plan, const void *A, int64_t lda,
                              int64_t M, int64_t ks, const void *W, int64_t n_cb, void *out,
                              int64_t ldo, int64_t n_store, int64_t ks_out,
                              const StreamScratch &ws, hipStream_t s,
                              const Timing &t = Timing(), const StreamZero &zero = StreamZero());

// Zero n ints (a plain kernel, so it may be captured in a graph).
hipError_t launch_zero_i32(int *p, int64_t n, hipStream_t s);

// Contraction split of the tiled products' last partial round: up to
// kTiledMaxSplit tiles, each run as two contraction halves whose fp32 sums meet
// in `buf` (2 * 256 * 256 floats per tile) through a zeroed arrival counter in
// `cnt` (one per tile, left at zero).  n_cu = compute units of the device.
// buf == nullptr turns the split off.
constexpr int kTiledMaxSplit = 128;
struct TiledSplit {
  void *buf = nullptr;
  int *cnt = nullptr;
  int n_cu = 0;
  int max_tiles = 0;  // capacity of buf and cnt, in tiles
};

// Tiles of a tiled product (tiles in total, on n_cu compute units, room for
// max_tiles) that run as two contraction halves.
int tiled_split_tiles(int64_t tiles, int n_cu, int max_tiles);

// Grouped tiled product: n_groups weights, packed back to back (w_stride 16-byte
// chunks apart), each applied to its own contiguous run of token rows whose
// lengths sit in device memory (counts[g]; the runs are taken in group order and
// clamped to the M rows there are).  Hidden rows of a group start on a 256-row
// boundary: the hidden buffer needs round_up(M, 256) + 256 n_groups rows.
// n_groups = 0: a single matrix.
struct TiledGroups {
  const int *counts = nullptr;
  int n_groups = 0;
  int64_t w_stride = 0;
};

// Prefill-path products, same operand and output conventions as above.
hipError_t launch_tiled_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t K,
                             const void *W, int64_t n_packed, void *out, int64_t ldo,
                             int64_t n_store, int64_t ks_out, const TiledSplit &sp, hipStream_t s,
                             const Timing &t = Timing(), const TiledGroups &grp = TiledGroups());

// Prefill-path products on the two-waves-per-SIMD GEMM (k_gemm.hip): same operand and
// output conventions as launch_tiled_gemm (no grouped mode); K a multiple of kGemmK.
constexpr int kGemmK = 32;  // contraction per LDS stage
hipError_t launch_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t K, const void *W,
                       int64_t n_packed, void *out, int64_t ldo, int64_t n_store, int64_t ks_out,
                       const TiledSplit &sp, hipStream_t s, const Timing &t = Timing());

// Either projection of the grouped expert MLP by weight streaming: tiles of up to
// kGroupStreamRows of one expert's tokens by 256 columns, each wave streaming one
// 32-column block of the expert's packed weight; same operands, counts and hidden
// layout as the grouped tiled product.  epi SILU_GATE, TANH or IDENTITY: A is X
// (row stride lda) and out the packed hidden buffer with ks_out k-steps.  epi
// OUT_F32 or OUT_BF16: A is the packed hidden buffer (K / 16 k-steps) and out the
// row-major output (row stride ldo, columns < n_store).  n_cb a multiple of 8, K of 64.
constexpr int64_t kGroupStreamRows = 128;
hipError_t launch_group_stream(int epi, const void *A, int64_t lda, int64_t T, int64_t K,
                               const void *W, int64_t w_stride, int64_t n_cb, const int *counts,
                               int n_groups, void *out, int64_t ldo, int64_t n_store,
                               int64_t ks_out, hipStream_t s);

hipError_t launch_f32_gemm(int epi, const float *A, int64_t lda, int64_t M, int64_t K,
                           const float *B, int64_t ldb, int64_t N, int64_t up_offset, void *out,
                           int64_t ldo, hipStream_t s, const Timing &t = Timing());

hipError_t launch_reduce(const void *const *parts, int k, int64_t numel, int in_dtype, void *out,
                         int out_dtype, hipStream_t s);

// Partials sum + residual add + RMSNorm, one row per workgroup (cols a multiple of
// 8, at most kNormMaxCols: 1024 threads x 4 chunks of 8 held in registers).
constexpr int64_t kNormMaxCols = 32768;
hipError_t launch_reduce_norm(const void *const *parts, int k, int64_t rows, int64_t cols,
                              int in_dtype, const void *res_in, void *res_out, int res_dtype,
                              const void *gamma, float eps, void *y, int out_dtype,
                              hipStream_t s);

// Merge of k attention partials (values [rows x dim], per-row maxima and sums of
// exponentials, fp32 statistics); dim a multiple of 8.  max_out / expsum_out may be
// null (both or neither).
hipError_t launch_attn_merge(const void *const *values, const float *const *maxima,
                             const float *const *expsums, int k, int64_t rows, int64_t dim,
                             int in_dtype, void *out, int out_dtype, float *max_out,
                             float *expsum_out, hipStream_t s);

// FP8 (E4M3) partials with one scale per row: quantize one partial, and the
// rank-order fp32 sum of k quantized partials.  cols a multiple of 16; the
// quantizer holds a row in registers (1024 threads x 2 chunks of 16).
constexpr int64_t kFp8MaxCols = 32768;
hipError_t launch_quant_fp8(const void *x, int64_t rows, int64_t cols, int in_dtype, void *q,
                            float *scale, hipStream_t s);
hipError_t launch_reduce_fp8(const void *const *q, const float *const *scales, int k, int64_t rows,
                             int64_t cols, void *out, int out_dtype, hipStream_t s);

}  // namespace tpm
