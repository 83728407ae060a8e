// LDS-tiled bf16 matrix-core GEMM for large token counts (prefill).
//
// At prefill sizes each weight element meets thousands of tokens, so the
// projections are compute-bound (page "7.4 推理侧并行", section 7.4.1: prefill is a
// large matrix multiply).  This kernel keeps the matrix cores fed from LDS:
//
//  * Block tile 256 x 256 (tokens x columns), K staged 64 at a time, four waves
//    (one per SIMD), each owning a 128 x 128 sub-tile = 4 x 4 MFMA 32x32x16 tiles
//    with fp32 accumulators (256 per lane).
//  * Two LDS stages of 64 KiB (A and B, 32 KiB each): the global loads of stage k+1
//    are issued before the MFMAs of stage k and written to LDS after them, one
//    barrier per stage.
//  * Both operands are stored in LDS in fragment order (tpm_internal.h), so each
//    wave reads one operand with one conflict-free 1 KiB ds_read_b128 (16 B per
//    lane, lane-contiguous).  The weight and the packed hidden buffer arrive from
//    HBM already in that order; row-major token rows are scattered into it on the
//    way to LDS.
//  * Work tiles are renumbered so that consecutive tiles land on the same XCD
//    (workgroup b runs on XCD b % 8), and grouped four tile rows at a time, so
//    tiles that share operands share that XCD's L2.
//  * The epilogue is fused: SiLU(gate) * up (each 32-column block holds 16 gate
//    and the 16 matching up columns; lane c meets lane c + 16 by a cross-lane
//    exchange), tanh or identity, staged through LDS and written as bf16 in the
//    packed hidden order; or the partial store.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

constexpr int kTiledThreads = 256;
constexpr int kStageChunks = 8 * 4 * 64;  // 16-byte chunks per operand per stage (32 KiB)
constexpr int kGroupRows = 4;             // tile rows per launch-order group

template <int EPI>
__global__ void __launch_bounds__(kTiledThreads, 1)
k_tiled(const uint16_t *__restrict__ A, int64_t lda, int M, int k_tiles,
        const u32x4_t *__restrict__ W, int k_blocks, int ntm, int ntn,
        void *__restrict__ out, int64_t ldo, int n_store, int ks_out) {
  constexpr bool FIRST = EPI == EPI_SILU_GATE || EPI == EPI_TANH || EPI == EPI_IDENTITY;
  __shared__ u32x4_t lds[2][2][kStageChunks];  // [stage][0 = tokens, 1 = weight]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Tile renumbering: XCD-contiguous, then grouped by kGroupRows tile rows.
  const int nt = ntm * ntn;
  int t = blockIdx.x;
  if ((nt & 7) == 0) t = (t & 7) * (nt >> 3) + (t >> 3);
  const int per_group = kGroupRows * ntn;
  const int first_m = (t / per_group) * kGroupRows;
  const int gm = min(ntm - first_m, kGroupRows);
  const int tm = first_m + (t % per_group) % gm;
  const int tn = (t % per_group) / gm;

  // Global -> LDS mapping.  Row-major tokens (first product): chunk c (8 bf16,
  // indices 8c..8c+7 of the 64-wide stage) of row r goes to fragment (row block
  // r/32, k-step 2(c/4) + c%2), lane 32((c/2)%2) + r%32.  Packed hidden rows
  // (second product) and the weight: already in fragment order.
  const int a_r = tid >> 3;  // 0..31, row within a 32-row block
  const int a_c = tid & 7;   // 16-byte chunk within the 64-wide k stage
  const u32x4_t *a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (FIRST) {
      int row = tm * kTileM + i * 32 + a_r;
      row = row < M ? row : M - 1;  // rows >= M repeat the last row; never stored as output
      a_src[i] = reinterpret_cast<const u32x4_t *>(A + static_cast<int64_t>(row) * lda) + a_c;
    } else {
      a_src[i] = reinterpret_cast<const u32x4_t *>(A) +
                 ((static_cast<int64_t>(tm) * 8 + i) * k_blocks + (tid >> 6)) * 64 + lane;
    }
  }
  const int a_dst = FIRST ? (2 * (a_c >> 2) + (a_c & 1)) * 64 + ((a_c >> 1) & 1) * 32 + a_r : tid;
  const u32x4_t *b_src = W + (static_cast<int64_t>(tn) * 8 * k_blocks + (tid >> 6)) * 64 + lane;
  // weight chunk for (column block j, stage kt) = b_src + (j * k_blocks + 4 * kt) * 64

  u32x4_t ra[8], rb[8];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (FIRST) ra[i] = a_src[i][kt * 8];
      else ra[i] = a_src[i][static_cast<int64_t>(4 * kt) * 64];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rb[j] = b_src[(static_cast<int64_t>(j) * k_blocks + 4 * kt) * 64];
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) lds[st][0][i * 256 + a_dst] = ra[i];  // FIRST: i*4*64 + slot
#pragma unroll
    for (int j = 0; j < 8; ++j) lds[st][1][j * 256 + tid] = rb[j];
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](int st) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds[st][0][((wm * 4 + i) * 4 + kb) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = lds[st][1][((wn * 4 + j) * 4 + kb) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16(fa[i], fb[j], acc[i][j]);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < k_tiles; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < k_tiles;
    if (more) gload(kt + 1);
    compute(st);
    if (more) lstore(st ^ 1);
    __syncthreads();
  }

  // Epilogue.
  if constexpr (FIRST) {
    // h of the wave's 128 rows, 64 features per pass, staged through LDS (free
    // after the last barrier of the main loop), then written as 16-byte chunks
    // of the packed hidden buffer.
    constexpr int JW = (EPI == EPI_SILU_GATE) ? 16 : 32;  // features per column block
    constexpr int BPP = 64 / JW;                          // column blocks per pass
    constexpr int HS = 64 + 8;                            // LDS row stride (bf16)
    uint16_t *hs = reinterpret_cast<uint16_t *>(&lds[0][0][0]) + wave * (128 * HS);
#pragma unroll
    for (int pass = 0; pass < 4 / BPP; ++pass) {
#pragma unroll
      for (int jj = 0; jj < BPP; ++jj) {
        const int j = pass * BPP + jj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int R = i * 32 + mfma32_row(r, lane);
            const int c = lane & 31;
            const float v = acc[i][j][r];
            if constexpr (EPI == EPI_SILU_GATE) {
              const float u = __shfl_xor(v, 16);
              if (c < 16) hs[R * HS + jj * 16 + c] = f32_to_bf16(silu_f(v) * u);
            } else {
              hs[R * HS + jj * 32 + c] = f32_to_bf16(act_f<EPI>(v));
            }
          }
        }
      }
      __syncthreads();
      const int f0 = (tn * 8 + wn * 4 + pass * BPP) * JW;  // first feature of this pass
#pragma unroll
      for (int q = lane; q < 128 * 8; q += 64) {
        const int R = q & 127, qc = q >> 7;
        const int jf = f0 + 8 * qc;
        const int s = 2 * (jf >> 5) + ((jf >> 3) & 1);
        const int row = tm * kTileM + wm * 128 + R;
        const int ln = 32 * ((jf >> 4) & 1) + (row & 31);
        const int64_t chunk = (static_cast<int64_t>(row >> 5) * ks_out + s) * 64 + ln;
        static_cast<u32x4_t *>(out)[chunk] = *reinterpret_cast<const u32x4_t *>(&hs[R * HS + 8 * qc]);
      }
      if (pass + 1 < 4 / BPP) __syncthreads();
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tm * kTileM + (wm * 4 + i) * 32 + mfma32_row(r, lane);
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = (tn * 8 + wn * 4 + j) * 32 + (lane & 31);
          const int64_t o = static_cast<int64_t>(row) * ldo + col;
          if constexpr (EPI == EPI_OUT_F32) {
            if (col < n_store) static_cast<float *>(out)[o] = acc[i][j][r];
          } else {
            if (col < n_store) static_cast<uint16_t *>(out)[o] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  }
}

template <int EPI>
static hipError_t launch_tiled_one(const void *A, int64_t lda, int64_t M, int64_t K, const void *W,
                                   int64_t n_packed, void *out, int64_t ldo, int64_t n_store,
                                   int64_t ks_out, hipStream_t s, const Timing &t) {
  const int ntm = static_cast<int>((M + kTileM - 1) / kTileM);
  const int ntn = static_cast<int>(n_packed / kTileN);
  hipExtLaunchKernelGGL((k_tiled<EPI>), dim3(ntm * ntn), dim3(kTiledThreads), 0, s, t.start, t.stop, 0,
                     static_cast<const uint16_t *>(A), lda, static_cast<int>(M),
                     static_cast<int>(K / kTileK), static_cast<const u32x4_t *>(W),
                     static_cast<int>(K / kFragK), ntm, ntn, out, ldo, static_cast<int>(n_store),
                     static_cast<int>(ks_out));
  return hipGetLastError();
}

hipError_t launch_tiled_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t K,
                             const void *W, int64_t n_packed, void *out, int64_t ldo,
                             int64_t n_store, int64_t ks_out, hipStream_t s, const Timing &t) {
  switch (epi) {
    case EPI_SILU_GATE:
      return launch_tiled_one<EPI_SILU_GATE>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, s, t);
    case EPI_TANH:
      return launch_tiled_one<EPI_TANH>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, s, t);
    case EPI_IDENTITY:
      return launch_tiled_one<EPI_IDENTITY>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, s, t);
    case EPI_OUT_F32:
      return launch_tiled_one<EPI_OUT_F32>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, s, t);
    case EPI_OUT_BF16:
      return launch_tiled_one<EPI_OUT_BF16>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, s, t);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tpm
