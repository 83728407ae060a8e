// Grouped expert MLP at small token counts per expert: both projections by weight
// streaming.
//
// Page "大模型推理系统揭秘（07）Multi-GPU", MoE section: the tokens routed to the
// experts of one GPU are laid out contiguously by expert and all experts' products
// run as one batched job.  At decode-like loads (a hundred or so tokens per
// expert) every weight element meets few tokens, so the product is bound by
// streaming the experts' weights from HBM, as in the dense decode kernel
// (k_stream.hip), not by the matrix cores.
//
//  * A workgroup owns 8 column blocks (256 columns) of one expert's packed weight
//    (either projection) for one tile of up to 128 of that expert's tokens; each
//    of its 8 waves owns one 32-column block over the whole contraction and
//    streams it straight into registers (1 KiB non-temporal loads, the next two
//    stages in flight).  No two waves read the same weight fragment, so the
//    weights never pass through LDS.
//  * The tile's tokens are the operand all 8 waves share, staged per stage of 64
//    contraction indices in a 3-buffer LDS ring, one barrier per stage, and
//    every wave reads its MFMA fragments from there.  First projection: each wave
//    loads 16 token rows of X as 128-byte row segments (row stride padded against
//    bank conflicts in LDS).  Second projection: the packed hidden buffer is already
//    in fragment order, so the stage's 16 fragments (4 row blocks x 4 k-steps) are
//    copied as they are, two per wave, and read back lane-contiguously.  Token bytes
//    per weight byte: 128 / 256.
//  * Tiles are mapped to experts through the token counts in device memory: tile
//    row t counts through the experts' 128-row tiles in expert order; a workgroup
//    past the last tile exits.  Hidden rows of an expert start on a 256-row
//    boundary, the layout the tiled kernel uses.
//  * First projection: the epilogue applies SiLU(gate) * up (lane c meets lane
//    c + 16 of the same block), tanh or identity per wave and writes the packed
//    hidden buffer.  Token rows of a partly filled 32-row block past the expert's
//    tokens repeat its last token (finite values, never part of an output row);
//    blocks wholly past them are neither loaded nor written.  Second projection:
//    the rows of the expert's tokens are stored row-major (fp32 or bf16); hidden
//    blocks wholly past them are not loaded.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

namespace {

constexpr int kGsRows = static_cast<int>(kGroupStreamRows);  // token rows per tile
constexpr int kGsWaves = 8;     // waves per workgroup = column blocks per tile
constexpr int kGsXStride = 72;  // staged token row stride in bf16 (64 + 8 padding)
constexpr int kGsDepth = 3;     // stages held at once: one being multiplied, the rest in flight

// A: X row-major [T x lda] (first projection) or the packed hidden buffer with ks
// k-steps (second); out: the packed hidden buffer with ks_out k-steps (first) or
// row-major [T x ldo], columns < n_store (second).
template <int EPI>
__global__ void __launch_bounds__(kGsWaves * 64)
k_group_stream(const uint16_t *__restrict__ A, int64_t lda, int T, int ks,
               const u32x4_t *__restrict__ W, int64_t w_stride, int n_cb,
               const int *__restrict__ counts, int n_groups, void *__restrict__ out,
               int64_t ldo, int n_store, int ks_out) {
  constexpr bool FIRST = writes_hidden(EPI);
  // token stages: row segments (first projection) or fragments (second)
  constexpr int D = kGsDepth;
  constexpr int XBYTES = FIRST ? D * kGsRows * kGsXStride * 2 : D * 16 * 1024;
  __shared__ __attribute__((aligned(16))) char smem[XBYTES];
  uint16_t (*xs)[kGsRows][kGsXStride] = reinterpret_cast<uint16_t (*)[kGsRows][kGsXStride]>(smem);
  u32x4_t (*fs)[16][64] = reinterpret_cast<u32x4_t (*)[16][64]>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Expert and row tile of this workgroup (uniform over the workgroup).
  int rt = blockIdx.y, off = 0, hoff = 0, g = 0, n = 0;
  for (; g < n_groups; ++g) {
    n = min(max(counts[g], 0), T - off);
    const int tiles = (n + kGsRows - 1) / kGsRows;
    if (rt < tiles) break;
    rt -= tiles;
    off += n;
    hoff += (n + kTileM - 1) / kTileM * kTileM;
  }
  if (g == n_groups) return;
  const int row0 = off + rt * kGsRows;                 // first token row of the tile
  const int rows = min(kGsRows, off + n - row0);       // tokens in the tile (>= 1)
  const int hrow0 = hoff + rt * kGsRows;               // first hidden row of the tile
  const int nvb = (rows + 31) >> 5;                    // 32-row blocks holding tokens
  const int cb = blockIdx.x * kGsWaves + wave;         // this wave's column block

  const u32x4_t *wp = W + static_cast<int64_t>(g) * w_stride + static_cast<int64_t>(cb) * 64 + lane;
  // What this wave stages per stage.  First projection: 16 token rows, two loads of
  // 8 rows x 128 bytes.  Second: fragments 2 w and 2 w + 1 of the stage (row block
  // f / 4, k-step f % 4), skipped for row blocks holding no tokens.
  const uint16_t *xr[2];
  int srow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if constexpr (FIRST) {
      const int r = 16 * wave + 8 * q + (lane >> 3);
      srow[q] = r;
      xr[q] = A + static_cast<int64_t>(row0 + min(r, rows - 1)) * lda + 8 * (lane & 7);
    } else {
      const int f = 2 * wave + q;
      srow[q] = f;
      xr[q] = reinterpret_cast<const uint16_t *>(
          reinterpret_cast<const u32x4_t *>(A) +
          ((static_cast<int64_t>(hrow0 >> 5) + (f >> 2)) * ks + (f & 3)) * 64 + lane);
    }
  }
  // Both stage rows of 32-row block wave / 2: skipped for blocks holding no tokens.
  const bool stage_own = (wave >> 1) < nvb;
  const int nst = ks / 4;  // stages of 4 k-steps

  f32x16_t acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;

  // Loads of stage st (clamped to the last stage: valid addresses, never used).
  u32x4_t wb[D][4], xb[D][2];
  auto load = [&](u32x4_t (&wb)[4], u32x4_t (&xb)[2], int st) {
    const int s = min(st, nst - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)  // streamed once: non-temporal
      wb[i] = __builtin_nontemporal_load(&wp[static_cast<int64_t>(4 * s + i) * n_cb * 64]);
    if (!stage_own) return;
    if constexpr (FIRST) {
#pragma unroll
      for (int q = 0; q < 2; ++q) xb[q] = *reinterpret_cast<const u32x4_t *>(xr[q] + 64 * s);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)  // 4 k-steps of 64 chunks per stage
        xb[q] = reinterpret_cast<const u32x4_t *>(xr[q])[static_cast<int64_t>(4 * s) * 64];
    }
  };
  auto stage_tokens = [&](const u32x4_t (&xb)[2], int buf) {
    if (!stage_own) return;
    if constexpr (FIRST) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<u32x4_t *>(&xs[buf][srow[q]][8 * (lane & 7)]) = xb[q];
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) fs[buf][srow[q]][lane] = xb[q];
    }
  };
  // Products of stage st: 4 k-steps x 4 row blocks.  The fragment of k-step ksi for
  // row 32 m + l % 32 holds contraction indices 32 (ksi / 2) + 16 (l / 32) +
  // 8 (ksi % 2) .. + 7 of the stage (fragment order).  Row blocks holding no tokens
  // are multiplied too, from whatever their LDS rows hold, so that no branch
  // separates a fragment read from its product; a row of a product depends only on
  // the same row of the token operand, and those rows are never stored.
  auto compute = [&](const u32x4_t (&wb)[4], int buf, int st) {
    const bool valid = st < nst;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ksi = 0; ksi < 4; ++ksi) {
      u32x4_t a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (FIRST)
          a[m] = *reinterpret_cast<const u32x4_t *>(
              &xs[buf][32 * m + (lane & 31)][32 * (ksi >> 1) + 16 * (lane >> 5) + 8 * (ksi & 1)]);
        else
          a[m] = fs[buf][4 * m + ksi][lane];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = mfma_32x32x16(valid ? a[m] : zero, wb[ksi], acc[m]);
    }
  };

  // Stage st's tokens sit in LDS buffer st % D (written before the barrier that
  // precedes its products) and its weights in register set st % D; stages st + 1
  // .. st + D - 1 are in flight.  A buffer is rewritten only after the barrier that
  // follows its last reads (D - 1 barriers later).
  load(wb[0], xb[0], 0);
  stage_tokens(xb[0], 0);
#pragma unroll
  for (int j = 1; j < D; ++j) load(wb[j], xb[j], j);
  __syncthreads();
  for (int st = 0; st < nst; st += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      compute(wb[j], j, st + j);
      stage_tokens(xb[(j + 1) % D], (j + 1) % D);
      load(wb[j], xb[j], st + j + D);
      __syncthreads();
    }
  }

  if constexpr (!FIRST) {
    // Row-major output rows of the expert's tokens.
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= nvb) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = 32 * m + mfma32_row(r, lane);
        const int col = cb * 32 + (lane & 31);
        if (R < rows && col < n_store) {
          const int64_t o = static_cast<int64_t>(row0 + R) * ldo + col;
          if constexpr (stores_f32(EPI)) static_cast<float *>(out)[o] = acc[m][r];
          else static_cast<uint16_t *>(out)[o] = f32_to_bf16(acc[m][r]);
        }
      }
    }
  } else {
    // Epilogue per wave and row block: the activation into LDS as bf16, then the
    // packed hidden chunks (8 features of one row per 16 bytes).
    __shared__ __attribute__((aligned(16))) uint16_t hs[kGsWaves][32][40];  // h of one block per wave
    constexpr int JW = (EPI == EPI_SILU_GATE) ? 16 : 32;  // features of this column block
    const int j0 = cb * JW;
    uint16_t (*h)[40] = hs[wave];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= nvb) break;
      const int c = lane & 31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = mfma32_row(r, lane);
        const float v = acc[m][r];
        if constexpr (EPI == EPI_SILU_GATE) {
          const float up = __shfl_xor(v, 16);
          if (c < 16) h[R][c] = f32_to_bf16(silu_f(v) * up);
        } else {
          h[R][c] = f32_to_bf16(act_f<EPI>(v));
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
      for (int e = lane; e < 32 * (JW / 8); e += 64) {
        const int R = e & 31, q = e >> 5;
        const int j = j0 + 8 * q;
        const int s = 2 * (j >> 5) + ((j >> 3) & 1);
        const int ln = 32 * ((j >> 4) & 1) + R;
        const int hrow = hrow0 + 32 * m;  // the 32-row block of hidden rows
        static_cast<u32x4_t *>(out)[(static_cast<int64_t>(hrow >> 5) * ks_out + s) * 64 + ln] =
            *reinterpret_cast<const u32x4_t *>(&h[R][8 * q]);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    }
  }
}

}  // namespace

hipError_t launch_group_stream(int epi, const void *A, int64_t lda, int64_t T, int64_t K,
                               const void *W, int64_t w_stride, int64_t n_cb, const int *counts,
                               int n_groups, void *out, int64_t ldo, int64_t n_store,
                               int64_t ks_out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (K % 64 || n_cb % kGsWaves || n_groups < 1) return hipErrorInvalidValue;
  const int64_t tiles_y = (T + kGsRows - 1) / kGsRows + n_groups;  // >= the sum of the experts' tiles
  if (tiles_y > 65535 || n_cb / kGsWaves > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(n_cb / kGsWaves), static_cast<unsigned>(tiles_y));
  dim3 block(kGsWaves * 64);
  const uint16_t *a = static_cast<const uint16_t *>(A);
  const u32x4_t *w = static_cast<const u32x4_t *>(W);
  const int t = static_cast<int>(T), ks = static_cast<int>(K / kFragK), nc = static_cast<int>(n_cb);
  const int ns = static_cast<int>(n_store), ko = static_cast<int>(ks_out);
#define TPM_GS_LAUNCH(E)                                                                           \
  hipLaunchKernelGGL(k_group_stream<E>, grid, block, 0, s, a, lda, t, ks, w, w_stride, nc, counts, \
                     n_groups, out, ldo, ns, ko)
  switch (epi) {
    case EPI_SILU_GATE: TPM_GS_LAUNCH(EPI_SILU_GATE); break;
    case EPI_TANH: TPM_GS_LAUNCH(EPI_TANH); break;
    case EPI_IDENTITY: TPM_GS_LAUNCH(EPI_IDENTITY); break;
    case EPI_OUT_F32: TPM_GS_LAUNCH(EPI_OUT_F32); break;
    case EPI_OUT_BF16: TPM_GS_LAUNCH(EPI_OUT_BF16); break;
    default: return hipErrorInvalidValue;
  }
#undef TPM_GS_LAUNCH
  return hipGetLastError();
}

}  // namespace tpm
