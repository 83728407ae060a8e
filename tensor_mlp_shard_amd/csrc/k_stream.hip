// Weight-streaming projection for small token counts (decode).
//
// At decode sizes the projection is a skinny product: a few tokens against a
// weight that is read once, so the kernel is bound by HBM bandwidth, not by
// arithmetic (page "7.4 推理侧并行", section 7.4.1: decode steps read all weights
// for little compute; page "LLM 推理并行化", section 一: decode is memory-bound).
//
// Design (gfx950):
//  * The weight is pre-packed into 32x32x16 MFMA operand fragments, so every wave
//    load is one 1 KiB fully coalesced 16-byte-per-lane read and is fed straight to
//    the matrix core without touching LDS.
//  * The tokens (<= 32 per MFMA tile) are the MFMA's A operand; they are small and
//    re-read from L2 by every workgroup.
//  * A workgroup owns one column unit (32 output columns, or a matching gate+up pair
//    of 32 hidden features for SiLU-gate) and a slice of K; its waves split that
//    slice again and their accumulators are summed in LDS in a fixed order.
//  * When more workgroups are needed to keep HBM busy than there are column units,
//    several workgroups share one unit along K (split-K).  Each writes its fp32 sum
//    to scratch and bumps a counter; the last to arrive adds all slices in slice
//    order, applies the epilogue and resets the counter.  Summation order never
//    depends on arrival order, so results are bitwise reproducible.
//  * The epilogue (SiLU(gate)*up, tanh, or the partial store) is fused: the
//    first projection never writes pre-activations to memory.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

constexpr int kStreamWaves = 4;   // waves per workgroup
constexpr int kStreamUnroll = 4;  // k-steps per software-pipelined load group

template <int EPI, int MT>
__global__ void __launch_bounds__(kStreamWaves * 64)
k_stream(const uint16_t *__restrict__ A, int64_t lda, int M, int k_blocks,
         const u32x4_t *__restrict__ W, void *__restrict__ out, int64_t ldo, int n_store,
         float *__restrict__ splitk, int *__restrict__ counters, int ksplit) {
  constexpr int NCB = (EPI == EPI_SILU_GATE) ? 2 : 1;  // 32-column blocks per unit
  constexpr int NW = kStreamWaves;
  constexpr int U = kStreamUnroll;
  constexpr int NREG = MT * NCB * 16;   // accumulator registers per lane
  constexpr int UNIT_FLOATS = NREG * 64;

  __shared__ float red[NW][NREG][64];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x;
  const int ky = blockIdx.y;
  const int z = blockIdx.z;
  const int row0 = z * 32 * MT;

  // k-steps [sb, se) of this wave: the workgroup's slice of K, split over waves.
  const int wg_lo = static_cast<int>(static_cast<int64_t>(k_blocks) * ky / ksplit);
  const int wg_hi = static_cast<int>(static_cast<int64_t>(k_blocks) * (ky + 1) / ksplit);
  const int len = wg_hi - wg_lo;
  const int sb = wg_lo + len * wave / NW;
  const int se = wg_lo + len * (wave + 1) / NW;

  const u32x4_t *wp[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c)
    wp[c] = W + (static_cast<int64_t>(unit * NCB + c) * k_blocks) * 64 + lane;
  // Token rows beyond M read a valid row instead; MFMA rows are independent and
  // those rows are never stored.
  const u32x4_t *xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int row = row0 + mt * 32 + (lane & 31);
    row = row < M ? row : M - 1;
    xp[mt] = reinterpret_cast<const u32x4_t *>(A + static_cast<int64_t>(row) * lda + 8 * (lane >> 5));
  }

  f32x16_t acc[MT][NCB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][c][r] = 0.0f;

  u32x4_t b0[U][NCB], a0[U][MT], b1[U][NCB], a1[U][MT];
  auto load = [&](u32x4_t (&bb)[U][NCB], u32x4_t (&aa)[U][MT], int s) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) bb[i][c] = wp[c][static_cast<int64_t>(s + i) * 64];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) aa[i][mt] = xp[mt][(s + i) * 2];
    }
  };
  auto compute = [&](const u32x4_t (&bb)[U][NCB], const u32x4_t (&aa)[U][MT]) {
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < NCB; ++c) acc[mt][c] = mfma_32x32x16(aa[i][mt], bb[i][c], acc[mt][c]);
  };

  // Full groups of U k-steps, double-buffered in registers: the loads of group g+1
  // are in flight while group g is multiplied.
  int s = sb;
  const int n_full = (se - sb) / U;
  if (n_full > 0) {
    int g = 0;
    load(b0, a0, s);
    while (true) {
      if (g + 1 < n_full) load(b1, a1, s + U);
      compute(b0, a0);
      s += U;
      if (++g >= n_full) break;
      if (g + 1 < n_full) load(b0, a0, s + U);
      compute(b1, a1);
      s += U;
      if (++g >= n_full) break;
    }
  }
  for (; s < se; ++s) {  // remaining k-steps, one at a time
    u32x4_t bb[NCB], aa[MT];
#pragma unroll
    for (int c = 0; c < NCB; ++c) bb[c] = wp[c][static_cast<int64_t>(s) * 64];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) aa[mt] = xp[mt][s * 2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[mt][c] = mfma_32x32x16(aa[mt], bb[c], acc[mt][c]);
  }

  // Sum the waves' accumulators in LDS, wave 0 first.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][(mt * NCB + c) * 16 + r][lane] = acc[mt][c][r];
  __syncthreads();

  auto store = [&](const float (&v)[NCB], int mt, int r, int ln) {
    const int row = row0 + mt * 32 + mfma32_row(r, ln);
    const int col = unit * 32 + (ln & 31);
    if (row >= M) return;
    const int64_t o = static_cast<int64_t>(row) * ldo + col;
    if constexpr (EPI == EPI_SILU_GATE) {
      static_cast<uint16_t *>(out)[o] = f32_to_bf16(silu_f(v[0]) * v[NCB - 1]);
    } else if constexpr (EPI == EPI_TANH || EPI == EPI_IDENTITY) {
      static_cast<uint16_t *>(out)[o] = f32_to_bf16(act_f<EPI>(v[0]));
    } else if constexpr (EPI == EPI_OUT_F32) {
      if (col < n_store) static_cast<float *>(out)[o] = v[0];
    } else {
      if (col < n_store) static_cast<uint16_t *>(out)[o] = f32_to_bf16(v[0]);
    }
  };

  constexpr int OUTS = MT * 16 * 64;  // outputs per unit (a gate/up pair counts once)
  float *ws = splitk + (static_cast<int64_t>(z) * gridDim.x + unit) * ksplit * UNIT_FLOATS;
  for (int e = threadIdx.x; e < OUTS; e += NW * 64) {
    const int mt = e >> 10, r = (e >> 6) & 15, ln = e & 63;
    float v[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int q = (mt * NCB + c) * 16 + r;
      float a = red[0][q][ln];
#pragma unroll
      for (int w = 1; w < NW; ++w) a += red[w][q][ln];
      v[c] = a;
    }
    if (ksplit == 1) {
      store(v, mt, r, ln);
    } else {
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        ws[static_cast<int64_t>(ky) * UNIT_FLOATS + ((mt * NCB + c) * 16 + r) * 64 + ln] = v[c];
    }
  }
  if (ksplit == 1) return;

  // Split-K: the last workgroup of this unit to arrive finishes it.
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int old = atomicAdd(&counters[z * gridDim.x + unit], 1);
    s_last = (old == ksplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = threadIdx.x; e < OUTS; e += NW * 64) {
    const int mt = e >> 10, r = (e >> 6) & 15, ln = e & 63;
    float v[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int q = ((mt * NCB + c) * 16 + r) * 64 + ln;
      float a = ws[q];
      for (int p = 1; p < ksplit; ++p) a += ws[static_cast<int64_t>(p) * UNIT_FLOATS + q];
      v[c] = a;
    }
    store(v, mt, r, ln);
  }
  if (threadIdx.x == 0) atomicExch(&counters[z * gridDim.x + unit], 0);
}

StreamCfg stream_config(int64_t M, int64_t units, int64_t k_blocks) {
  StreamCfg c;
  c.mt = M <= 32 ? 1 : 2;
  c.units = static_cast<int>(units);
  c.zgroups = static_cast<int>((M + 32 * c.mt - 1) / (32 * c.mt));
  c.ksplit = 1;
  if (c.zgroups == 1) {
    const int64_t target_wgs = 512;
    int64_t ks = (target_wgs + units - 1) / units;
    const int64_t max_split = k_blocks / (kStreamWaves * 8);  // >= 8 k-steps per wave
    if (ks > max_split) ks = max_split;
    if (ks > 16) ks = 16;
    if (ks < 1) ks = 1;
    c.ksplit = static_cast<int>(ks);
  }
  return c;
}

template <int EPI, int MT>
static hipError_t launch_one(const void *A, int64_t lda, int64_t M, int64_t k_blocks,
                             const void *W, const StreamCfg &cfg, void *out, int64_t ldo,
                             int64_t n_store, float *splitk, int *counters, hipStream_t s) {
  dim3 grid(cfg.units, cfg.ksplit, cfg.zgroups);
  hipLaunchKernelGGL((k_stream<EPI, MT>), grid, dim3(kStreamWaves * 64), 0, s,
                     static_cast<const uint16_t *>(A), lda, static_cast<int>(M),
                     static_cast<int>(k_blocks), static_cast<const u32x4_t *>(W), out, ldo,
                     static_cast<int>(n_store), splitk, counters, cfg.ksplit);
  return hipGetLastError();
}

hipError_t launch_stream_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t k_blocks,
                              const void *W, const StreamCfg &cfg, void *out, int64_t ldo,
                              int64_t n_store, float *splitk, int *counters, hipStream_t s) {
#define TPM_STREAM_CASE(E)                                                                       \
  case E:                                                                                        \
    return cfg.mt == 1 ? launch_one<E, 1>(A, lda, M, k_blocks, W, cfg, out, ldo, n_store,        \
                                          splitk, counters, s)                                   \
                       : launch_one<E, 2>(A, lda, M, k_blocks, W, cfg, out, ldo, n_store,        \
                                          splitk, counters, s);
  switch (epi) {
    TPM_STREAM_CASE(EPI_SILU_GATE)
    TPM_STREAM_CASE(EPI_TANH)
    TPM_STREAM_CASE(EPI_IDENTITY)
    TPM_STREAM_CASE(EPI_OUT_F32)
    TPM_STREAM_CASE(EPI_OUT_BF16)
    default:
      return hipErrorInvalidValue;
  }
#undef TPM_STREAM_CASE
}

}  // namespace tpm
