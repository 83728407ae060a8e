// Weight-streaming projections for small token counts (decode).
//
// At decode sizes each weight element meets a few tokens, so the products are
// bound by HBM bandwidth (page "7.4 推理侧并行", section 7.4.1: decode reads all
// weights for little compute; page "LLM 推理并行化", section 一: decode is
// memory-bound).  The kernel is built to keep HBM busy and to do nothing else:
//
//  * One workgroup owns one 32-column block of the packed weight over the whole
//    contraction, so no partial sums leave the workgroup: no split-K scratch, no
//    atomics, no cross-workgroup fences, bitwise reproducible results.  A shard
//    of width 3584 gives 224 workgroups for the gate/up product (16 SiLU-gate
//    features per block), about one per compute unit.  Shards too narrow to occupy
//    the compute units slice the contraction instead, and the last arriving slice
//    adds them in slice order (stream_plan; the hand-off is described at the kernel).
//  * Its waves split the contraction into contiguous runs of k-steps.  Each wave
//    streams its run of the column block with 1 KiB fully coalesced,
//    non-temporal loads that are fed straight to the matrix cores (the weight is
//    pre-packed in operand order, k-step major, so the workgroups' streams read
//    neighbouring memory), with two batches of loads in flight.  The load addresses of a batch
//    past the end of the run are clamped to the last k-step (an L2 hit) and the
//    matching products are multiplied by zero, so the loop has no branch around a
//    load and the compiler waits for exactly one batch at a time.
//  * The token operand is small and read from L2: row-major X for the first product,
//    staged per wave through LDS as whole 128-byte row segments (8 rows per wave
//    load) and read back as fragments; the packed hidden buffer (1 KiB contiguous
//    per wave load, straight into fragments) for the second.
//  * A few tokens (at most 16): only the 8 or 16 token rows that exist are loaded
//    per batch instead of the tile's 32, and fragment lanes of rows past M read
//    row M - 1 (products never stored); for the packed hidden operand those lanes
//    load row M - 1's piece, so a fragment load touches only existing rows' lines.
//    The token share of the per-CU load traffic drops 4x at M <= 8 (70B-class TP=8
//    shard: 35.1 -> 33.6 us at M = 8, 37.3 -> 34.5 us at M = 1).
//  * The second product with an fp32 output (stream_plan_out): two column blocks per
//    workgroup over half the contraction each, so a workgroup loads the hidden
//    operand of its half once for both blocks; the two halves are added into the
//    output, which the first product clears as a side job.  With exactly two
//    addends onto zero the result is the same in either arrival order.  4 waves
//    (8 would give each wave only 14 k-steps of the 3584-deep shard: 14.8 us); 70B
//    TP=8 decode shard: 13.0 -> 12.6 us.
//  * The waves' accumulators are summed in LDS in wave order, then the epilogue
//    runs: SiLU(gate) * up, tanh or identity, written as bf16 into the packed
//    hidden buffer, or the partial store.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

static_assert(kStreamMaxSlices <= 16, "the hand-off holds every slice's sums in registers");

// Launch shapes.  C column blocks per workgroup: every token fragment a wave loads
// feeds C products, so the token operand costs 1/C of the weight traffic through
// the vector caches.  D k-steps per load batch (two batches in flight per wave),
// chosen so each shape stays in registers.  Waves per workgroup (NW, a template
// parameter of the kernel): see stream_waves.
template <int MT, int C>
struct StreamShape {
  // k-steps per load batch: two pairs when the token operand is staged as 128-byte
  // row segments; one pair for the packed hidden operand, whose short contraction
  // (a few batches per wave) gains from the finer pipeline (measured: 7% on the
  // 3584-deep down projection).
  template <bool FIRST>
  static constexpr int depth = FIRST ? 4 : 2;
};


// Epilogue of one 32 x 32 output block whose fp32 sums sit in LDS `v` in MFMA
// accumulator order (v[r][lane] = D[mfma32_row(r, lane)][lane % 32]).
template <int EPI, int NT>
__device__ __forceinline__ void stream_epilogue(const float (*v)[64], uint16_t (*hb)[40], int tid,
                                                int tile, int cb, int M, void *out, int64_t ldo,
                                                int n_store, int ks_out) {
  if constexpr (writes_hidden(EPI)) {
    for (int e = tid; e < 1024; e += NT) {
      const int r = e >> 6, l = e & 63, c = l & 31;
      const int R = mfma32_row(r, l);
      if constexpr (EPI == EPI_SILU_GATE) {
        if (c < 16) hb[R][c] = f32_to_bf16(silu_f(v[r][l]) * v[r][l + 16]);
      } else {
        hb[R][c] = f32_to_bf16(act_f<EPI>(v[r][l]));
      }
    }
    __syncthreads();
    // Packed hidden buffer: 8 features of one row per 16-byte chunk.
    constexpr int JW = (EPI == EPI_SILU_GATE) ? 16 : 32;  // features of this column block
    const int j0 = cb * JW;
    for (int e = tid; e < 32 * (JW / 8); e += NT) {
      const int R = e & 31, q = e >> 5;
      const int j = j0 + 8 * q;
      const int s = 2 * (j >> 5) + ((j >> 3) & 1);
      const int ln = 32 * ((j >> 4) & 1) + R;
      const int64_t chunk = (static_cast<int64_t>(tile) * ks_out + s) * 64 + ln;
      static_cast<u32x4_t *>(out)[chunk] = *reinterpret_cast<const u32x4_t *>(&hb[R][8 * q]);
    }
  } else {
    for (int e = tid; e < 1024; e += NT) {
      const int r = e >> 6, l = e & 63;
      const int row = 32 * tile + mfma32_row(r, l);
      const int col = 32 * cb + (l & 31);
      if (row < M && col < n_store) {
        const int64_t o = static_cast<int64_t>(row) * ldo + col;
        if constexpr (stores_f32(EPI)) static_cast<float *>(out)[o] = v[r][l];
        else static_cast<uint16_t *>(out)[o] = f32_to_bf16(v[r][l]);
      }
    }
  }
}

// Grid: n_units * S * groups workgroups.  Workgroup (unit u, slice sl, group z)
// owns column blocks [C u, C u + C) for token tiles [MT z, MT z + MT) over the
// sl-th of S equal slices of the contraction; its waves split the slice again.
// With S > 1 each workgroup leaves its sums in `scratch` and bumps the unit's
// arrival counter; the last to arrive adds the S slices in slice order (so the
// result does not depend on arrival order), runs the epilogue and resets the
// counter to zero for the next call.  Nothing ever waits for another workgroup.
template <int EPI, int MT, int C, int NW, int TRQ, bool ATOM>
__global__ void __launch_bounds__(NW * 64)
k_stream(const uint16_t *__restrict__ A, int64_t lda, int M, int ks,
         const u32x4_t *__restrict__ W, int n_units, int S, void *__restrict__ out, int64_t ldo,
         int n_store, int ks_out, float *__restrict__ scratch, int *__restrict__ counters,
         float *__restrict__ zero_out, int64_t zero_n) {
  constexpr bool FIRST = tokens_row_major(EPI);  // row-major token operand
  constexpr int D = StreamShape<MT, C>::template depth<FIRST>;
  constexpr int PB = D / 2;  // k-step pairs per batch
  constexpr int NT = NW * 64;
  // Row-major tokens are staged per wave through LDS: a batch is 32 PB contiguous
  // contraction indices (64 PB bytes) of each token row, loaded 8 rows x 128 bytes
  // per wave instruction (whole cache lines), then read back as MFMA fragments.
  constexpr int XROW = 32 * PB + 8;  // staged row stride in bf16 (padded against bank conflicts)
  constexpr int XWAVE = MT * 32 * XROW;
  constexpr int XBYTES = FIRST ? NW * XWAVE * 2 : 0;
  constexpr int RBYTES = NW * 16 * 64 * 4;
  constexpr int SBYTES = XBYTES > RBYTES ? XBYTES : RBYTES;
  static_assert(!FIRST || PB == 2, "token staging assumes 128-byte row segments");
  // TRQ < 4 (at most 8 TRQ tokens, one token tile): only the first 8 TRQ rows of the
  // tile are loaded; fragment lanes of rows past M read row M - 1 (never stored).
  static_assert(TRQ == 4 || (MT == 1 && (TRQ == 1 || TRQ == 2)), "token row groups");
  static_assert(!ATOM || EPI == EPI_OUT_F32, "atomic slices add fp32 partials");

  __shared__ __attribute__((aligned(16))) char smem[SBYTES];  // token staging, then reduction
  __shared__ float vsum[16][64];
  __shared__ __attribute__((aligned(16))) uint16_t hb[32][40];  // h of one block, bf16
  __shared__ int s_last;
  float (*red)[16][64] = reinterpret_cast<float (*)[16][64]>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = blockIdx.x % n_units;
  const int sl = (blockIdx.x / n_units) % S;
  const int z = blockIdx.x / (n_units * S);
  const int mt0 = z * MT;  // first 32-row token tile of this workgroup

  // Side job of a first product whose second product adds its contraction halves
  // atomically: clear that product's fp32 output (16-byte stores, a contiguous share
  // per workgroup).  The next launch on the stream sees the zeros.
  if (zero_out) {
    const int64_t n4 = zero_n >> 2;
    const int64_t per = (n4 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = per * blockIdx.x, hi = min(lo + per, n4);
    const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = lo + tid; i < hi; i += NT) reinterpret_cast<f32x4_t *>(zero_out)[i] = z;
  }

  // Batches of this wave.  The contraction is cut into batches of PB k-step pairs
  // (ks is a multiple of 4, so the count is exact); slice sl takes a contiguous run
  // of batches and each wave a contiguous run of those, [wb_lo, wb_hi).  Loads for
  // batch indices past the run re-read its last batch (valid addresses) and their
  // products are multiplied by zero.
  const int nbat_all = (ks >> 1) / PB;
  const int b_lo = static_cast<int>(static_cast<int64_t>(nbat_all) * sl / S);
  const int b_hi = static_cast<int>(static_cast<int64_t>(nbat_all) * (sl + 1) / S);
  const int wb_lo = b_lo + (b_hi - b_lo) * wave / NW;
  const int wb_hi = b_lo + (b_hi - b_lo) * (wave + 1) / NW;
  const int nb = wb_hi - wb_lo;

  const int trow = TRQ < 4 ? min(lane & 31, M - 1) : (lane & 31);  // staged row a fragment lane reads

  // Weight fragments of block C u + c at k-step s: wp[(s * n_cb + c) * 64].
  const int n_cb = n_units * C;
  const u32x4_t *wp = W + static_cast<int64_t>(u) * C * 64 + lane;
  // Token operand.  FIRST: row-major X; lane l loads 16 bytes of row 8 j + l / 8 of
  // the batch's 128-byte segment, chunk l % 8.  Otherwise: packed H fragments.
  const u32x4_t *ap[MT];
  const uint16_t *xrow[MT * TRQ];
  if constexpr (FIRST) {
#pragma unroll
    for (int j = 0; j < MT * TRQ; ++j) {
      int row = 32 * mt0 + 8 * j + (lane >> 3);
      row = row < M ? row : M - 1;  // rows >= M repeat the last row; never stored as output
      xrow[j] = A + static_cast<int64_t>(row) * lda + 8 * (lane & 7);
    }
  } else {
    // TRQ < 4: lanes of rows past M load row M - 1's piece, so a fragment load
    // touches only the cache lines of the rows that exist
    const int alane = TRQ < 4 ? (lane & 32) + min(lane & 31, M - 1) : lane;
#pragma unroll
    for (int m = 0; m < MT; ++m)
      ap[m] = reinterpret_cast<const u32x4_t *>(A) + static_cast<int64_t>(mt0 + m) * ks * 64 + alane;
  }
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem) + wave * XWAVE;

  f32x16_t acc[MT][C];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][c][r] = 0.0f;

  {
    // One batch in registers: weight fragments and the token operand (FIRST: the
    // raw 16-byte pieces of the staged rows; otherwise fragments).
    constexpr int NA = FIRST ? MT * TRQ : D * MT;
    u32x4_t w0[D][C], a0[NA], w1[D][C], a1[NA];
    auto load = [&](u32x4_t (&wb)[D][C], u32x4_t (&ab)[NA], int b) {
      const int p0 = PB * min(wb_lo + b, wb_hi - 1);  // first pair of the batch
#pragma unroll
      for (int i = 0; i < D; ++i)
#pragma unroll
        for (int c = 0; c < C; ++c)  // streamed once: non-temporal
          wb[i][c] = __builtin_nontemporal_load(&wp[(static_cast<int64_t>(2 * p0 + i) * n_cb + c) * 64]);
      if constexpr (FIRST) {
#pragma unroll
        for (int j = 0; j < MT * TRQ; ++j)
          ab[j] = *reinterpret_cast<const u32x4_t *>(xrow[j] + 32 * p0);
      } else {
#pragma unroll
        for (int i = 0; i < D; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m) ab[i * MT + m] = ap[m][static_cast<int64_t>(2 * p0 + i) * 64];
      }
    };
    auto compute = [&](const u32x4_t (&wb)[D][C], const u32x4_t (&ab)[NA], int b) {
      u32x4_t frag[D][MT];
      if constexpr (FIRST) {
#pragma unroll
        for (int j = 0; j < MT * TRQ; ++j)
          *reinterpret_cast<u32x4_t *>(&xs[(8 * j + (lane >> 3)) * XROW + 8 * (lane & 7)]) = ab[j];
#pragma unroll
        for (int i = 0; i < D; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m)
            frag[i][m] = *reinterpret_cast<const u32x4_t *>(
                &xs[(32 * m + trow) * XROW + 32 * (i >> 1) + 16 * (lane >> 5) + 8 * (i & 1)]);
      } else {
#pragma unroll
        for (int i = 0; i < D; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m) frag[i][m] = ab[i * MT + m];
      }
      const bool valid = wb_lo + b < wb_hi;
#pragma unroll
      for (int i = 0; i < D; ++i) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4_t zero = {0u, 0u, 0u, 0u};
          const u32x4_t a = valid ? frag[i][m] : zero;
#pragma unroll
          for (int c = 0; c < C; ++c) acc[m][c] = mfma_32x32x16(a, wb[i][c], acc[m][c]);
        }
      }
    };
    if (nb > 0) load(w0, a0, 0);
    // The scheduling barriers keep each batch's loads ahead of the previous batch's
    // products, so the products wait only for their own batch.
    for (int b = 0; b < nb; b += 2) {
      load(w1, a1, b + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(w0, a0, b);
      __builtin_amdgcn_sched_barrier(0);
      load(w0, a0, b + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, a1, b + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();  // token staging area becomes the reduction buffer

  // Per output block: sum the waves' accumulators in LDS (wave order), then either
  // finish the block or park the sum in this slice's scratch slot.
  constexpr int BLK = MT * C;  // 32 x 32 output blocks of this workgroup
  const int64_t wg_slot = (static_cast<int64_t>(z) * n_units + u) * S;  // + sl
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      __syncthreads();  // red / vsum / hb free again
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[m][c][r];
      __syncthreads();
      for (int e = tid; e < 1024; e += NT) {
        float a = red[0][e >> 6][e & 63];
#pragma unroll
        for (int w = 1; w < NW; ++w) a += red[w][e >> 6][e & 63];
        if constexpr (ATOM) {
          // the two contraction halves meet in the zeroed output: 0 + a + b is the
          // same in either arrival order, so the sum is deterministic
          const int row = 32 * (mt0 + m) + mfma32_row(e >> 6, e & 63);
          const int col = 32 * (C * u + c) + (e & 31);
          if (row < M && col < n_store)
            __hip_atomic_fetch_add(static_cast<float *>(out) + static_cast<int64_t>(row) * ldo + col, a,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (S == 1)
          vsum[e >> 6][e & 63] = a;
        else  // write-through store: complete at the device coherence point when counted
          __hip_atomic_store(&scratch[((wg_slot + sl) * BLK + m * C + c) * 1024 + e], a,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (!ATOM && S == 1) {
        __syncthreads();
        stream_epilogue<EPI, NT>(vsum, hb, tid, mt0 + m, C * u + c, M, out, ldo, n_store, ks_out);
      }
    }
  }
  if (ATOM || S == 1) return;

  // Arrival.  Every thread waits until its write-through stores have completed,
  // then one thread counts the workgroup in.  The scratch traffic never touches a
  // non-coherent cache line, so no cache write-back or invalidation is needed
  // (those would also evict the weight stream of the other workgroups on the XCD).
  // The ordering rests on the code emitted for gfx950, not on the language memory
  // model (a relaxed counter orders nothing there): the parked sums are agent-scope
  // atomic stores (the sc1 bit: written through to the device coherence point), the
  // explicit wait below holds every wave until they are acknowledged there, the barrier
  // holds thread 0 until every wave has waited, and the last arriver reads the sums
  // with agent-scope atomic loads (sc1: at the coherence point, never from a stale line
  // of its own L2).  tests/test_handoff_asm.py checks these properties in the compiled
  // kernels.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[static_cast<int64_t>(z) * n_units + u], 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == S - 1);
  }
  __syncthreads();
  if (!s_last) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      __syncthreads();
      // Every slice's sums of this thread's elements are loaded before any is added,
      // so the hand-off costs one round trip to the coherence point, not one per
      // slice.  Coherent loads: read at the device coherence point, never from a
      // stale line.
      constexpr int EPT = 1024 / NT;
      float t[EPT][kStreamMaxSlices];
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        float *p = scratch + (wg_slot * BLK + m * C + c) * 1024 + tid + j * NT;
#pragma unroll
        for (int q = 0; q < kStreamMaxSlices; ++q)
          if (q < S)
            t[j][q] = __hip_atomic_load(p + static_cast<int64_t>(q) * BLK * 1024, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        float a = t[j][0];
#pragma unroll
        for (int q = 1; q < kStreamMaxSlices; ++q)  // slice order
          if (q < S) a += t[j][q];
        const int e = tid + j * NT;
        vsum[e >> 6][e & 63] = a;
      }
      __syncthreads();
      stream_epilogue<EPI, NT>(vsum, hb, tid, mt0 + m, C * u + c, M, out, ldo, n_store, ks_out);
    }
  }
  if (tid == 0)
    __hip_atomic_store(&counters[static_cast<int64_t>(z) * n_units + u], 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Waves per workgroup, measured at the 70B-class decode shapes.  A whole contraction
// of the row-major token product streams fastest with 4 (gate/up, one token tile,
// time against 4 waves: 16 waves +4%, 8 +2%, 2 +25%, deeper register pipelines of 3
// or 4 batches +3%; two token tiles: 8 waves up to +6%; the 1024-deep attention
// output shard: 8 waves +10%); its contraction slices with 8 (the 40-block QKV shard
// in 4 slices: 4 waves +10%, 16 +2%); the packed hidden product with 8 (16, whose
// waves then get only 14 k-steps each: +14%; 4: +6%).
constexpr int stream_waves(bool first, int S) { return first && S == 1 ? 4 : 8; }

template <int EPI, int MT, int C, int NW, int TRQ = 4, bool ATOM = false>
hipError_t launch_stream_nw(const void *A, int64_t lda, int64_t M, int64_t ks, const void *W,
                            int64_t n_units, int64_t blocks, int S, void *out, int64_t ldo,
                            int64_t n_store, int64_t ks_out, float *scratch, int *counters,
                            hipStream_t s, const Timing &t, const StreamZero &zero) {
  hipExtLaunchKernelGGL((k_stream<EPI, MT, C, NW, TRQ, ATOM>), dim3(static_cast<unsigned>(blocks)),
                        dim3(NW * 64), 0, s, t.start, t.stop, 0, static_cast<const uint16_t *>(A),
                        lda, static_cast<int>(M), static_cast<int>(ks),
                        static_cast<const u32x4_t *>(W), static_cast<int>(n_units), S, out, ldo,
                        static_cast<int>(n_store), static_cast<int>(ks_out), scratch, counters,
                        zero.out, zero.n);
  return hipGetLastError();
}

template <int EPI, int MT, int C, bool ATOM = false>
hipError_t launch_stream_cfg(const void *A, int64_t lda, int64_t M, int64_t ks, const void *W,
                             int64_t n_cb, int S, void *out, int64_t ldo, int64_t n_store,
                             int64_t ks_out, const StreamScratch &ws, hipStream_t s,
                             const Timing &t, const StreamZero &zero) {
  const int64_t groups = (M + 32 * MT - 1) / (32 * MT);
  const int64_t n_units = n_cb / C;
  const int64_t blocks = n_units * S * groups;
  if (n_cb % C || S < 1 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if constexpr (ATOM) {
    // atomic halves: exactly two slices (deterministic), no scratch
    if (S != 2) return hipErrorInvalidConfiguration;
    return launch_stream_nw<EPI, MT, C, kStreamAtomWaves, 4, true>(
        A, lda, M, ks, W, n_units, blocks, S, out, ldo, n_store, ks_out, nullptr, nullptr, s, t, zero);
  }
  // Slices park MT * C blocks of 1024 sums per workgroup and count in per (group, unit):
  // refuse a launch whose scratch or counters would not fit the caller's workspace.
  if (S > 1 && (!ws.buf || !ws.cnt || groups * n_units * S * MT * C * 1024 > ws.floats ||
                groups * n_units > ws.n_counters))
    return hipErrorInvalidConfiguration;
  float *scratch = ws.buf;
  int *counters = ws.cnt;
  if constexpr (MT == 1 && C == 1) {
    constexpr bool first = tokens_row_major(EPI);
    // a few tokens: load only the token rows that exist (8 or 16 of the tile's 32)
    if (M <= 16) {
      if (stream_waves(first, S) == 4) {
        if (M <= 8)
          return launch_stream_nw<EPI, MT, C, 4, 1>(A, lda, M, ks, W, n_units, blocks, S, out,
                                                           ldo, n_store, ks_out, scratch, counters, s, t, zero);
        return launch_stream_nw<EPI, MT, C, 4, 2>(A, lda, M, ks, W, n_units, blocks, S, out, ldo,
                                                         n_store, ks_out, scratch, counters, s, t, zero);
      }
      if (M <= 8)
        return launch_stream_nw<EPI, MT, C, 8, 1>(A, lda, M, ks, W, n_units, blocks, S, out, ldo,
                                                         n_store, ks_out, scratch, counters, s, t, zero);
      return launch_stream_nw<EPI, MT, C, 8, 2>(A, lda, M, ks, W, n_units, blocks, S, out, ldo,
                                                       n_store, ks_out, scratch, counters, s, t, zero);
    }
  }
  if (stream_waves(tokens_row_major(EPI), S) == 4)
    return launch_stream_nw<EPI, MT, C, 4>(A, lda, M, ks, W, n_units, blocks, S, out, ldo, n_store,
                                           ks_out, scratch, counters, s, t, zero);
  return launch_stream_nw<EPI, MT, C, 8>(A, lda, M, ks, W, n_units, blocks, S, out, ldo, n_store,
                                         ks_out, scratch, counters, s, t, zero);
}

StreamPlan stream_plan(int64_t M, int64_t n_cb, int64_t ks) {
  StreamPlan p;
  p.mt = M <= 32 ? 1 : 2;
  p.c = 1;
  p.s = 1;
  const int64_t groups = (M + 32 * p.mt - 1) / (32 * p.mt);
  // Contraction slices only for a single token group (M <= 64, the decode sizes): the
  // handles size their slice scratch and arrival counters for one group, and more
  // token groups give more workgroups anyway.
  if (groups > 1) return p;
  // One column block per workgroup over the whole contraction is the fastest shape
  // whenever there are enough blocks to occupy most compute units (measured at the
  // 70B-class decode shapes: wider groups or contraction slices only add traffic or
  // arrival latency there).  Narrow shards instead slice the contraction so that
  // about 160 workgroups stream the weight: each slice adds its share of the
  // hand-off through the last arriving workgroup (measured on the 40-block QKV shard
  // of the 70B-class attention, 8 waves: 80, 120, 160, 240, 320 and 480 workgroups
  // take 14.8, 13.0, 11.7, 12.6, 14.6 and 17.1 us).
  const int64_t wgs = n_cb * groups;
  if (wgs >= 192) return p;
  int64_t s = (160 + wgs / 2) / wgs;
  const int64_t max_s = (ks / 4) / 8;  // >= 8 batches of 2 pairs per slice
  if (s > max_s) s = max_s;
  if (s > kStreamMaxSlices) s = kStreamMaxSlices;
  if (s < 1) s = 1;
  p.s = static_cast<int>(s);
  return p;
}

StreamPlan stream_plan_out(int64_t M, int64_t n_cb, int64_t ks, bool out_f32) {
  StreamPlan p = stream_plan(M, n_cb, ks);
  const int64_t groups = (M + 32 * p.mt - 1) / (32 * p.mt);
  // The second product with an fp32 output and no slices of its own: two column
  // blocks per workgroup over half the contraction each, the halves added into the
  // zeroed output.  Each workgroup then loads the token operand for its half only,
  // once for both blocks: the per-CU load traffic drops by a quarter (one token
  // tile) or a third (two).
  if (out_f32 && groups == 1 && p.s == 1 && n_cb % 2 == 0 && (ks / 2) >= 4) {
    p.c = 2;
    p.s = 2;
    p.atom = 1;
  }
  return p;
}

template <int E>
static hipError_t launch_epi(const StreamPlan &plan, const void *A, int64_t lda, int64_t M,
                             int64_t ks, const void *W, int64_t n_cb, void *out, int64_t ldo,
                             int64_t n_store, int64_t ks_out, const StreamScratch &ws,
                             hipStream_t s, const Timing &t, const StreamZero &zero) {
  if (plan.atom) {
    // two column blocks, two atomic contraction halves (fp32 output only)
    if constexpr (E == EPI_OUT_F32) {
      if (plan.c != 2) return hipErrorInvalidConfiguration;
      if (plan.mt == 1)
        return launch_stream_cfg<E, 1, 2, true>(A, lda, M, ks, W, n_cb, plan.s, out, ldo, n_store,
                                                ks_out, ws, s, t, zero);
      return launch_stream_cfg<E, 2, 2, true>(A, lda, M, ks, W, n_cb, plan.s, out, ldo, n_store,
                                              ks_out, ws, s, t, zero);
    }
    return hipErrorInvalidConfiguration;
  }
  if (plan.c != 1) return hipErrorInvalidConfiguration;  // wider groups are not instantiated
  if (plan.mt == 1)
    return launch_stream_cfg<E, 1, 1>(A, lda, M, ks, W, n_cb, plan.s, out, ldo, n_store, ks_out,
                                      ws, s, t, zero);
  return launch_stream_cfg<E, 2, 1>(A, lda, M, ks, W, n_cb, plan.s, out, ldo, n_store, ks_out,
                                    ws, s, t, zero);
}

hipError_t launch_stream_gemm(int epi, const StreamPlan &plan, const void *A, int64_t lda,
                              int64_t M, int64_t ks, const void *W, int64_t n_cb, void *out,
                              int64_t ldo, int64_t n_store, int64_t ks_out, const StreamScratch &ws,
                              hipStream_t s, const Timing &t, const StreamZero &zero) {
  switch (epi) {
    case EPI_SILU_GATE:
      return launch_epi<EPI_SILU_GATE>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    case EPI_TANH:
      return launch_epi<EPI_TANH>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    case EPI_IDENTITY:
      return launch_epi<EPI_IDENTITY>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    case EPI_OUT_F32:
      return launch_epi<EPI_OUT_F32>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    case EPI_OUT_BF16:
      return launch_epi<EPI_OUT_BF16>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    case EPI_PROJ_F32:
      return launch_epi<EPI_PROJ_F32>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    case EPI_PROJ_BF16:
      return launch_epi<EPI_PROJ_BF16>(plan, A, lda, M, ks, W, n_cb, out, ldo, n_store, ks_out, ws, s, t, zero);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tpm
