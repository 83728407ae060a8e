// Matrix-core GEMM for large token counts (prefill).
//
// At prefill sizes each weight element meets thousands of tokens, so both
// projections of the shard are compute-bound (page "7.4 推理侧并行", section 7.4.1:
// prefill is one large matrix multiply).  The kernel is shaped around what limits a
// gfx950 compute unit when the matrix cores are meant to stay busy:
//
//  * Block tile 256 x 256 (tokens x columns), 8 waves (two per SIMD), each owning a
//    128 x 64 sub-tile: 128 fp32 sums per lane.  It multiplies with 16x16x32 products
//    (32 per stage per wave, 8 row blocks x 4 column blocks), which move fewer
//    register bytes per flop than 32x32x16 ones: flat out on every SIMD the 16x16x32
//    loop holds a 2.14 GHz shader clock against 1.77 GHz for 32x32x16, and since the
//    prefill products are power-limited that clock is what they gain (gate/up of the
//    TP=8 shard at M = 8192: 785-792 us with 32x32x16 products -> 701-716 us).  Their
//    fragments are gathered from the 32x32x16 operand order of the packed buffers with
//    a per-lane remap (see fragA / fragB).  Per stage a wave reads 8 token and 4 weight
//    fragments (12 KiB) from LDS; the second wave on the SIMD issues its products while
//    the first waits on its reads.  The wave count is a template parameter: NW = 4 (one
//    wave per SIMD, 128 x 128 sub-tiles, a third less LDS traffic per flop) measured
//    slower, since the lone wave has nothing to issue while it waits.
//  * Operands go from global memory straight into LDS through a ring of R stages of
//    32 contraction indices (32 KiB each: 16 token and 16 weight chunks of 1 KiB), so
//    R - 1 stages are in flight while one is multiplied (R = 3 in the library).  The
//    loads are buffer loads to LDS: one 32-bit lane offset per chunk and the stage
//    advance in a scalar offset (64-bit global addresses cost two vector additions per
//    chunk per stage and measured 2-3% slower).  A wave waits only for its own loads
//    of the next stage (an exact count of its outstanding loads), then one plain
//    barrier per stage; the loop is peeled so that the steady-state stages carry no
//    branch around a load.
//  * The weight and the packed hidden buffer arrive in fragment order
//    (tpm_internal.h), read with conflict-free ds_read_b128.  Row-major tokens are
//    loaded as 64-byte row segments of 16 rows per 1 KiB chunk, stored transposed
//    (piece p of row r at slot 16 p + r), so that a fragment read (lane l: row l % 16,
//    piece l / 16) is lane-contiguous: measured on MI355X, every arrangement that keeps
//    a row's four pieces side by side costs 4 bank-conflict cycles per such read
//    (58.5 M per gate/up launch), the transposed one none.
//  * Tiles are renumbered XCD-contiguous (workgroup b runs on XCD b mod 8) and grouped
//    four tile rows at a time, so the tiles an XCD runs together share operands in
//    its L2.  When the last round of tiles would leave at least half of the compute
//    units idle, its tiles run as two contraction halves; the halves park fp32 sums
//    with write-through stores and the second to arrive adds the other's (addition
//    of two values is order-free, so the result does not depend on arrival order)
//    and runs the epilogue.
//  * Fused epilogue: SiLU(gate) * up (a 32-column block holds 16 gate and the 16
//    matching up columns: two accumulator blocks, so a feature's gate and up sums sit
//    in the same lane), tanh or identity, staged through LDS and written as bf16 in the
//    packed hidden order; or the row-major partial store (fp32 or bf16).
#include <type_traits>

#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

namespace {

constexpr int kGemmGroupRows = 4;  // tile rows per launch-order group
constexpr int kStageChunks = 32;   // 1 KiB chunks per stage: 16 token, 16 weight

// s_waitcnt immediate: at most n vector-memory operations of this wave outstanding.
template <int n>
__device__ __forceinline__ void wait_vmem() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most n stages of PW loads (n in 0 .. R - 1, a run-time count turned
// into an immediate) of this wave are outstanding.
template <int PW, int R>
__device__ __forceinline__ void wait_stages(int n) {
  if (R >= 5 && n >= 4) wait_vmem<(R >= 5 ? 4 : 0) * PW>();
  else if (R >= 4 && n >= 3) wait_vmem<(R >= 4 ? 3 : 0) * PW>();
  else if (R >= 3 && n >= 2) wait_vmem<(R >= 3 ? 2 : 0) * PW>();
  else if (n >= 1) wait_vmem<PW>();
  else wait_vmem<0>();
}

}  // namespace

// A wave's 128 x (32 WNB) sub-tile: acc[i][j] for 16-row block i and 16-column block j,
// 4 fp32 sums per lane (row 4 (lane / 16) + r, column lane % 16): 128 per lane.
template <int NW>
struct GemmShape {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static constexpr int WNB = 16 / NW;  // 32-column blocks per wave
  static constexpr int AI = 8;         // 16-row blocks
  static constexpr int AJ = 2 * WNB;   // 16-column blocks
};

// Epilogue of a 256 x 256 tile held by NW waves as 128 x (32 WNB) sub-tiles (wave at
// row half wm, column group wn): SiLU(gate) * up, tanh or identity written as bf16 into
// the packed hidden buffer (staged through the LDS ring, free after the main loop), or
// the row-major partial store.
template <int EPI, int NW, int R>
__device__ __forceinline__ void gemm_epilogue(f32x4_t (&acc)[GemmShape<NW>::AI][GemmShape<NW>::AJ],
                                              u32x4_t (*lds)[kStageChunks][64], int wave, int wm,
                                              int wn, int lane, int tn, int row0, int M,
                                              void *__restrict__ out, int64_t ldo, int n_store,
                                              int ks_out) {
  using Sh = GemmShape<NW>;
  constexpr int WNB = Sh::WNB;
  constexpr bool HIDDEN = writes_hidden(EPI);
  if constexpr (HIDDEN) {
    // h of the wave's 128 rows, BPP column blocks (JW features each) per pass, staged
    // through LDS (the ring, free after the main loop) and written as 16-byte chunks
    // of the packed hidden buffer.
    constexpr int JW = (EPI == EPI_SILU_GATE) ? 16 : 32;          // features per column block
    constexpr int MAXF = R * kStageChunks * 1024 / NW / 256 - 8;  // features per pass that fit
    constexpr int BPP = (WNB * JW <= MAXF) ? WNB : (WNB / 2) * JW <= MAXF ? WNB / 2 : 1;
    static_assert(BPP * JW <= MAXF && WNB % BPP == 0, "epilogue staging must fit the ring");
    constexpr int FPP = BPP * JW;                                 // features per pass
    constexpr int HS = FPP + 8;                                   // LDS row stride (bf16)
    uint16_t *hs = reinterpret_cast<uint16_t *>(&lds[0][0][0]) + wave * (128 * HS);
#pragma unroll
    for (int pass = 0; pass < WNB / BPP; ++pass) {
#pragma unroll
      for (int jj = 0; jj < BPP; ++jj) {
        const int j = pass * BPP + jj;
        // 32-column block j is 16-column blocks 2 j (gate, or its first half) and 2 j + 1
        // (up, or its second half): gate and up of a feature share a lane
#pragma unroll
        for (int i = 0; i < Sh::AI; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = 16 * i + 4 * (lane >> 4) + r;
            const int c = lane & 15;
            const float v = acc[i][2 * j][r], u = acc[i][2 * j + 1][r];
            if constexpr (EPI == EPI_SILU_GATE) {
              hs[rr * HS + jj * 16 + c] = f32_to_bf16(silu_f(v) * u);
            } else {
              hs[rr * HS + jj * 32 + c] = f32_to_bf16(act_f<EPI>(v));
              hs[rr * HS + jj * 32 + 16 + c] = f32_to_bf16(act_f<EPI>(u));
            }
          }
        }
      }
      __syncthreads();
      const int fp0 = (tn * 8 + wn * WNB + pass * BPP) * JW;  // first feature of this pass
#pragma unroll
      for (int q = lane; q < 128 * (FPP / 8); q += 64) {
        const int rr = q & 127, qc = q >> 7;
        const int jf = fp0 + 8 * qc;
        const int s = 2 * (jf >> 5) + ((jf >> 3) & 1);
        const int row = row0 + wm * 128 + rr;
        const int ln = 32 * ((jf >> 4) & 1) + (row & 31);
        const int64_t chunk = (static_cast<int64_t>(row >> 5) * ks_out + s) * 64 + ln;
        static_cast<u32x4_t *>(out)[chunk] = *reinterpret_cast<const u32x4_t *>(&hs[rr * HS + 8 * qc]);
      }
      if (pass + 1 < WNB / BPP) __syncthreads();
    }
  } else {
#pragma unroll
    for (int i = 0; i < Sh::AI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wm * 128 + 16 * i + 4 * (lane >> 4) + r;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < Sh::AJ; ++j) {
          const int col = (tn * 8 + wn * WNB) * 32 + 16 * j + (lane & 15);
          const int64_t o = static_cast<int64_t>(row) * ldo + col;
          if constexpr (stores_f32(EPI)) {
            if (col < n_store) static_cast<float *>(out)[o] = acc[i][j][r];
          } else {
            if (col < n_store) static_cast<uint16_t *>(out)[o] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  }
}

// Buffer descriptor of a raw byte-addressed buffer (gfx9 layout: dword 3 = 0x00020000,
// 32-bit data format, no swizzle); every access made through it stays in bounds by
// construction, so the record count is the largest one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(0xffffffffu), 0x00020000);
}
// 16 bytes per lane from global memory (buffer r, byte offset voff + soff) straight
// into LDS: lane l's bytes land at lds + 16 l (lds is wave-uniform).  Counted by the
// vector-memory counter.  The builtin exists only for the device; the host pass sees
// an empty body.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                          void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, soff, 0, 0);
#endif
}

template <int EPI, int NW, int R>
__global__ void __launch_bounds__(NW * 64, 1)
k_gemm(const uint16_t *__restrict__ A, int64_t lda, int M, int k_stages,
       const u32x4_t *__restrict__ W, int ks_a, int ntm, int ntn, void *__restrict__ out,
       int64_t ldo, int n_store, int ks_out, int n_whole, uint64_t *__restrict__ split_buf,
       int *__restrict__ split_cnt) {
  constexpr bool FIRST = tokens_row_major(EPI);  // row-major token operand
  using Sh = GemmShape<NW>;
  constexpr int WNB = Sh::WNB, AI = Sh::AI, AJ = Sh::AJ;
  constexpr int PT = 16 / NW;   // token chunks each wave loads per stage
  constexpr int PWW = 16 / NW;  // weight chunks each wave loads per stage
  constexpr int PW = PT + PWW;
  static_assert(R >= 2 && R <= 5, "the ring must fit the 160 KiB of LDS");
  __shared__ u32x4_t lds[R][kStageChunks][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  // Work item: workgroups [0, n_whole) run whole tiles, the others one contraction
  // half (khalf) of tiles [n_whole, nt), two per tile.
  const int nt = ntm * ntn;
  const int b = blockIdx.x;
  const bool split = b >= n_whole;
  int t, pair = 0, khalf = 0;
  if (!split) {
    t = b;
    if ((n_whole & 7) == 0) t = (b & 7) * (n_whole >> 3) + (b >> 3);  // XCD-contiguous
  } else {
    const int h = b - n_whole, rem = nt - n_whole;
    if ((rem & 7) == 0 && (n_whole & 7) == 0) {
      // the two halves of a tile 8 workgroups apart: the same XCD, so the exchange
      // of the sums usually stays in its L2
      pair = 8 * (h >> 4) + (h & 7);
      khalf = (h >> 3) & 1;
    } else {
      pair = h >> 1;
      khalf = h & 1;
    }
    t = n_whole + pair;
  }
  const int k_lo = split && khalf ? k_stages / 2 : 0;
  const int k_n = split && !khalf ? k_stages / 2 : k_stages - k_lo;

  // Tile coordinates, tiles grouped by kGemmGroupRows tile rows.
  const int per_group = kGemmGroupRows * ntn;
  const int first_m = (t / per_group) * kGemmGroupRows;
  const int gm = min(ntm - first_m, kGemmGroupRows);
  const int tm = first_m + (t % per_group) % gm;
  const int tn = (t % per_group) / gm;
  const int row0 = tm * kTileM;

  // Stage layout: chunks 0..15 hold the token operand, 16..31 the weight: chunk
  // 16 + 8 ks + cb is the weight fragment of column block cb of the tile at k-step ks
  // of the stage; for the packed hidden buffer chunk 8 ks + rb is the fragment of row
  // block rb; for row-major tokens chunk c holds 64 bytes of tile rows 16 c ..
  // 16 c + 15, transposed (piece p of row r at slot 16 p + r).  The direct-to-LDS
  // load puts lane l's 16 bytes at 16 l of the chunk, so each source offset is the
  // lane's own piece of that chunk.  Wave w loads token chunks [PT w, PT w + PT) and
  // weight chunks 16 + [PWW w, PWW w + PWW).  Offsets are in bytes from per-tile
  // bases: the token rows of the tile and the tile's first column block.
  const uint16_t *tbase = FIRST ? A + static_cast<int64_t>(row0) * lda
                                : A + static_cast<int64_t>(row0 >> 5) * ks_a * 512;
  const u32x4_t *wbase = W + static_cast<int64_t>(tn) * 8 * 64;
  const unsigned tstep = FIRST ? 64u : 2048u;                            // bytes per stage
  const unsigned wstep = static_cast<unsigned>(ntn) * 8u * 2048u;        // bytes per stage
  unsigned tvo[PT], wvo[PWW];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int c = PT * wave + q;
    if constexpr (FIRST) {
      // transposed token chunk: lane l holds piece l / 16 of row l % 16, so that a
      // fragment read is lane-contiguous
      const int r = 16 * c + (lane & 15);
      const int rr = row0 + r < M ? r : M - 1 - row0;  // rows past the end repeat the last
      tvo[q] = static_cast<unsigned>((static_cast<int64_t>(rr) * lda + 8 * (lane >> 4)) * 2);
    } else {
      const int ks = c >> 3, rb = c & 7;
      tvo[q] = static_cast<unsigned>(((rb * ks_a + ks) * 64 + lane) * 16);
    }
  }
#pragma unroll
  for (int q = 0; q < PWW; ++q) {
    const int c = PWW * wave + q;
    const int ks = c >> 3, cb = c & 7;
    wvo[q] = static_cast<unsigned>(((ks * ntn * 8 + cb) * 64 + lane) * 16);
  }
  const __amdgpu_buffer_rsrc_t trs = raw_rsrc(tbase), wrs = raw_rsrc(wbase);
  auto issue = [&](int kt, int buf, int q) {
    const unsigned st = static_cast<unsigned>(k_lo + kt);
    if (q < PT) {
      dma16_buf(trs, tvo[q], st * tstep, &lds[buf][PT * wave + q][0]);
    } else {
      const int qq = q - PT;
      dma16_buf(wrs, wvo[qq], st * wstep, &lds[buf][16 + PWW * wave + qq][0]);
    }
  };

  f32x4_t acc[AI][AJ];
#pragma unroll
  for (int i = 0; i < AI; ++i)
#pragma unroll
    for (int j = 0; j < AJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
  auto mma = [&](int i, int j, const u32x4_t &a, const u32x4_t &w) {
    acc[i][j] = mfma_16x16x32(a, w, acc[i][j]);
  };

  // Fragments of a whole stage (its 32 contraction indices).  The packed buffers hold
  // the 32x32x16 operand order (two k-steps of 16, lane halves of 8); the k-group
  // g = lane / 16 of a 16x16x32 operand is k-step g & 1, lane half g >> 1 of that
  // order, so A and B agree on the contraction order.  Each 16-lane group reads 256
  // contiguous bytes (row-major tokens: the whole transposed chunk, lane by lane),
  // free of bank conflicts.
  const u32x4_t *lds_flat = &lds[0][0][0];
  const int g16 = lane >> 4, r16 = lane & 15;
  auto fragA = [&](int buf, int ri) -> u32x4_t {  // rows 16 ri .. 16 ri + 15 of the wave's 128
    const int row = wm * 128 + 16 * ri + r16;      // row of the tile
    if constexpr (FIRST) {
      return lds_flat[(buf * kStageChunks + (row >> 4)) * 64 + lane];
    } else {
      return lds[buf][8 * (g16 & 1) + (row >> 5)][32 * (g16 >> 1) + (row & 31)];
    }
  };
  auto fragB = [&](int buf, int cj) -> u32x4_t {  // columns 16 cj .. of the wave's 32 WNB
    const int cb = WNB * wn + (cj >> 1);
    return lds[buf][16 + 8 * (g16 & 1) + cb][32 * (g16 >> 1) + 16 * (cj & 1) + r16];
  };

  // Wait until this wave's loads of stage kt + 1 have landed (later stages may stay
  // in flight) and its LDS reads are done, then meet the other waves: after the
  // barrier all of stage kt + 1 is in LDS and nobody reads stage kt's buffer any
  // more.
  auto sync_next = [&](int kt) {
    wait_stages<PW, R>(min(R - 2, k_n - 2 - kt));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto sync_mid = [&](int kt, auto refill_c) {
    if constexpr (decltype(refill_c)::value) {
      wait_vmem<(R - 2) * PW>();  // stages kt + 2 .. kt + R - 1 stay in flight
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      sync_next(kt);
    }
  };

  // Prologue: R stages in flight, then stage 0's first fragments in registers.
#pragma unroll
  for (int st = 0; st < R; ++st)
    if (st < k_n) {
#pragma unroll
      for (int q = 0; q < PW; ++q) issue(st, st, q);
    }
  wait_stages<PW, R>(min(R - 1, k_n - 1));
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // f0[0..3]: A row blocks 0..3, f0[4 .. 4 + AJ): the B blocks; f1: A row blocks 4..7
  u32x4_t f0[4 + AJ], f1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) f0[i] = fragA(0, i);
#pragma unroll
  for (int j = 0; j < AJ; ++j) f0[4 + j] = fragB(0, j);

  // Stage kt: the first half multiplies row blocks 0..3 (f0) by every column block
  // while row blocks 4..7 are read into f1; then (sync) the second half multiplies row
  // blocks 4..7, column block by column block, so that each B fragment is dead after
  // its four products and the next stage's copy can be read in its place; meanwhile
  // the buffer of stage kt is refilled with stage kt + R and the next stage's row
  // blocks 0..3 are read.  The scheduling barriers keep one fragment read or load
  // between products.  REFILL and MORE are compile-time so the steady-state loop has
  // no branches: the last R stages run in a peeled tail.
  auto stage = [&](int kt, int buf, auto refill_c, auto more_c) {
    constexpr bool REFILL = decltype(refill_c)::value;
    constexpr bool MORE = decltype(more_c)::value;
    const int nbuf = buf + 1 == R ? 0 : buf + 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < AJ; ++j) {
        mma(i, j, f0[i], f0[4 + j]);
        __builtin_amdgcn_sched_barrier(0);
        if (j == 0) f1[i] = fragA(buf, 4 + i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (MORE) sync_mid(kt, refill_c);
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mma(4 + i, j, f1[i], f0[4 + j]);
        __builtin_amdgcn_sched_barrier(0);
        const int q = j * 4 + i;
        if constexpr (REFILL)
          if (q < PW) issue(kt + R, buf, q);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MORE) {
          if (j == 0) f0[i] = fragA(nbuf, i);
          if (i == 3) f0[4 + j] = fragB(nbuf, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0, buf = 0;
  for (; kt + R < k_n; ++kt) {
    stage(kt, buf, T_(), T_());
    buf = buf + 1 == R ? 0 : buf + 1;
  }
  for (; kt + 1 < k_n; ++kt) {
    stage(kt, buf, F_(), T_());
    buf = buf + 1 == R ? 0 : buf + 1;
  }
  stage(kt, buf, F_(), F_());
  __syncthreads();  // the ring is reused by the epilogue

  if (split) {
    // Park this half's sums (write-through stores: complete at the device coherence
    // point once counted), count the workgroup in; the second to arrive reads the
    // other half's sums with coherent loads and goes on.
    int *s_second = reinterpret_cast<int *>(&lds[0][0][0]);  // the ring is free now
    constexpr int NV = AI * AJ * 2;  // 64-bit pairs of sums per thread
    uint64_t *mine = split_buf + (static_cast<int64_t>(pair) * 2 + khalf) * (NW * 64 * NV);
    uint64_t *other = split_buf + (static_cast<int64_t>(pair) * 2 + (khalf ^ 1)) * (NW * 64 * NV);
#pragma unroll
    for (int i = 0; i < AI; ++i)
#pragma unroll
      for (int j = 0; j < AJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint64_t v = static_cast<uint64_t>(__float_as_uint(acc[i][j][r])) |
                             (static_cast<uint64_t>(__float_as_uint(acc[i][j][r + 1])) << 32);
          __hip_atomic_store(&mine[((i * AJ + j) * 2 + r / 2) * (NW * 64) + tid], v,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    // The stores above are complete at the coherence point once the wave's memory
    // counters drain (s_waitcnt 0); only then is the workgroup counted in.  As in the
    // streaming kernel's slice hand-off, the ordering rests on the emitted code (sc1
    // stores and loads, the wait and the barrier before the counter), which
    // tests/test_handoff_asm.py checks, not on relaxed atomics' language semantics.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(&split_cnt[pair], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      *s_second = old == 1;
      if (old == 1)  // both halves in: reset for the next call
        __hip_atomic_store(&split_cnt[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const bool second = *s_second;
    __syncthreads();  // every wave has read the flag before the epilogue reuses the ring
    if (!second) return;
#pragma unroll
    for (int i = 0; i < AI; ++i)
#pragma unroll
      for (int j = 0; j < AJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint64_t v = __hip_atomic_load(&other[((i * AJ + j) * 2 + r / 2) * (NW * 64) + tid],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          acc[i][j][r] += __uint_as_float(static_cast<uint32_t>(v));
          acc[i][j][r + 1] += __uint_as_float(static_cast<uint32_t>(v >> 32));
        }
  }
  gemm_epilogue<EPI, NW, R>(acc, lds, wave, wm, wn, lane, tn, row0, M, out, ldo, n_store, ks_out);
}

}  // namespace tpm

namespace tpm {

// The configuration the library launches: 8 waves, a 3-stage ring (TP=8 shard at
// M = 8192, medians of 20 launches; gate/up / down: 4 stages 710-716 / 370 us, 3 stages
// 701-704 / 367-369 us, 4 waves 752-767 / 372-382 us; with 32x32x16 products and 4
// stages, a form since removed, 785-792 / 373-374 us).
constexpr int kGemmWaves = 8;
constexpr int kGemmRing = 3;

template <int EPI, int NW = kGemmWaves, int R = kGemmRing>
hipError_t launch_gemm_one(const void *A, int64_t lda, int64_t M, int64_t K, const void *W,
                           int64_t n_packed, void *out, int64_t ldo, int64_t n_store,
                           int64_t ks_out, const TiledSplit &sp, hipStream_t s, const Timing &t) {
  if (K % kGemmK || n_packed % kTileN || M < 1) return hipErrorInvalidValue;
  // Buffer offsets are 32-bit: operands past that reach take the global-address form
  // of the tiled kernel instead.
  const int64_t w_bytes = K * n_packed * 2, tile_rows_bytes = kTileM * (tokens_row_major(EPI) ? lda * 2 : K * 2);
  if (w_bytes >= (int64_t(1) << 32) || tile_rows_bytes >= (int64_t(1) << 31))
    return launch_tiled_gemm(EPI, A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
  const int ntm = static_cast<int>((M + kTileM - 1) / kTileM);
  const int ntn = static_cast<int>(n_packed / kTileN);
  const int k_stages = static_cast<int>(K / kGemmK);
  const int split = (sp.buf && sp.cnt && k_stages >= 2 * R)
                        ? tiled_split_tiles(static_cast<int64_t>(ntm) * ntn, sp.n_cu, sp.max_tiles)
                        : 0;
  const int n_whole = ntm * ntn - split;
  hipExtLaunchKernelGGL((k_gemm<EPI, NW, R>), dim3(n_whole + 2 * split), dim3(NW * 64), 0, s,
                        t.start, t.stop, 0, static_cast<const uint16_t *>(A), lda,
                        static_cast<int>(M), k_stages, static_cast<const u32x4_t *>(W),
                        static_cast<int>(K / kFragK), ntm, ntn, out, ldo,
                        static_cast<int>(n_store), static_cast<int>(ks_out), n_whole,
                        static_cast<uint64_t *>(sp.buf), sp.cnt);
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t K, const void *W,
                       int64_t n_packed, void *out, int64_t ldo, int64_t n_store, int64_t ks_out,
                       const TiledSplit &sp, hipStream_t s, const Timing &t) {
  switch (epi) {
    case EPI_SILU_GATE:
      return launch_gemm_one<EPI_SILU_GATE>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    case EPI_TANH:
      return launch_gemm_one<EPI_TANH>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    case EPI_IDENTITY:
      return launch_gemm_one<EPI_IDENTITY>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    case EPI_OUT_F32:
      return launch_gemm_one<EPI_OUT_F32>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    case EPI_OUT_BF16:
      return launch_gemm_one<EPI_OUT_BF16>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    case EPI_PROJ_F32:
      return launch_gemm_one<EPI_PROJ_F32>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    case EPI_PROJ_BF16:
      return launch_gemm_one<EPI_PROJ_BF16>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, s, t);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tpm
