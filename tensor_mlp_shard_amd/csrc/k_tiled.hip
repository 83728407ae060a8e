// LDS-tiled bf16 matrix-core GEMM for large token counts, with a grouped mode.
//
// At prefill sizes each weight element meets thousands of tokens, so the
// projections are compute-bound (page "7.4 推理侧并行", section 7.4.1: prefill is a
// large matrix multiply).  The plain prefill products run on k_gemm.hip; this kernel
// serves the grouped experts with many tokens per expert (one launch over every
// expert's rows, the counts read on the device) and operands beyond the 32-bit
// buffer offsets k_gemm.hip uses.  It keeps the matrix cores fed from LDS:
//
//  * Block tile 256 x 256 (tokens x columns).  NW waves: four (one per SIMD, each
//    owning a 128 x 128 sub-tile = 4 x 4 MFMA 32x32x16 tiles, 256 fp32
//    accumulators per lane) or eight (two per SIMD, 128 x 64 sub-tiles, so one
//    wave's waits are covered by the other's products).
//  * Operands go from global memory straight into an LDS ring of 128 KiB
//    (global_load_lds: no register staging), several stages ahead of use; a wave
//    waits only for the stage it needs, then a plain barrier.
//  * The weight and the packed hidden buffer arrive already in fragment order
//    (tpm_internal.h) and are stored so, so each wave reads one operand with one
//    conflict-free 1 KiB ds_read_b128 (16 B per lane, lane-contiguous).
//    Row-major tokens are loaded as whole 128-byte row segments (8 cache lines per
//    load instead of 32 partial ones) into a swizzled layout that the fragment
//    reads gather from without bank conflicts.
//  * Work tiles are renumbered so that consecutive tiles land on the same XCD
//    (workgroup b runs on XCD b % 8), and grouped four tile rows at a time, so
//    tiles that share operands share that XCD's L2.
//  * One workgroup holds a compute unit, so tiles run in rounds of one tile per
//    compute unit.  When the last round would leave at least half of the units
//    idle, its tiles are split into two halves of the contraction run by two
//    workgroups; each half parks its fp32 sums, and the second to arrive adds the
//    other's (addition of two values is order-free, so the result does not depend
//    on arrival order) and runs the epilogue.
//  * The epilogue is fused: SiLU(gate) * up (each 32-column block holds 16 gate
//    and the 16 matching up columns; lane c meets lane c + 16 by a cross-lane
//    exchange), tanh or identity, staged through LDS and written as bf16 in the
//    packed hidden order; or the partial store.
#include "device_common.h"
#include "tpm_internal.h"

namespace tpm {

constexpr int kGroupRows = 4;  // tile rows per launch-order group

// Shape of one configuration: SP k-step pairs per LDS stage, NW waves, R stages.
//   R      stages in the LDS ring (32 SP KiB each; at most 160 KiB in total)
//   CH     1 KiB chunks per stage: per k-step 8 token fragments (32-row blocks)
//          and 8 weight fragments (32-column blocks) of the 256 x 256 tile
//   PW     chunks each wave loads per stage
//   WNB    32-column blocks per wave (its rows are always 4 blocks = 128 rows)
template <int SP, int NW, int RING>
struct TiledShape {
  static constexpr int R = RING;
  static_assert(R >= 2 && R * SP <= 5, "the ring must fit the 160 KiB of LDS");
  static constexpr int CH = 32 * SP;
  static constexpr int PW = CH / NW;
  static constexpr int WNB = 16 / NW;
  static constexpr int NF = 4 + WNB;  // fragments per k-step per wave
  static_assert(PW % 4 == 0 || PW == 4 || PW == 8, "loads per stage split in quarters");
};

// s_waitcnt immediate that waits until at most n vector-memory operations of this
// wave are outstanding (and does not wait on the other counters).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// lds + 16 l (lds is wave-uniform).  Counted by the vector-memory counter.  The
// builtin exists only for the device; the host pass sees an empty body.
__device__ __forceinline__ void load_lds16(const void *g, void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
#endif
}

// Swizzle of the row-major token stages: piece p of tile row r sits at slot
// 8 (r % 8) + (p ^ tok_swz(r)) of its 1 KiB chunk.  The 32 rows a fragment read
// touches land, for any 8 or 16 consecutive lanes, on distinct 16-byte bank groups.
__device__ __forceinline__ int tok_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int EPI, int SP, int NW, int RING, bool PART>
__global__ void __launch_bounds__(NW * 64, 1)
k_tiled(const uint16_t *__restrict__ A, int64_t lda, int M, int k_total,
        const u32x4_t *__restrict__ W, int k_blocks, int ntm, int ntn,
        void *__restrict__ out, int64_t ldo, int n_store, int ks_out, int n_whole,
        uint64_t *__restrict__ split_buf, int *__restrict__ split_cnt, TiledGroups grp) {
  constexpr bool FIRST = tokens_row_major(EPI);  // row-major token operand
  constexpr bool HIDDEN = writes_hidden(EPI);     // epilogue writes the packed hidden buffer
  using Sh = TiledShape<SP, NW, RING>;
  static_assert(!FIRST || SP == 2, "row-major token stages are 128-byte row segments");
  constexpr int R = Sh::R, CH = Sh::CH, PW = Sh::PW, WNB = Sh::WNB, NF = Sh::NF;
  __shared__ u32x4_t lds[R][CH][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  // Work item.  Workgroups [0, n_whole) run whole tiles [0, n_whole); the others
  // run one contraction half (khalf) of tiles [n_whole, nt), two per tile.
  const int nt = ntm * ntn;
  const int b = blockIdx.x;
  const bool split = b >= n_whole;
  int t, pair = 0, khalf = 0;
  if (!split) {
    // XCD-contiguous renumbering of the whole tiles
    t = b;
    if ((n_whole & 7) == 0) t = (b & 7) * (n_whole >> 3) + (b >> 3);
  } else {
    const int h = b - n_whole, rem = nt - n_whole;
    if ((rem & 7) == 0 && (n_whole & 7) == 0) {
      // halves of one tile 8 workgroups apart: the same XCD, so the exchange of
      // the sums usually stays in its L2
      pair = 8 * (h >> 4) + (h & 7);
      khalf = (h >> 3) & 1;
    } else {
      pair = h >> 1;
      khalf = h & 1;
    }
    t = n_whole + pair;
  }
  const int k_lo = split && khalf ? k_total / 2 : 0;
  const int k_tiles = split && !khalf ? k_total / 2 : k_total - k_lo;
  // Tile coordinates.  row0: first token row of the tile (X rows / output rows),
  // row_end: end of the valid rows, hrow0: first row in the packed hidden buffer,
  // Wt: the weight the tile multiplies.
  int tn, row0, row_end, hrow0;
  const u32x4_t *Wt = W;
  if (grp.n_groups == 0) {
    // one matrix: tiles grouped by kGroupRows tile rows
    const int per_group = kGroupRows * ntn;
    const int first_m = (t / per_group) * kGroupRows;
    const int gm = min(ntm - first_m, kGroupRows);
    const int tm = first_m + (t % per_group) % gm;
    tn = (t % per_group) / gm;
    row0 = hrow0 = tm * kTileM;
    row_end = M;
  } else {
    // grouped (one weight per group, the groups' rows contiguous in X): tile row
    // t / ntn counts through the groups' row tiles in group order; each group's
    // hidden rows start on a tile boundary.  Group sizes come from device memory and
    // are clamped to the M rows there are; a workgroup past the last tile exits.
    int rt = t / ntn;
    tn = t % ntn;
    int off = 0, hoff = 0, g = 0, n = 0;
    for (; g < grp.n_groups; ++g) {
      n = min(max(grp.counts[g], 0), M - off);
      const int tiles = (n + kTileM - 1) / kTileM;
      if (rt < tiles) break;
      rt -= tiles;
      off += n;
      hoff += tiles * kTileM;
    }
    if (g == grp.n_groups) return;  // uniform over the workgroup: no tile left
    row0 = off + rt * kTileM;
    row_end = off + n;
    hrow0 = hoff + rt * kTileM;
    Wt = W + static_cast<int64_t>(g) * grp.w_stride;
  }

  // Stage layout: chunk c < 16 SP is token fragment (row block (c / 2) % 8, k-step
  // 2 (c / 16) + c % 2 of the stage) for the packed hidden buffer, or 8 whole token
  // rows for row-major X (below); chunk 16 SP + c the weight fragment of column
  // block (c / 2) % 8 at the same k-step.  Wave w loads chunks [PW w, PW w + PW):
  // the direct-to-LDS load puts lane l's 16 bytes at 16 l of the chunk, so every
  // source address is the lane's own piece of that chunk.
  const u32x4_t *src[PW];
  int64_t step[PW];  // source advance per stage, in 16-byte units
  bool skip[PW];     // PART: token chunk wholly past the valid rows, never loaded
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    const int c = PW * wave + q;  // wave-uniform
    const bool tok = c < 16 * SP;
    const int cc = tok ? c : c - 16 * SP;
    const int blk = (cc >> 1) & 7;               // row or column block within the tile
    const int kstep = 2 * (cc >> 4) + (cc & 1);  // k-step within the stage
    skip[q] = PART && tok && row0 + (FIRST ? 8 * c : 32 * blk) >= row_end;
    if (tok) {
      if constexpr (FIRST) {
        // Row-major tokens: chunk c holds tile rows 8 c .. 8 c + 7, each as its
        // whole 128-byte segment of the stage (8 pieces of 16 bytes), piece p of
        // row r at slot 8 (r % 8) + (p ^ tok_swz(r)).  Every load fetches 8 whole
        // cache lines, and the swizzle keeps the fragment reads free of bank
        // conflicts.
        const int r = 8 * c + (lane >> 3);
        int row = row0 + r;
        row = row < row_end ? row : row_end - 1;  // rows past the end repeat the last; never stored
        const int piece = (lane & 7) ^ tok_swz(r);
        src[q] = reinterpret_cast<const u32x4_t *>(A + static_cast<int64_t>(row) * lda + 8 * piece);
        step[q] = 4 * SP;  // 32 SP bf16
      } else {
        src[q] = reinterpret_cast<const u32x4_t *>(A) +
                 ((static_cast<int64_t>(hrow0 >> 5) + blk) * k_blocks + kstep) * 64 + lane;
        step[q] = 2 * SP * 64;
      }
    } else {
      src[q] = Wt + (static_cast<int64_t>(kstep) * ntn * 8 + tn * 8 + blk) * 64 + lane;
      step[q] = static_cast<int64_t>(2 * SP) * ntn * 8 * 64;
    }
    src[q] += step[q] * k_lo;  // first stage of this workgroup's contraction range
  }
  // Quarter `part` (0..3) of this wave's loads of a stage.
  auto issue_part = [&](int kt, int buf, int part) {
#pragma unroll
    for (int q = part * (PW / 4); q < (part + 1) * (PW / 4); ++q)
      if (!skip[q]) load_lds16(src[q] + step[q] * kt, &lds[buf][PW * wave + q][0]);
  };
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int q = 0; q < PW; ++q)
      if (!skip[q]) load_lds16(src[q] + step[q] * kt, &lds[buf][PW * wave + q][0]);
  };

  f32x16_t acc[4][WNB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment f of k-step ksi of a stage: f < 4 token row block wm*4 + f, else
  // weight column block wn*WNB + f - 4.
  // Row-major token stages: the slot of this lane's row within its chunk, and the
  // lane's piece of k-step ksi (kappa order: 32 (ksi / 2) + 16 h + 8 (ksi % 2))
  // after the swizzle.  The swizzle depends on the row only through lane % 32.
  const int tok_slot = 8 * (lane & 7);
  const int tok_x = tok_swz(lane & 31);
  auto tok_piece = [&](int ksi) { return (4 * (ksi >> 1) + 2 * (lane >> 5) + (ksi & 1)) ^ tok_x; };
  const u32x4_t *lds_flat = &lds[0][0][0];
  auto frag = [&](int buf, int ksi, int f) -> u32x4_t {
    const int cbase = 16 * (ksi >> 1) + (ksi & 1);
    if (f < 4) {
      if constexpr (FIRST) {
        // chunk of rows 32 (wm 4 + f) + lane % 32
        const int chunk = 4 * (wm * 4 + f) + ((lane & 31) >> 3);
        return lds_flat[(buf * CH + chunk) * 64 + tok_slot + tok_piece(ksi)];
      } else {
        return lds[buf][cbase + 2 * (wm * 4 + f)][lane];
      }
    }
    return lds[buf][16 * SP + cbase + 2 * (wn * WNB + (f - 4))][lane];
  };
  auto read_k = [&](int buf, int ksi, u32x4_t (&f)[NF]) {
#pragma unroll
    for (int q = 0; q < NF; ++q) f[q] = frag(buf, ksi, q);
  };
  // PART (grouped launches, whose tiles often hold a short run of tokens): the row
  // blocks of this wave's 128 rows past the valid rows (wave-uniform) skip their
  // products and token fragment reads; their sums stay zero and are never stored as
  // output (a hidden row past the end holds act(0) = 0).
  const int wrows = row_end - row0 - wm * 128;
  const int nvb = !PART ? 4 : wrows <= 0 ? 0 : min(4, (wrows + 31) >> 5);
  // Fragments q, q + 1 (if they exist) of one k-step.
  auto read_pair = [&](int buf, int ksi, u32x4_t (&f)[NF], int q) {
#pragma unroll
    for (int r = q; r < q + 2; ++r)
      if (r < NF && (!PART || r >= 4 || r < nvb)) f[r] = frag(buf, ksi, r);
  };
  // The products of token fragment row i of one k-step.
  auto mfma_row = [&](const u32x4_t (&f)[NF], int i) {
    if (PART && i >= nvb) return;
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = mfma_32x32x16(f[i], f[4 + j], acc[i][j]);
  };
  // Wait until this wave's loads of the stage after `kt` have landed (the later
  // stages' loads may stay in flight) and its LDS reads have completed, then meet
  // the other waves: after the barrier every wave's loads of stage kt + 1 are in
  // LDS and nobody reads the buffer of stage kt any more.
  auto sync_stage = [&](int kt) {
    const int later = min(R - 2, k_tiles - 2 - kt);  // stages after kt + 1 in flight
    // (with skipped loads a stage holds fewer than PW of this wave's loads: wait for all)
    if (PART) wait_vm<0>();
    else if (R >= 5 && later >= 3) wait_vm<(R >= 5 ? 3 : 0) * PW>();
    else if (R >= 4 && later >= 2) wait_vm<(R >= 4 ? 2 : 0) * PW>();
    else if (R >= 3 && later >= 1) wait_vm<PW>();
    else wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
    // A plain hardware barrier: no fence (it would wait for every load in flight);
    // the empty asm statements keep the compiler from moving LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Prologue: R stages in flight, the first k-step's fragments in registers.
#pragma unroll
  for (int st = 0; st < R; ++st)
    if (st < k_tiles) issue(st, st);
  u32x4_t fc[NF], fn[NF];  // fragments of the current and of the next k-step
  sync_stage(-1);
  read_k(0, 0, fc);
  // Stage kt (2 SP k-steps): each k-step's products run while the next k-step's
  // fragments are read, a fragment pair per row of products (a wait on LDS reads
  // is always a wait for all of them, so the reads must not sit right before
  // products that do not need them).  Before the last k-step: sync (stage kt + 1
  // landed, buffer of stage kt free), then refill that buffer with stage kt + R,
  // its loads spread between the rows, while stage kt + 1's first k-step is read.
  // The last stage re-reads its own buffer instead (valid, unused).  The
  // scheduling barriers keep this order.
  auto stage = [&](int kt, u32x4_t (&c)[NF], u32x4_t (&n)[NF]) {
    const bool more = kt + 1 < k_tiles;
    const int cb = kt % R, nb = (more ? kt + 1 : kt) % R;
#pragma unroll
    for (int ksi = 0; ksi + 1 < 2 * SP; ++ksi) {
      u32x4_t (&cur)[NF] = (ksi & 1) ? n : c;
      u32x4_t (&nxt)[NF] = (ksi & 1) ? c : n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mfma_row(cur, i);
        __builtin_amdgcn_sched_barrier(0);
        read_pair(cb, ksi + 1, nxt, 2 * i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) sync_stage(kt);
    const bool refill = kt + R < k_tiles;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (refill) issue_part(kt + R, cb, i);
      __builtin_amdgcn_sched_barrier(0);
      mfma_row(n, i);
      __builtin_amdgcn_sched_barrier(0);
      read_pair(nb, 0, c, 2 * i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < k_tiles; ++kt) stage(kt, fc, fn);
  __syncthreads();  // the ring is reused by the epilogue

  if (split) {
    // Park this half's sums (write-through stores: complete at the device
    // coherence point once counted), count the workgroup in; the second to
    // arrive reads the other half's sums with coherent loads and goes on.  The
    // ordering rests on the emitted code (sc1 stores and loads, the wait and the
    // barrier before the counter), which tests/test_handoff_asm.py checks, not on
    // relaxed atomics' language semantics.
    __shared__ int s_second;
    constexpr int NV = 4 * WNB * 8;  // 64-bit pairs of sums per thread
    uint64_t *mine = split_buf + (static_cast<int64_t>(pair) * 2 + khalf) * (NW * 64 * NV);
    uint64_t *other = split_buf + (static_cast<int64_t>(pair) * 2 + (khalf ^ 1)) * (NW * 64 * NV);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < WNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint64_t v = static_cast<uint64_t>(__float_as_uint(acc[i][j][r])) |
                             (static_cast<uint64_t>(__float_as_uint(acc[i][j][r + 1])) << 32);
          __hip_atomic_store(&mine[((i * WNB + j) * 8 + r / 2) * (NW * 64) + tid], v,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(&split_cnt[pair], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      s_second = old == 1;
      if (old == 1)  // both halves in: reset for the next call
        __hip_atomic_store(&split_cnt[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_second) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < WNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint64_t v = __hip_atomic_load(&other[((i * WNB + j) * 8 + r / 2) * (NW * 64) + tid],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          acc[i][j][r] += __uint_as_float(static_cast<uint32_t>(v));
          acc[i][j][r + 1] += __uint_as_float(static_cast<uint32_t>(v >> 32));
        }
  }

  // Epilogue.
  if constexpr (HIDDEN) {
    // h of the wave's 128 rows, FP features per pass, staged through LDS (free
    // after the last barrier of the main loop), then written as 16-byte chunks
    // of the packed hidden buffer.
    constexpr int JW = (EPI == EPI_SILU_GATE) ? 16 : 32;  // features per column block
    constexpr int FP = NW == 4 ? 64 : 32;                 // features per pass (LDS fits)
    constexpr int BPP = FP / JW < WNB ? FP / JW : WNB;    // column blocks per pass
    constexpr int FPP = BPP * JW;                         // features per pass
    constexpr int HS = FPP + 8;                           // LDS row stride (bf16)
    uint16_t *hs = reinterpret_cast<uint16_t *>(&lds[0][0][0]) + wave * (128 * HS);
#pragma unroll
    for (int pass = 0; pass < WNB / BPP; ++pass) {
#pragma unroll
      for (int jj = 0; jj < BPP; ++jj) {
        const int j = pass * BPP + jj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int R_ = i * 32 + mfma32_row(r, lane);
            const int c = lane & 31;
            const float v = acc[i][j][r];
            if constexpr (EPI == EPI_SILU_GATE) {
              const float u = __shfl_xor(v, 16);
              if (c < 16) hs[R_ * HS + jj * 16 + c] = f32_to_bf16(silu_f(v) * u);
            } else {
              hs[R_ * HS + jj * 32 + c] = f32_to_bf16(act_f<EPI>(v));
            }
          }
        }
      }
      __syncthreads();
      const int f0 = (tn * 8 + wn * WNB + pass * BPP) * JW;  // first feature of this pass
#pragma unroll
      for (int q = lane; q < 128 * (FPP / 8); q += 64) {
        const int R_ = q & 127, qc = q >> 7;
        const int jf = f0 + 8 * qc;
        const int s = 2 * (jf >> 5) + ((jf >> 3) & 1);
        const int row = hrow0 + wm * 128 + R_;
        const int ln = 32 * ((jf >> 4) & 1) + (row & 31);
        const int64_t chunk = (static_cast<int64_t>(row >> 5) * ks_out + s) * 64 + ln;
        static_cast<u32x4_t *>(out)[chunk] = *reinterpret_cast<const u32x4_t *>(&hs[R_ * HS + 8 * qc]);
      }
      if (pass + 1 < WNB / BPP) __syncthreads();
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + (wm * 4 + i) * 32 + mfma32_row(r, lane);
        if (row >= row_end) continue;
#pragma unroll
        for (int j = 0; j < WNB; ++j) {
          const int col = (tn * 8 + wn * WNB + j) * 32 + (lane & 31);
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

// The configuration the library launches.
constexpr int kTiledSP = 2;
constexpr int kTiledWaves = 8;
constexpr int kTiledRing = 2;

int tiled_split_tiles(int64_t tiles, int n_cu, int max_tiles) {
  if (n_cu <= 0) return 0;
  const int64_t rem = tiles % n_cu;
  return (rem > 0 && 2 * rem <= n_cu && rem <= max_tiles && rem <= kTiledMaxSplit)
             ? static_cast<int>(rem)
             : 0;
}

template <int EPI, int SP = kTiledSP, int NW = kTiledWaves, int RING = kTiledRing>
static hipError_t launch_tiled_one(const void *A, int64_t lda, int64_t M, int64_t K, const void *W,
                                   int64_t n_packed, void *out, int64_t ldo, int64_t n_store,
                                   int64_t ks_out, const TiledSplit &sp, const TiledGroups &grp,
                                   hipStream_t s, const Timing &t) {
  // grouped: every group may add one partial row tile
  const int ntm = static_cast<int>((M + kTileM - 1) / kTileM) + grp.n_groups;
  const int ntn = static_cast<int>(n_packed / kTileN);
  if (K % (32 * SP)) return hipErrorInvalidValue;
  const int k_total = static_cast<int>(K / (32 * SP));
  const int split = (grp.n_groups == 0 && sp.buf && sp.cnt && k_total >= 2 * RING)
                        ? tiled_split_tiles(static_cast<int64_t>(ntm) * ntn, sp.n_cu, sp.max_tiles)
                        : 0;
  const int n_whole = ntm * ntn - split;
  auto kern = grp.n_groups > 0 ? k_tiled<EPI, SP, NW, RING, true> : k_tiled<EPI, SP, NW, RING, false>;
  hipExtLaunchKernelGGL(kern, dim3(n_whole + 2 * split), dim3(NW * 64), 0, s, t.start, t.stop, 0,
                        static_cast<const uint16_t *>(A), lda, static_cast<int>(M), k_total,
                        static_cast<const u32x4_t *>(W), static_cast<int>(K / kFragK), ntm, ntn,
                        out, ldo, static_cast<int>(n_store), static_cast<int>(ks_out), n_whole,
                        static_cast<uint64_t *>(sp.buf), sp.cnt, grp);
  return hipGetLastError();
}

hipError_t launch_tiled_gemm(int epi, const void *A, int64_t lda, int64_t M, int64_t K,
                             const void *W, int64_t n_packed, void *out, int64_t ldo,
                             int64_t n_store, int64_t ks_out, const TiledSplit &sp, hipStream_t s,
                             const Timing &t, const TiledGroups &grp) {
  switch (epi) {
    case EPI_SILU_GATE:
      return launch_tiled_one<EPI_SILU_GATE>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    case EPI_TANH:
      return launch_tiled_one<EPI_TANH>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    case EPI_IDENTITY:
      return launch_tiled_one<EPI_IDENTITY>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    case EPI_OUT_F32:
      return launch_tiled_one<EPI_OUT_F32>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    case EPI_OUT_BF16:
      return launch_tiled_one<EPI_OUT_BF16>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    case EPI_PROJ_F32:
      return launch_tiled_one<EPI_PROJ_F32>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    case EPI_PROJ_BF16:
      return launch_tiled_one<EPI_PROJ_BF16>(A, lda, M, K, W, n_packed, out, ldo, n_store, ks_out, sp, grp, s, t);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tpm
