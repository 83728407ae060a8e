// C ABI of libtpmlp: argument checks, handle lifetime, kernel choice.
//
// Every argument is checked on the host before anything is enqueued, so a call
// that fails has no effect on the device.  fwd makes exactly two launches (first
// projection with its fused activation, then the second projection), allocates
// nothing and never synchronizes, so it can be captured in a HIP graph.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "tpm_internal.h"

using namespace tpm;

namespace {

constexpr int64_t kAlign = 16;
constexpr int64_t kSubAlign = 256;
constexpr int kMaxParts = 16;

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

tpm_status check_desc(const tpm_desc *d) {
  if (!d) return TPM_ERR_INVALID_ARG;
  if (d->act < TPM_ACT_TANH || d->act > TPM_ACT_IDENTITY) return TPM_ERR_INVALID_ARG;
  if (d->in_dtype != TPM_F32 && d->in_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (d->out_dtype != TPM_F32 && d->out_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (d->path < TPM_PATH_AUTO || d->path > TPM_PATH_TILED) return TPM_ERR_INVALID_ARG;
  if (d->d_model < 1 || d->ffn_shard < 1 || d->max_tokens < 0) return TPM_ERR_SHAPE;
  // Keep every index the kernels form inside 32-bit ints and every size sane.
  if (d->d_model > (int64_t(1) << 20) || d->ffn_shard > (int64_t(1) << 20) ||
      d->max_tokens > (int64_t(1) << 24))
    return TPM_ERR_SHAPE;
  if (d->in_dtype == TPM_BF16 && d->d_model % 64 != 0) return TPM_ERR_SHAPE;
  return TPM_OK;
}

int first_epi(int act) {
  return act == TPM_ACT_SILU_GATE ? EPI_SILU_GATE : act == TPM_ACT_TANH ? EPI_TANH : EPI_IDENTITY;
}

tpm_status from_hip(hipError_t e) {
  if (e == hipSuccess) return TPM_OK;
  if (e == hipErrorOutOfMemory) return TPM_ERR_OOM;
  return TPM_ERR_HIP;
}

// Scratch of tp_mlp_shard_fwd_noalloc: one array per device, held from module load
// to process end.  In host code `scratch` only names the symbol; its device address
// comes from hipGetSymbolAddress (per device, at the first call there) and only that
// address is ever passed to kernels.
constexpr int64_t kNoAllocScratchBytes = TPM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

tpm_status scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return TPM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return TPM_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TPM_OK;
}

}  // namespace

namespace tpm {

Sizes compute_sizes(const tpm_desc &d) {
  Sizes z = {};
  const int64_t F = d.ffn_shard, D = d.d_model;
  const bool silu = d.act == TPM_ACT_SILU_GATE;
  if (d.in_dtype == TPM_BF16) {
    z.ffn_pad = silu ? round_up(F, kTileN / 2) : round_up(F, kTileN);
    z.n1 = silu ? 2 * z.ffn_pad : z.ffn_pad;
    z.n2 = round_up(D, kTileN);
    z.w1_bytes = z.n1 * D * 2;
    z.w2_bytes = z.n2 * z.ffn_pad * 2;
    z.hidden_bytes = round_up(d.max_tokens, kHiddenRowPad) * z.ffn_pad * 2;
    // Streaming-path scratch: the largest need over the token counts that run on
    // one token group (M <= 64), for both products (they run one after the other).
    const int64_t tok[2] = {32, 64};
    for (int i = 0; i < 2; ++i) {
      if (d.max_tokens < tok[i] - 31) break;
      const StreamPlan p1 = stream_plan(tok[i], z.n1 / kFragN, D / kFragK);
      const StreamPlan p2 = stream_plan(tok[i], z.n2 / kFragN, z.ffn_pad / kFragK);
      const int64_t f1 = p1.s > 1 ? (z.n1 / kFragN) * p1.s * p1.mt * 1024 : 0;
      const int64_t f2 = p2.s > 1 ? (z.n2 / kFragN) * p2.s * p2.mt * 1024 : 0;
      const int64_t c1 = p1.s > 1 ? z.n1 / kFragN / p1.c : 0;
      const int64_t c2 = p2.s > 1 ? z.n2 / kFragN / p2.c : 0;
      if (f1 > z.scratch_floats) z.scratch_floats = f1;
      if (f2 > z.scratch_floats) z.scratch_floats = f2;
      if (c1 > z.n_counters) z.n_counters = c1;
      if (c2 > z.n_counters) z.n_counters = c2;
    }
    // Tiled-path scratch: the fp32 sums of the contraction halves of a split last
    // round (at most kTiledMaxSplit tiles, never more than the tiles there are).
    const bool tiled = d.path == TPM_PATH_TILED ||
                       (d.path == TPM_PATH_AUTO && d.max_tokens > kStreamMaxTokens);
    if (tiled) {
      const int64_t tm = (d.max_tokens + kTileM - 1) / kTileM;
      int64_t tiles = tm * (z.n1 > z.n2 ? z.n1 : z.n2) / kTileN;
      if (tiles > kTiledMaxSplit) tiles = kTiledMaxSplit;
      const int64_t f = 2 * tiles * kTileM * kTileN;
      if (f > z.scratch_floats) z.scratch_floats = f;
      if (tiles > z.n_counters) z.n_counters = tiles;
      z.split_tiles = tiles;
    }
  } else {
    z.ffn_pad = F;
    z.n1 = silu ? 2 * F : F;
    z.n2 = D;
    z.w1_bytes = z.n1 * D * 4;
    z.w2_bytes = F * D * 4;
    z.hidden_bytes = d.max_tokens * F * 4;
  }
  return z;
}

}  // namespace tpm

extern "C" {

const char *tpm_status_str(tpm_status s) {
  switch (s) {
    case TPM_OK: return "ok";
    case TPM_ERR_INVALID_ARG: return "invalid argument (null pointer or enum out of range)";
    case TPM_ERR_SHAPE: return "unsupported shape or size out of range";
    case TPM_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case TPM_ERR_HIP: return "HIP runtime error";
    case TPM_ERR_OOM: return "device out of memory";
    default: return "unknown status";
  }
}

tpm_status tp_mlp_shard_plan(const tpm_desc *desc, tpm_plan_info *out) {
  if (!out) return TPM_ERR_INVALID_ARG;
  const tpm_status st = check_desc(desc);
  if (st != TPM_OK) return st;
  const Sizes z = compute_sizes(*desc);
  tpm_plan_info info = {};
  info.packed_weight_bytes = z.w1_bytes + z.w2_bytes;
  info.workspace_bytes = z.hidden_bytes + z.scratch_floats * 4 + z.n_counters * 4;
  info.ffn_padded = z.ffn_pad;
  info.stream_max_tokens = desc->in_dtype == TPM_BF16 ? kStreamMaxTokens : 0;
  info.kernels_per_fwd = 2;
  *out = info;
  return TPM_OK;
}

tpm_status tp_mlp_shard_create(const tpm_desc *desc, const void *A_dev, const void *B_dev,
                               void *stream, tpm_shard_t *out) {
  if (!out) return TPM_ERR_INVALID_ARG;
  *out = nullptr;
  tpm_status st = check_desc(desc);
  if (st != TPM_OK) return st;
  if (!A_dev || !B_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(A_dev) || !aligned(B_dev)) return TPM_ERR_ALIGN;

  const tpm_desc d = *desc;
  const Sizes z = compute_sizes(d);
  Shard *h = new (std::nothrow) Shard();
  if (!h) return TPM_ERR_OOM;
  h->desc = d;
  h->ffn_pad = z.ffn_pad;
  h->n1 = z.n1;
  h->n2 = z.n2;
  h->ks1 = d.d_model / kFragK;
  h->ks2 = z.ffn_pad / kFragK;
  h->split_tiles = static_cast<int>(z.split_tiles);
  h->n_events = 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&h->device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&h->n_cu, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess) {
    delete h;
    return from_hip(e);
  }
  const int64_t o_w1 = 0;
  const int64_t o_w2 = round_up(o_w1 + z.w1_bytes, kSubAlign);
  const int64_t o_hid = round_up(o_w2 + z.w2_bytes, kSubAlign);
  const int64_t o_sk = round_up(o_hid + z.hidden_bytes, kSubAlign);
  const int64_t o_cnt = round_up(o_sk + z.scratch_floats * 4, kSubAlign);
  const int64_t total = round_up(o_cnt + z.n_counters * 4, kSubAlign);
  e = hipMalloc(&h->alloc_base, static_cast<size_t>(total));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return TPM_ERR_OOM;
  }
  char *base = static_cast<char *>(h->alloc_base);
  h->alloc_bytes = total;
  h->w1 = base + o_w1;
  h->w2 = base + o_w2;
  h->hidden = z.hidden_bytes ? base + o_hid : nullptr;
  h->scratch = z.scratch_floats ? reinterpret_cast<float *>(base + o_sk) : nullptr;
  h->counters = z.n_counters ? reinterpret_cast<int *>(base + o_cnt) : nullptr;
  h->scratch_floats = z.scratch_floats;
  h->n_counters = z.n_counters;

  const bool silu = d.act == TPM_ACT_SILU_GATE;
  const int64_t a_cols = silu ? 2 * d.ffn_shard : d.ffn_shard;
  if (d.in_dtype == TPM_BF16) {
    e = launch_pack_bf16(A_dev, a_cols, d.d_model, a_cols, silu, d.ffn_shard, z.n1 / kFragN,
                         h->ks1, h->w1, s);
    if (e == hipSuccess)
      e = launch_pack_bf16(B_dev, d.d_model, d.ffn_shard, d.d_model, false, d.ffn_shard,
                           z.n2 / kFragN, h->ks2, h->w2, s);
    if (e == hipSuccess) e = launch_zero_i32(h->counters, z.n_counters, s);
  } else {
    e = hipMemcpyAsync(h->w1, A_dev, static_cast<size_t>(z.w1_bytes), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(h->w2, B_dev, static_cast<size_t>(z.w2_bytes), hipMemcpyDeviceToDevice, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(h->alloc_base);
    delete h;
    return from_hip(e);
  }
  *out = reinterpret_cast<tpm_shard_t>(h);
  return TPM_OK;
}

tpm_status tp_mlp_shard_fwd(tpm_shard_t handle, const void *X_dev, int64_t M, void *partial_dev,
                            void *stream) {
  Shard *h = reinterpret_cast<Shard *>(handle);
  if (!h) return TPM_ERR_INVALID_ARG;
  const tpm_desc &d = h->desc;
  if (M < 0 || M > d.max_tokens) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X_dev || !partial_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(X_dev) || !aligned(partial_dev)) return TPM_ERR_ALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return TPM_ERR_INVALID_ARG;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int epi1 = first_epi(d.act);
  const int epi2 = d.out_dtype == TPM_F32 ? EPI_OUT_F32 : EPI_OUT_BF16;
  Timing t1, t2;
  if (h->n_events >= 4) {
    t1.start = h->events[0];
    t1.stop = h->events[1];
    t2.start = h->events[2];
    t2.stop = h->events[3];
  }
  hipError_t e = hipSuccess;

  if (d.in_dtype == TPM_F32) {
    const int64_t a_cols = d.act == TPM_ACT_SILU_GATE ? 2 * d.ffn_shard : d.ffn_shard;
    e = launch_f32_gemm(epi1, static_cast<const float *>(X_dev), d.d_model, M, d.d_model,
                        static_cast<const float *>(h->w1), a_cols, d.ffn_shard, d.ffn_shard,
                        h->hidden, d.ffn_shard, s, t1);
    if (e == hipSuccess)
      e = launch_f32_gemm(epi2, static_cast<const float *>(h->hidden), d.ffn_shard, M,
                          d.ffn_shard, static_cast<const float *>(h->w2), d.d_model, d.d_model, 0,
                          partial_dev, d.d_model, s, t2);
    return from_hip(e);
  }

  int path = d.path;
  if (path == TPM_PATH_AUTO) path = M <= kStreamMaxTokens ? TPM_PATH_STREAM : TPM_PATH_TILED;
  StreamScratch ws;
  ws.buf = h->scratch;
  ws.cnt = h->counters;
  ws.floats = h->scratch_floats;
  ws.n_counters = h->n_counters;
  // decode path: the second product may add two contraction halves atomically into
  // the partial, which the first product then clears as a side job
  const StreamPlan p2 = stream_plan_out(M, h->n2 / kFragN, h->ks2, d.out_dtype == TPM_F32);
  StreamZero zero;
  if (p2.atom) {
    zero.out = static_cast<float *>(partial_dev);
    zero.n = M * d.d_model;
  }
  if (path == TPM_PATH_STREAM)
    e = launch_stream_gemm(epi1, stream_plan(M, h->n1 / kFragN, h->ks1), X_dev, d.d_model, M,
                           h->ks1, h->w1, h->n1 / kFragN, h->hidden, 0, 0, h->ks2, ws, s, t1, zero);
  TiledSplit split;
  if (h->scratch && h->counters && h->split_tiles > 0) {
    split.buf = h->scratch;
    split.cnt = h->counters;
    split.n_cu = h->n_cu;
    split.max_tiles = h->split_tiles;
  }
  if (path == TPM_PATH_TILED)
    e = launch_gemm(epi1, X_dev, d.d_model, M, d.d_model, h->w1, h->n1, h->hidden, 0, 0,
                          h->ks2, split, s, t1);
  if (e == hipSuccess) {
    if (path == TPM_PATH_STREAM)
      e = launch_stream_gemm(epi2, p2, h->hidden, 0, M, h->ks2, h->w2, h->n2 / kFragN, partial_dev,
                             d.d_model, d.d_model, 0, ws, s, t2);
    else
      e = launch_gemm(epi2, h->hidden, 0, M, h->ffn_pad, h->w2, h->n2, partial_dev,
                            d.d_model, d.d_model, 0, split, s, t2);
  }
  return from_hip(e);
}

tpm_status tp_mlp_shard_fwd_noalloc(tpm_shard_t handle, const void *X_dev, int64_t M,
                                    void *partial_dev, void *stream) {
  Shard *h = reinterpret_cast<Shard *>(handle);
  if (!h) return TPM_ERR_INVALID_ARG;
  const tpm_desc &d = h->desc;
  if (d.in_dtype != TPM_BF16 || M < 0 || M > kStreamMaxTokens) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X_dev || !partial_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(X_dev) || !aligned(partial_dev)) return TPM_ERR_ALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return TPM_ERR_INVALID_ARG;

  // Carve the scratch: the packed hidden rows of the token tiles, then the
  // contraction slices' sums and arrival counters (the larger need of the two
  // products, which run one after the other).
  const StreamPlan p1 = stream_plan(M, h->n1 / kFragN, h->ks1);
  const StreamPlan p2 = stream_plan_out(M, h->n2 / kFragN, h->ks2, d.out_dtype == TPM_F32);
  const int64_t hidden_bytes = (M + 31) / 32 * h->ks2 * 1024;
  const int64_t f1 = p1.s > 1 ? (h->n1 / kFragN) * p1.s * p1.mt * 1024 : 0;
  const int64_t f2 = p2.s > 1 && !p2.atom ? (h->n2 / kFragN) * p2.s * p2.mt * 1024 : 0;
  const int64_t c1 = p1.s > 1 ? h->n1 / kFragN / p1.c : 0;
  const int64_t c2 = p2.s > 1 && !p2.atom ? h->n2 / kFragN / p2.c : 0;
  const int64_t floats = f1 > f2 ? f1 : f2;
  const int64_t n_cnt = c1 > c2 ? c1 : c2;
  const int64_t o_sk = round_up(hidden_bytes, kSubAlign);
  const int64_t o_cnt = round_up(o_sk + floats * 4, kSubAlign);
  const int64_t need = o_cnt + n_cnt * 4;
  if (need > kNoAllocScratchBytes) return TPM_ERR_SHAPE;
  void *base = nullptr;
  const tpm_status st = scratch_address(dev, &base);
  if (st != TPM_OK) return st;
  char *b = static_cast<char *>(base);
  StreamScratch ws;
  ws.buf = floats ? reinterpret_cast<float *>(b + o_sk) : nullptr;
  ws.cnt = n_cnt ? reinterpret_cast<int *>(b + o_cnt) : nullptr;
  ws.floats = floats;
  ws.n_counters = n_cnt;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int epi1 = first_epi(d.act);
  const int epi2 = d.out_dtype == TPM_F32 ? EPI_OUT_F32 : EPI_OUT_BF16;
  // the arrival counters must start at zero (a fill kernel, so a caller may capture it)
  hipError_t e = n_cnt ? launch_zero_i32(ws.cnt, n_cnt, s) : hipSuccess;
  StreamZero zero;
  if (p2.atom) {
    zero.out = static_cast<float *>(partial_dev);
    zero.n = M * d.d_model;
  }
  if (e == hipSuccess)
    e = launch_stream_gemm(epi1, p1, X_dev, d.d_model, M, h->ks1, h->w1, h->n1 / kFragN, b, 0, 0,
                           h->ks2, ws, s, Timing(), zero);
  if (e == hipSuccess)
    e = launch_stream_gemm(epi2, p2, b, 0, M, h->ks2, h->w2, h->n2 / kFragN, partial_dev,
                           d.d_model, d.d_model, 0, ws, s);
  return from_hip(e);
}

tpm_status tp_partials_reduce(const void *const *partials_dev, int32_t k, int64_t numel,
                              int32_t in_dtype, void *out_dev, int32_t out_dtype, void *stream) {
  if (!partials_dev || !out_dev) return TPM_ERR_INVALID_ARG;
  if (in_dtype != TPM_F32 && in_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (out_dtype != TPM_F32 && out_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxParts || numel < 0) return TPM_ERR_SHAPE;
  for (int i = 0; i < k; ++i) {
    if (!partials_dev[i]) return TPM_ERR_INVALID_ARG;
    if (!aligned(partials_dev[i])) return TPM_ERR_ALIGN;
  }
  if (!aligned(out_dev)) return TPM_ERR_ALIGN;
  if (out_dev == partials_dev[0] && in_dtype != out_dtype) return TPM_ERR_INVALID_ARG;
  if (numel == 0) return TPM_OK;
  return from_hip(launch_reduce(partials_dev, k, numel, in_dtype, out_dev, out_dtype,
                                static_cast<hipStream_t>(stream)));
}

tpm_status tp_partials_reduce_add_rmsnorm(const void *const *partials_dev, int32_t k,
                                          int64_t rows, int64_t cols, int32_t in_dtype,
                                          const void *residual_dev, void *residual_out_dev,
                                          int32_t res_dtype, const void *gamma_dev, float eps,
                                          void *y_dev, int32_t out_dtype, void *stream) {
  if (!partials_dev || !residual_dev || !residual_out_dev || !gamma_dev || !y_dev)
    return TPM_ERR_INVALID_ARG;
  for (int32_t t : {in_dtype, res_dtype, out_dtype})
    if (t != TPM_F32 && t != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return TPM_ERR_INVALID_ARG;  // rejects NaN and inf
  if (k < 1 || k > kMaxParts || rows < 0 || rows > 0x7fffffff) return TPM_ERR_SHAPE;
  if (cols < 8 || cols % 8 || cols > kNormMaxCols) return TPM_ERR_SHAPE;
  for (int i = 0; i < k; ++i) {
    if (!partials_dev[i]) return TPM_ERR_INVALID_ARG;
    if (!aligned(partials_dev[i])) return TPM_ERR_ALIGN;
  }
  if (!aligned(residual_dev) || !aligned(residual_out_dev) || !aligned(gamma_dev) ||
      !aligned(y_dev))
    return TPM_ERR_ALIGN;
  if (rows == 0) return TPM_OK;
  return from_hip(launch_reduce_norm(partials_dev, k, rows, cols, in_dtype, residual_dev,
                                     residual_out_dev, res_dtype, gamma_dev, eps, y_dev,
                                     out_dtype, static_cast<hipStream_t>(stream)));
}

tpm_status tp_partials_quantize_fp8(const void *partial_dev, int64_t rows, int64_t cols,
                                    int32_t in_dtype, void *q_dev, float *scale_dev,
                                    void *stream) {
  if (!partial_dev || !q_dev || !scale_dev) return TPM_ERR_INVALID_ARG;
  if (in_dtype != TPM_F32 && in_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (rows < 0 || rows > 0x7fffffff || cols < 16 || cols % 16 || cols > kFp8MaxCols)
    return TPM_ERR_SHAPE;
  if (!aligned(partial_dev) || !aligned(q_dev) || !aligned(scale_dev)) return TPM_ERR_ALIGN;
  if (rows == 0) return TPM_OK;
  return from_hip(launch_quant_fp8(partial_dev, rows, cols, in_dtype, q_dev, scale_dev,
                                   static_cast<hipStream_t>(stream)));
}

tpm_status tp_partials_reduce_fp8(const void *const *q_dev, const float *const *scale_dev,
                                  int32_t k, int64_t rows, int64_t cols, void *out_dev,
                                  int32_t out_dtype, void *stream) {
  if (!q_dev || !scale_dev || !out_dev) return TPM_ERR_INVALID_ARG;
  if (out_dtype != TPM_F32 && out_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxParts || rows < 0 || cols < 16 || cols % 16 ||
      rows > (int64_t(1) << 40) / cols)
    return TPM_ERR_SHAPE;
  for (int i = 0; i < k; ++i) {
    if (!q_dev[i] || !scale_dev[i]) return TPM_ERR_INVALID_ARG;
    if (!aligned(q_dev[i])) return TPM_ERR_ALIGN;
  }
  if (!aligned(out_dev)) return TPM_ERR_ALIGN;
  if (rows == 0) return TPM_OK;
  return from_hip(launch_reduce_fp8(q_dev, scale_dev, k, rows, cols, out_dev, out_dtype,
                                    static_cast<hipStream_t>(stream)));
}

tpm_status tp_attn_partials_merge(const void *const *values_dev, const float *const *max_dev,
                                  const float *const *expsum_dev, int32_t k, int64_t rows,
                                  int64_t dim, int32_t in_dtype, void *out_dev, int32_t out_dtype,
                                  float *max_out_dev, float *expsum_out_dev, void *stream) {
  if (!values_dev || !max_dev || !expsum_dev || !out_dev) return TPM_ERR_INVALID_ARG;
  if (in_dtype != TPM_F32 && in_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (out_dtype != TPM_F32 && out_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (!max_out_dev != !expsum_out_dev) return TPM_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxParts || rows < 0 || dim < 8 || dim % 8 || dim > (int64_t(1) << 20) ||
      rows > (int64_t(1) << 40) / dim)
    return TPM_ERR_SHAPE;
  auto stat_aligned = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 4 == 0; };
  for (int i = 0; i < k; ++i) {
    if (!values_dev[i] || !max_dev[i] || !expsum_dev[i]) return TPM_ERR_INVALID_ARG;
    if (!aligned(values_dev[i]) || !stat_aligned(max_dev[i]) || !stat_aligned(expsum_dev[i]))
      return TPM_ERR_ALIGN;
    if (max_out_dev && (max_out_dev == max_dev[i] || expsum_out_dev == expsum_dev[i] ||
                        max_out_dev == expsum_dev[i] || expsum_out_dev == max_dev[i]))
      return TPM_ERR_INVALID_ARG;
  }
  if (!aligned(out_dev)) return TPM_ERR_ALIGN;
  if (max_out_dev && (!stat_aligned(max_out_dev) || !stat_aligned(expsum_out_dev)))
    return TPM_ERR_ALIGN;
  if (out_dev == values_dev[0] && in_dtype != out_dtype) return TPM_ERR_INVALID_ARG;
  if (rows == 0) return TPM_OK;
  return from_hip(launch_attn_merge(values_dev, max_dev, expsum_dev, k, rows, dim, in_dtype,
                                    out_dev, out_dtype, max_out_dev, expsum_out_dev,
                                    static_cast<hipStream_t>(stream)));
}

tpm_status tp_mlp_shard_destroy(tpm_shard_t handle) {
  Shard *h = reinterpret_cast<Shard *>(handle);
  if (!h) return TPM_OK;
  hipError_t e = hipDeviceSynchronize();
  const hipError_t e2 = hipFree(h->alloc_base);
  if (e == hipSuccess) e = e2;
  delete h;
  return from_hip(e);
}

tpm_status tp_mlp_shard_set_timing_events(tpm_shard_t handle, void *const *events,
                                          int32_t n_events) {
  Shard *h = reinterpret_cast<Shard *>(handle);
  if (!h) return TPM_ERR_INVALID_ARG;
  if (!events) {
    if (n_events != 0) return TPM_ERR_INVALID_ARG;
    h->n_events = 0;
    return TPM_OK;
  }
  if (n_events < 4) return TPM_ERR_SHAPE;
  for (int i = 0; i < 4; ++i) {
    if (!events[i]) return TPM_ERR_INVALID_ARG;
    h->events[i] = static_cast<hipEvent_t>(events[i]);
  }
  h->n_events = 4;
  return TPM_OK;
}

}  // extern "C"
