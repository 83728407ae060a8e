// C ABI of single tensor-parallel projections, Y = X W on one rank's shard of W.
//
// Page "大模型推理系统揭秘（07）Multi-GPU", section 1.2.4: in the attention block
// the Q, K and V projections are column-parallel (each GPU owns some heads), the
// attention itself is local, and the output projection is row-parallel, its rank
// partials closed by one all-reduce.  The attention core sits between the two
// projections, so each runs as its own call here: the column shard of [Wq|Wk|Wv]
// (bf16 output for the local attention), and the row shard of Wo (fp32 partial
// for tp_partials_reduce).  Same kernels as the MLP's products, with the token
// operand row-major on input and the result row-major on output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>

#include "tpm_internal.h"

using namespace tpm;

namespace {

constexpr int64_t kAlign = 16;

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

tpm_status from_hip(hipError_t e) {
  if (e == hipSuccess) return TPM_OK;
  if (e == hipErrorOutOfMemory) return TPM_ERR_OOM;
  return TPM_ERR_HIP;
}

struct Proj {
  tpm_proj_desc desc;
  int device;
  int n_cu;
  int64_t n_pad;     // output columns padded to the tile width (bf16 path)
  int64_t ks;        // k-steps (in_features / 16)
  void *w;           // packed W (bf16) or a copy (fp32)
  float *scratch;    // contraction slices (streaming) / split halves (tiled)
  int *counters;     // arrival counters, zero between calls
  int64_t scratch_floats, n_counters;  // room in scratch and counters
  int split_tiles;
  void *alloc_base;
};

struct ProjSizes {
  int64_t n_pad, w_bytes, scratch_floats, n_counters, split_tiles;
};

tpm_status check_proj_desc(const tpm_proj_desc *d) {
  if (!d) return TPM_ERR_INVALID_ARG;
  if (d->in_dtype != TPM_F32 && d->in_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (d->out_dtype != TPM_F32 && d->out_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (d->path < TPM_PATH_AUTO || d->path > TPM_PATH_TILED) return TPM_ERR_INVALID_ARG;
  if (d->in_features < 1 || d->out_features < 1 || d->max_tokens < 0) return TPM_ERR_SHAPE;
  if (d->in_features > (int64_t(1) << 20) || d->out_features > (int64_t(1) << 20) ||
      d->max_tokens > (int64_t(1) << 24))
    return TPM_ERR_SHAPE;
  if (d->in_dtype == TPM_BF16 && d->in_features % 64 != 0) return TPM_ERR_SHAPE;
  return TPM_OK;
}

ProjSizes proj_sizes(const tpm_proj_desc &d) {
  ProjSizes z = {};
  if (d.in_dtype != TPM_BF16) {
    z.w_bytes = d.in_features * d.out_features * 4;
    return z;
  }
  z.n_pad = round_up(d.out_features, kTileN);
  z.w_bytes = z.n_pad * d.in_features * 2;
  const int64_t n_cb = z.n_pad / kFragN, ks = d.in_features / kFragK;
  const bool stream = d.path == TPM_PATH_STREAM || d.path == TPM_PATH_AUTO;
  const bool tiled = d.path == TPM_PATH_TILED ||
                     (d.path == TPM_PATH_AUTO && d.max_tokens > kStreamMaxTokens);
  if (stream) {
    const int64_t tok[2] = {32, 64};
    for (int i = 0; i < 2; ++i) {
      if (d.max_tokens < tok[i] - 31) break;
      const StreamPlan p = stream_plan(tok[i], n_cb, ks);
      if (p.s > 1) {
        const int64_t f = n_cb * p.s * p.mt * 1024, c = n_cb / p.c;
        if (f > z.scratch_floats) z.scratch_floats = f;
        if (c > z.n_counters) z.n_counters = c;
      }
    }
  }
  if (tiled) {
    int64_t tiles = (d.max_tokens + kTileM - 1) / kTileM * (z.n_pad / kTileN);
    if (tiles > kTiledMaxSplit) tiles = kTiledMaxSplit;
    const int64_t f = 2 * tiles * kTileM * kTileN;
    if (f > z.scratch_floats) z.scratch_floats = f;
    if (tiles > z.n_counters) z.n_counters = tiles;
    z.split_tiles = tiles;
  }
  return z;
}

}  // namespace

extern "C" {

tpm_status tp_proj_create(const tpm_proj_desc *desc, const void *W_dev, void *stream,
                          tpm_proj_t *out) {
  if (!out) return TPM_ERR_INVALID_ARG;
  *out = nullptr;
  tpm_status st = check_proj_desc(desc);
  if (st != TPM_OK) return st;
  if (!W_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(W_dev)) return TPM_ERR_ALIGN;
  const tpm_proj_desc d = *desc;
  const ProjSizes z = proj_sizes(d);
  Proj *h = new (std::nothrow) Proj();
  if (!h) return TPM_ERR_OOM;
  h->desc = d;
  h->n_pad = z.n_pad;
  h->ks = d.in_features / kFragK;
  h->split_tiles = static_cast<int>(z.split_tiles);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&h->device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&h->n_cu, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess) {
    delete h;
    return from_hip(e);
  }
  constexpr int64_t kSub = 256;
  const int64_t o_sk = round_up(z.w_bytes, kSub);
  const int64_t o_cnt = round_up(o_sk + z.scratch_floats * 4, kSub);
  const int64_t total = round_up(o_cnt + z.n_counters * 4, kSub);
  e = hipMalloc(&h->alloc_base, static_cast<size_t>(total));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return TPM_ERR_OOM;
  }
  char *base = static_cast<char *>(h->alloc_base);
  h->w = base;
  h->scratch = z.scratch_floats ? reinterpret_cast<float *>(base + o_sk) : nullptr;
  h->counters = z.n_counters ? reinterpret_cast<int *>(base + o_cnt) : nullptr;
  h->scratch_floats = z.scratch_floats;
  h->n_counters = z.n_counters;
  if (d.in_dtype == TPM_BF16) {
    e = launch_pack_bf16(W_dev, d.out_features, d.in_features, d.out_features, false,
                         d.out_features, z.n_pad / kFragN, h->ks, h->w, s);
    if (e == hipSuccess) e = launch_zero_i32(h->counters, z.n_counters, s);
  } else {
    e = hipMemcpyAsync(h->w, W_dev, static_cast<size_t>(z.w_bytes), hipMemcpyDeviceToDevice, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(h->alloc_base);
    delete h;
    return from_hip(e);
  }
  *out = reinterpret_cast<tpm_proj_t>(h);
  return TPM_OK;
}

tpm_status tp_proj_fwd(tpm_proj_t handle, const void *X_dev, int64_t M, void *Y_dev,
                       void *stream) {
  Proj *h = reinterpret_cast<Proj *>(handle);
  if (!h) return TPM_ERR_INVALID_ARG;
  const tpm_proj_desc &d = h->desc;
  if (M < 0 || M > d.max_tokens) return TPM_ERR_SHAPE;
  if (M == 0) return TPM_OK;
  if (!X_dev || !Y_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(X_dev) || !aligned(Y_dev)) return TPM_ERR_ALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return TPM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t K = d.in_features, N = d.out_features;
  if (d.in_dtype == TPM_F32) {
    const int epi = d.out_dtype == TPM_F32 ? EPI_OUT_F32 : EPI_OUT_BF16;
    return from_hip(launch_f32_gemm(epi, static_cast<const float *>(X_dev), K, M, K,
                                    static_cast<const float *>(h->w), N, N, 0, Y_dev, N, s));
  }
  const int epi = d.out_dtype == TPM_F32 ? EPI_PROJ_F32 : EPI_PROJ_BF16;
  int path = d.path;
  if (path == TPM_PATH_AUTO) path = M <= kStreamMaxTokens ? TPM_PATH_STREAM : TPM_PATH_TILED;
  hipError_t e;
  if (path == TPM_PATH_STREAM) {
    StreamScratch ws;
    ws.buf = h->scratch;
    ws.cnt = h->counters;
    ws.floats = h->scratch_floats;
    ws.n_counters = h->n_counters;
    e = launch_stream_gemm(epi, stream_plan(M, h->n_pad / kFragN, h->ks), X_dev, K, M, h->ks, h->w,
                           h->n_pad / kFragN, Y_dev, N, N, 0, ws, s);
  } else {
    TiledSplit split;
    if (h->scratch && h->counters && h->split_tiles > 0) {
      split.buf = h->scratch;
      split.cnt = h->counters;
      split.n_cu = h->n_cu;
      split.max_tiles = h->split_tiles;
    }
    e = launch_gemm(epi, X_dev, K, M, K, h->w, h->n_pad, Y_dev, N, N, 0, split, s);
  }
  return from_hip(e);
}

tpm_status tp_proj_destroy(tpm_proj_t handle) {
  Proj *h = reinterpret_cast<Proj *>(handle);
  if (!h) return TPM_OK;
  hipError_t e = hipDeviceSynchronize();
  const hipError_t e2 = hipFree(h->alloc_base);
  if (e == hipSuccess) e = e2;
  delete h;
  return from_hip(e);
}

}  // extern "C"
