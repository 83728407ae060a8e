// C ABI of the grouped expert MLP: the SwiGLU (or tanh / identity) MLP of several
// experts, each applied to its own contiguous run of token rows, in one launch per
// projection.
//
// Page "大模型推理系统揭秘（07）Multi-GPU", MoE section: an expert is the MLP
// W2,e [SiLU(W1,e x) (.) (W3,e x)]; the tokens routed to the experts of one GPU are
// laid out contiguously by expert, and a grouped GEMM runs all the experts'
// products as one batched job instead of one launch per expert.  Routing,
// dispatch and combine (the all-to-all exchanges and the router weighting) are
// not part of this library: the caller hands over the tokens already grouped and
// the number of tokens per expert, in device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>

#include "tpm_internal.h"

using namespace tpm;

namespace {

constexpr int64_t kAlign = 16;
constexpr int64_t kMaxExperts = 1024;

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

tpm_status from_hip(hipError_t e) {
  if (e == hipSuccess) return TPM_OK;
  if (e == hipErrorOutOfMemory) return TPM_ERR_OOM;
  return TPM_ERR_HIP;
}

struct Moe {
  tpm_moe_desc desc;
  int device;
  int64_t ffn_pad, n1, n2, ks1, ks2;
  int64_t w1_stride, w2_stride;  // 16-byte chunks per expert
  void *w1, *w2, *hidden;
  void *alloc_base;
};

tpm_status check_moe_desc(const tpm_moe_desc *d) {
  if (!d) return TPM_ERR_INVALID_ARG;
  if (d->act < TPM_ACT_TANH || d->act > TPM_ACT_IDENTITY) return TPM_ERR_INVALID_ARG;
  if (d->in_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;  // the grouped path is bf16
  if (d->out_dtype != TPM_F32 && d->out_dtype != TPM_BF16) return TPM_ERR_INVALID_ARG;
  if (d->d_model < 64 || d->d_model % 64 || d->d_model > (int64_t(1) << 20)) return TPM_ERR_SHAPE;
  if (d->ffn_expert < 1 || d->ffn_expert > (int64_t(1) << 20)) return TPM_ERR_SHAPE;
  if (d->n_experts < 1 || d->n_experts > kMaxExperts) return TPM_ERR_SHAPE;
  if (d->max_tokens < 0 || d->max_tokens > (int64_t(1) << 24)) return TPM_ERR_SHAPE;
  if (d->path < TPM_PATH_AUTO || d->path > TPM_PATH_TILED) return TPM_ERR_INVALID_ARG;
  return TPM_OK;
}

}  // namespace

extern "C" {

tpm_status tp_moe_create(const tpm_moe_desc *desc, const void *W1_dev, const void *W2_dev,
                         void *stream, tpm_moe_t *out) {
  if (!out) return TPM_ERR_INVALID_ARG;
  *out = nullptr;
  tpm_status st = check_moe_desc(desc);
  if (st != TPM_OK) return st;
  if (!W1_dev || !W2_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(W1_dev) || !aligned(W2_dev)) return TPM_ERR_ALIGN;
  const tpm_moe_desc d = *desc;
  const bool silu = d.act == TPM_ACT_SILU_GATE;
  Moe *h = new (std::nothrow) Moe();
  if (!h) return TPM_ERR_OOM;
  h->desc = d;
  h->ffn_pad = silu ? round_up(d.ffn_expert, kTileN / 2) : round_up(d.ffn_expert, kTileN);
  h->n1 = silu ? 2 * h->ffn_pad : h->ffn_pad;
  h->n2 = round_up(d.d_model, kTileN);
  h->ks1 = d.d_model / kFragK;
  h->ks2 = h->ffn_pad / kFragK;
  h->w1_stride = h->ks1 * (h->n1 / kFragN) * 64;
  h->w2_stride = h->ks2 * (h->n2 / kFragN) * 64;
  const int64_t E = d.n_experts;
  const int64_t w1_bytes = E * h->w1_stride * 16, w2_bytes = E * h->w2_stride * 16;
  const int64_t hid_rows = round_up(d.max_tokens, kTileM) + E * kTileM;
  const int64_t hid_bytes = hid_rows * h->ffn_pad * 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return from_hip(e);
  }
  constexpr int64_t kSub = 256;
  const int64_t o_w2 = round_up(w1_bytes, kSub);
  const int64_t o_hid = round_up(o_w2 + w2_bytes, kSub);
  const int64_t total = round_up(o_hid + hid_bytes, kSub);
  e = hipMalloc(&h->alloc_base, static_cast<size_t>(total));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return TPM_ERR_OOM;
  }
  char *base = static_cast<char *>(h->alloc_base);
  h->w1 = base;
  h->w2 = base + o_w2;
  h->hidden = base + o_hid;
  const int64_t a_cols = silu ? 2 * d.ffn_expert : d.ffn_expert;
  for (int64_t x = 0; x < E && e == hipSuccess; ++x) {
    const char *a = static_cast<const char *>(W1_dev) + x * d.d_model * a_cols * 2;
    const char *b = static_cast<const char *>(W2_dev) + x * d.ffn_expert * d.d_model * 2;
    e = launch_pack_bf16(a, a_cols, d.d_model, a_cols, silu, d.ffn_expert, h->n1 / kFragN, h->ks1,
                         static_cast<char *>(h->w1) + x * h->w1_stride * 16, s);
    if (e == hipSuccess)
      e = launch_pack_bf16(b, d.d_model, d.ffn_expert, d.d_model, false, d.ffn_expert,
                           h->n2 / kFragN, h->ks2, static_cast<char *>(h->w2) + x * h->w2_stride * 16,
                           s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(h->alloc_base);
    delete h;
    return from_hip(e);
  }
  *out = reinterpret_cast<tpm_moe_t>(h);
  return TPM_OK;
}

tpm_status tp_moe_fwd(tpm_moe_t handle, const void *X_dev, const int32_t *counts_dev, int64_t T,
                      void *Y_dev, void *stream) {
  Moe *h = reinterpret_cast<Moe *>(handle);
  if (!h) return TPM_ERR_INVALID_ARG;
  const tpm_moe_desc &d = h->desc;
  if (T < 0 || T > d.max_tokens) return TPM_ERR_SHAPE;
  if (T == 0) return TPM_OK;
  if (!X_dev || !counts_dev || !Y_dev) return TPM_ERR_INVALID_ARG;
  if (!aligned(X_dev) || !aligned(Y_dev) || reinterpret_cast<uintptr_t>(counts_dev) % 4)
    return TPM_ERR_ALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return TPM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int epi1 = d.act == TPM_ACT_SILU_GATE ? EPI_SILU_GATE
                   : d.act == TPM_ACT_TANH    ? EPI_TANH
                                              : EPI_IDENTITY;
  const int epi2 = d.out_dtype == TPM_F32 ? EPI_OUT_F32 : EPI_OUT_BF16;
  TiledGroups g1, g2;
  g1.counts = g2.counts = counts_dev;
  g1.n_groups = g2.n_groups = static_cast<int>(d.n_experts);
  g1.w_stride = h->w1_stride;
  g2.w_stride = h->w2_stride;
  const TiledSplit none;
  // Weight streaming at a hundred or so tokens per expert, the tiled matrix-core
  // kernel for more (both read and write the same hidden layout).
  const bool streamed =
      d.path == TPM_PATH_STREAM || (d.path == TPM_PATH_AUTO && T <= kGroupStreamRows * d.n_experts);
  // the streaming launch takes one grid row per 128-token tile (+ one per expert)
  if (streamed && (T + kGroupStreamRows - 1) / kGroupStreamRows + d.n_experts > 65535)
    return TPM_ERR_SHAPE;
  hipError_t e = streamed
                     ? launch_group_stream(epi1, X_dev, d.d_model, T, d.d_model, h->w1, h->w1_stride,
                                           h->n1 / kFragN, counts_dev, g1.n_groups, h->hidden, 0, 0,
                                           h->ks2, s)
                     : launch_tiled_gemm(epi1, X_dev, d.d_model, T, d.d_model, h->w1, h->n1,
                                         h->hidden, 0, 0, h->ks2, none, s, Timing(), g1);
  if (e == hipSuccess)
    e = streamed ? launch_group_stream(epi2, h->hidden, 0, T, h->ffn_pad, h->w2, h->w2_stride,
                                       h->n2 / kFragN, counts_dev, g2.n_groups, Y_dev, d.d_model,
                                       d.d_model, 0, s)
                 : launch_tiled_gemm(epi2, h->hidden, 0, T, h->ffn_pad, h->w2, h->n2, Y_dev,
                                     d.d_model, d.d_model, 0, none, s, Timing(), g2);
  return from_hip(e);
}

tpm_status tp_moe_destroy(tpm_moe_t handle) {
  Moe *h = reinterpret_cast<Moe *>(handle);
  if (!h) return TPM_OK;
  hipError_t e = hipDeviceSynchronize();
  const hipError_t e2 = hipFree(h->alloc_base);
  if (e == hipSuccess) e = e2;
  delete h;
  return from_hip(e);
}

}  // extern "C"
