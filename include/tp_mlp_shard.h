/*
 * tp_mlp_shard.h -- C ABI of the tensor-parallel MLP shard library (libtpmlp.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation.  One rank of a Megatron-style tensor-parallel MLP block holds a
 * column block A_i of the first weight and the matching row block B_i of the
 * second weight, and computes the full-shape partial
 *
 *     P_i = act(X A_i) B_i                       (one tp_mlp_shard_fwd call)
 *
 * The layer output is the sum of the partials of all ranks,
 *
 *     Z = sum_i P_i                              (one tp_partials_reduce call)
 *
 * which tensor parallelism obtains with an all-reduce; here the k partials are
 * held on one GPU and summed on it.  Sources:
 *   - page "大模型推理系统揭秘（07）Multi-GPU", section 1.2.2 (column- and
 *     row-parallel split of Y = XW), section 1.2.3 (the column output shard is the
 *     row input shard; Z = Z_0 + ... + Z_3), section 1.2.4 (gate/up projections
 *     column-parallel, activation local to the GPU, down projection row-parallel,
 *     one all-reduce after the MLP);
 *   - page "LLM 推理并行化：先找瓶颈，再决定怎么切", section 三.2: the NumPy
 *     function that, for each matched pair of shards, takes act(x @ a) @ b and sums
 *     the partials (tanh is its default activation; mismatched shard lists are an
 *     error);
 *   - page "大模型推理系统揭秘（07）", section 1.4.3: the SwiGLU form
 *     SiLU(x W1) (.) (x W3) before W2 (SiLU on the gate branch);
 *   - page "7.4 推理侧并行", section 7.4.2 (communication quantization): partial
 *     sums are accumulated in high precision, so partials and the reduction are fp32
 *     by default.
 *
 * Conventions for every call:
 *   - All matrices are dense, row-major, with no padding between rows.
 *   - "_dev" pointers are device pointers (hipMalloc or torch CUDA tensors) on the
 *     current HIP device; every other pointer is a host pointer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued on it and the call returns without waiting, except create(), which
 *     waits for its own work before returning.
 *   - Calls return a status code; they never abort or throw across the ABI.
 *     Arguments are checked on the host before anything is enqueued: a call that
 *     returns an error has enqueued nothing.  Faults inside kernels surface at the
 *     caller's next synchronization with the stream.
 *   - Device pointers must be 16-byte aligned (TPM_ERR_ALIGN otherwise).
 */
#ifndef TP_MLP_SHARD_H
#define TP_MLP_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tpm_status {
  TPM_OK = 0,
  TPM_ERR_INVALID_ARG = 1, /* NULL pointer where one is required, enum out of range */
  TPM_ERR_SHAPE = 2,       /* size out of range or not a supported multiple */
  TPM_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  TPM_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  TPM_ERR_OOM = 5          /* device allocation failed */
} tpm_status;

typedef enum tpm_act {
  TPM_ACT_TANH = 0,      /* h = tanh(X A); the default of the pages' NumPy function */
  TPM_ACT_SILU_GATE = 1, /* h = SiLU(X G) * (X U), SiLU(x) = x / (1 + exp(-x)) */
  TPM_ACT_IDENTITY = 2   /* h = X A */
} tpm_act;

typedef enum tpm_dtype {
  TPM_F32 = 0,
  TPM_BF16 = 1
} tpm_dtype;

/* Which kernels fwd uses.  AUTO picks by the token count M of each call:
 * M <= tpm_plan_info.stream_max_tokens takes the weight-streaming path (decode),
 * larger M the LDS-tiled matrix-core path (prefill).  The other two force a path,
 * for any M (used to test both on the same input).  Ignored for TPM_F32 input. */
typedef enum tpm_path {
  TPM_PATH_AUTO = 0,
  TPM_PATH_STREAM = 1,
  TPM_PATH_TILED = 2
} tpm_path;

/* Shape and numerics of one rank's shard.
 *
 *   d_model    d: width of X, of each row of A_i and of the partial.
 *   ffn_shard  F: hidden features held by this rank (F = ffn / TP degree).
 *   max_tokens largest M a fwd call may pass; sizes the internal hidden buffer.
 *   act        tpm_act.
 *   in_dtype   dtype of X, A_i and B_i (TPM_F32 or TPM_BF16).
 *   out_dtype  dtype of the partial written by fwd (TPM_F32 default, or TPM_BF16).
 *   path       tpm_path.
 *
 * Constraints (TPM_ERR_SHAPE otherwise): d >= 1, F >= 1, max_tokens >= 0;
 * for TPM_BF16 input d must be a multiple of 64.  F has no multiple constraint:
 * the hidden dimension is zero-padded internally. */
typedef struct tpm_desc {
  int64_t d_model;
  int64_t ffn_shard;
  int64_t max_tokens;
  int32_t act;
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t path;
} tpm_desc;

/* What create() would allocate and how fwd would run (filled by plan()). */
typedef struct tpm_plan_info {
  int64_t packed_weight_bytes; /* device bytes of the handle's repacked A_i and B_i */
  int64_t workspace_bytes;     /* device bytes of the hidden buffer and split-K scratch */
  int64_t ffn_padded;          /* F rounded up to the internal tile width */
  int64_t stream_max_tokens;   /* AUTO uses the streaming path for M <= this */
  int32_t kernels_per_fwd;     /* kernel launches one fwd call makes (M > 0) */
  int32_t reserved;
} tpm_plan_info;

typedef struct tpm_shard *tpm_shard_t;

/* Status code -> static, NUL-terminated English text (never NULL). */
const char *tpm_status_str(tpm_status status);

/* Validate `desc` and report sizes, host only (no HIP call, no allocation).
 * desc, out: host pointers, required.  On error *out is left untouched. */
tpm_status tp_mlp_shard_plan(const tpm_desc *desc, tpm_plan_info *out);

/* Create a shard handle: allocate its device memory on the current device, repack
 * the rank's weights into the layout the kernels stream, and wait for `stream`.
 *
 *   A_dev  first-weight shard, [d x F] (tanh, identity) or [d x 2F] (silu_gate:
 *          each row holds the F gate weights, then the F up weights, both over the
 *          rank's hidden indices), dtype desc->in_dtype.
 *   B_dev  second-weight shard, [F x d], dtype desc->in_dtype.
 *   out    host pointer that receives the handle.
 *
 * The handle owns copies of the weights: A_dev and B_dev may be freed once create
 * returns.  On error *out is set to NULL and nothing stays allocated. */
tpm_status tp_mlp_shard_create(const tpm_desc *desc, const void *A_dev, const void *B_dev,
                               void *stream, tpm_shard_t *out);

/* One rank's forward: partial_dev = act(X_dev A_i) B_i.
 *
 *   X_dev        tokens, [M x d], dtype in_dtype.
 *   M            token count, 0 <= M <= max_tokens; M = 0 is a successful no-op.
 *   partial_dev  output, [M x d], dtype out_dtype, fully overwritten.
 *
 * Asynchronous on `stream`; allocates nothing, so it may be captured in a HIP
 * graph.  A handle keeps per-call state (hidden buffer, split-K scratch): use one
 * handle on one stream at a time.  X_dev and partial_dev must not overlap. */
tpm_status tp_mlp_shard_fwd(tpm_shard_t h, const void *X_dev, int64_t M, void *partial_dev,
                            void *stream);

/* For callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as tp_mlp_shard_fwd on the decode (weight-streaming) path, 1 <= M <= 64
 * (M = 0 is a successful no-op), bf16 handles only, with the hidden buffer and the
 * contraction-slice scratch in one array of TPM_NOALLOC_SCRATCH_BYTES that the
 * library holds per device from load to process end, instead of the handle's
 * workspace (so a handle created with max_tokens = 0 works too).  Its arguments,
 * layouts and results are those of tp_mlp_shard_fwd; the two return the same
 * partial bit for bit.  Allocates nothing, calls no allocating routine.
 *
 * Errors: TPM_ERR_SHAPE for M > 64, a non-bf16 handle or a shard whose scratch need
 * (ceil(M / 32) * ffn_padded / 16 KiB of hidden rows, plus slice sums for narrow
 * shards) exceeds TPM_NOALLOC_SCRATCH_BYTES; TPM_ERR_HIP if the array's device
 * address cannot be obtained (first call on a device).  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, or a handle
 * used from two threads) race. */
#define TPM_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
tpm_status tp_mlp_shard_fwd_noalloc(tpm_shard_t h, const void *X_dev, int64_t M,
                                    void *partial_dev, void *stream);

/* Sum k partials held on this GPU, in rank order, with fp32 accumulation:
 *   out_dev[e] = (((p_0[e] + p_1[e]) + p_2[e]) + ...) + p_{k-1}[e],  0 <= e < numel.
 *
 *   partials_dev  host array of k device pointers, each to numel elements of in_dtype.
 *   k             1 <= k <= 16 (k = 1 copies, or converts the dtype).
 *   numel         elements per partial, >= 0 (0 is a no-op).
 *   out_dev       numel elements of out_dtype.  It may be partials_dev[0] itself
 *                 (same pointer, same dtype); any other overlap is undefined.
 * The result is bitwise reproducible from call to call.  Asynchronous on `stream`. */
tpm_status tp_partials_reduce(const void *const *partials_dev, int32_t k, int64_t numel,
                              int32_t in_dtype, void *out_dev, int32_t out_dtype, void *stream);

/* The partials sum fused with what follows the all-reduce of a tensor-parallel
 * block (page "7.4 推理侧并行", section 7.4.2: fusing the residual add and RMSNorm
 * that follow the all-reduce into one kernel saves a round trip through device
 * memory).  For each row r of [rows x cols], in fp32:
 *   z               = ((p_0[r] + p_1[r]) + ...) + p_{k-1}[r]    (rank order)
 *   h               = residual[r] + z
 *   residual_out[r] = h                                         (rounded to res_dtype)
 *   y[r]            = h / sqrt(mean_c(h^2) + eps) * gamma       (rounded to out_dtype)
 * RMSNorm is not defined on the pages; this is its textbook form (no mean
 * subtraction, no bias), with the mean of squares taken over the row's cols values
 * of the fp32 h.
 *
 *   partials_dev      host array of k device pointers, each [rows x cols] of in_dtype.
 *   k                 1 <= k <= 16.
 *   rows              >= 0 (0 is a no-op), at most 2^31 - 1.
 *   cols              a multiple of 8, 8 <= cols <= 32768.
 *   residual_dev      [rows x cols] of res_dtype.
 *   residual_out_dev  [rows x cols] of res_dtype; may be residual_dev itself.
 *   gamma_dev         [cols] of res_dtype (the RMSNorm weight).
 *   eps               finite, >= 0.
 *   y_dev             [rows x cols] of out_dtype.
 * Outputs must not overlap the partials, gamma or each other (apart from the
 * in-place residual).  Bitwise reproducible from call to call.  Asynchronous on
 * `stream`; allocates nothing. */
tpm_status tp_partials_reduce_add_rmsnorm(const void *const *partials_dev, int32_t k,
                                          int64_t rows, int64_t cols, int32_t in_dtype,
                                          const void *residual_dev, void *residual_out_dev,
                                          int32_t res_dtype, const void *gamma_dev, float eps,
                                          void *y_dev, int32_t out_dtype, void *stream);

/* Low-precision partials (page "7.4 推理侧并行", section 7.4.2, communication
 * quantization: partials may travel in FP8 with a per-token scale, but the sum is
 * done in high precision after dequantizing).  FP8 here is OCP E4M3 (1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities, codes
 * 0x7f / 0xff are NaN, largest finite value 448); the pages do not fix the layout.
 *
 * Quantize one partial, per row r of [rows x cols]:
 *   amax_r    = max_c |x[r][c]|
 *   scale[r]  = amax_r / 448                 (fp32, correctly rounded; 1 if amax_r = 0)
 *   q[r][c]   = E4M3(x[r][c] * (448 / amax_r)), both fp32 operations correctly
 *               rounded, the code rounded to nearest (ties to even) and saturated to
 *               +-448; all zero when amax_r = 0.
 * A row holding NaN or infinity gives unspecified codes and scale.
 *
 *   partial_dev  [rows x cols] of in_dtype (TPM_F32 or TPM_BF16).
 *   rows         >= 0 (0 is a no-op), at most 2^31 - 1.
 *   cols         a multiple of 16, 16 <= cols <= 32768.
 *   q_dev        [rows x cols] bytes (E4M3 codes).
 *   scale_dev    [rows] fp32.
 * Asynchronous on `stream`; allocates nothing. */
tpm_status tp_partials_quantize_fp8(const void *partial_dev, int64_t rows, int64_t cols,
                                    int32_t in_dtype, void *q_dev, float *scale_dev,
                                    void *stream);

/* Sum k quantized partials with fp32 accumulation, in rank order:
 *   out[r][c] = ((d_0 + d_1) + ...) + d_{k-1},  d_i = value(q_i[r][c]) * scale_i[r]
 * (each product rounded to fp32).
 *
 *   q_dev      host array of k device pointers, each [rows x cols] E4M3 codes.
 *   scale_dev  host array of k device pointers, each [rows] fp32.
 *   k          1 <= k <= 16.
 *   rows, cols cols a multiple of 16 (>= 16), rows >= 0 (0 is a no-op).
 *   out_dev    [rows x cols] of out_dtype (TPM_F32 or TPM_BF16); must not overlap
 *              the inputs.
 * Bitwise reproducible from call to call.  Asynchronous on `stream`. */
tpm_status tp_partials_reduce_fp8(const void *const *q_dev, const float *const *scale_dev,
                                  int32_t k, int64_t rows, int64_t cols, void *out_dev,
                                  int32_t out_dtype, void *stream);

/* Merge of k attention partials held on one GPU.
 *
 * Page "LLM 推理并行化：先找瓶颈，再决定怎么切", section 三.4 (decode context
 * parallelism): the stored KV history is split by sequence position; each rank
 * attends over its own keys and reports, per query row, its local score maximum
 * m_i, its sum of exponentials s_i = sum_j exp(z_j - m_i) and its weighted value
 * sum v_i = sum_j exp(z_j - m_i) V_j.  The merge rescales every rank to the global
 * maximum (so no exponential exceeds 1):
 *   g[r]      = max_i m_i[r]
 *   c_i       = exp(m_i[r] - g[r])                 (0 for a rank with m_i = -inf)
 *   S[r]      = sum_i c_i * s_i[r]                 (rank order, fp32)
 *   out[r][:] = (sum_i c_i * v_i[r][:]) / S[r]     (rank order, fp32)
 * A row with no keys on any rank (every m_i = -inf) gives out = 0, g = -inf, S = 0.
 *
 *   values_dev   host array of k device pointers, each [rows x dim] of in_dtype
 *                (TPM_F32 or TPM_BF16), 16-byte aligned.
 *   max_dev      host array of k device pointers, each [rows] fp32 (m_i).
 *   expsum_dev   host array of k device pointers, each [rows] fp32 (s_i).
 *   k            1 <= k <= 16.
 *   rows         >= 0 (0 is a no-op); dim: a multiple of 8, 8 <= dim <= 2^20.
 *   out_dev      [rows x dim] of out_dtype, 16-byte aligned; may be values_dev[0]
 *                exactly when in_dtype == out_dtype, must not overlap the others.
 *   max_out_dev, expsum_out_dev
 *                [rows] fp32 each, the merged statistics (g, S), so that the merged
 *                result (out * S, g, S) can be merged again; both NULL to skip.
 *                They must not overlap any input.
 * Statistics pointers need 4-byte alignment.  Bitwise reproducible from call to
 * call.  Asynchronous on `stream`; allocates nothing. */
tpm_status tp_attn_partials_merge(const void *const *values_dev, const float *const *max_dev,
                                  const float *const *expsum_dev, int32_t k, int64_t rows,
                                  int64_t dim, int32_t in_dtype, void *out_dev, int32_t out_dtype,
                                  float *max_out_dev, float *expsum_out_dev, void *stream);

/* Free a handle and its device memory (waits for the device first).  NULL is OK. */
tpm_status tp_mlp_shard_destroy(tpm_shard_t h);

/* Single tensor-parallel projections, Y = X W on one rank's shard of W.
 *
 * Page "大模型推理系统揭秘（07）Multi-GPU", section 1.2.4: in the attention block
 * the Q, K and V projections are column-parallel (each GPU holds some heads), the
 * attention is computed locally, and the output projection is row-parallel, its
 * rank partials summed by one all-reduce.  The attention itself is not part of
 * this library; the two projections around it are:
 *   - column-parallel QKV: W = the rank's columns of [Wq | Wk | Wv] ([d x n_i]),
 *     Y = [M x n_i] (bf16 for the local attention);
 *   - row-parallel output: W = the rank's rows of Wo ([q_i x d]), X = the rank's
 *     attention output [M x q_i], Y = its fp32 partial [M x d], summed over ranks
 *     with tp_partials_reduce.
 *
 *   in_features   K: width of X and rows of W.
 *   out_features  N: columns of W and of Y.
 *   max_tokens    largest M a fwd call may pass.
 *   in_dtype      dtype of X and W (TPM_F32 or TPM_BF16); out_dtype: dtype of Y.
 *   path          tpm_path (AUTO: M <= stream_max_tokens streams the weight).
 * Constraints (TPM_ERR_SHAPE otherwise): K, N >= 1, max_tokens >= 0; for TPM_BF16
 * input K must be a multiple of 64.  N has no multiple constraint. */
typedef struct tpm_proj_desc {
  int64_t in_features;
  int64_t out_features;
  int64_t max_tokens;
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t path;
  int32_t reserved;
} tpm_proj_desc;

typedef struct tpm_proj *tpm_proj_t;

/* Create a projection handle: allocate its device memory on the current device,
 * repack W_dev ([K x N] row-major, in_dtype) and wait for `stream`.  The handle owns
 * its copy; W_dev may be freed once create returns.  On error *out is NULL. */
tpm_status tp_proj_create(const tpm_proj_desc *desc, const void *W_dev, void *stream,
                          tpm_proj_t *out);

/* Y_dev = X_dev W with fp32 accumulation.  X_dev [M x K] in_dtype, Y_dev [M x N]
 * out_dtype, fully overwritten; 0 <= M <= max_tokens (0 is a no-op).  Asynchronous
 * on `stream`, allocates nothing (graph-capturable); one handle on one stream at a
 * time.  X_dev and Y_dev must not overlap. */
tpm_status tp_proj_fwd(tpm_proj_t h, const void *X_dev, int64_t M, void *Y_dev, void *stream);

/* Free a projection handle (waits for the device first).  NULL is OK. */
tpm_status tp_proj_destroy(tpm_proj_t h);

/* Grouped expert MLP: E experts held on this GPU, each expert e the MLP
 * act(X_e W1_e) W2_e of the tokens X_e routed to it (page "大模型推理系统揭秘（07）
 * Multi-GPU", MoE section: Expert_e(x) = W2,e [SiLU(W1,e x) (.) (W3,e x)], the
 * tokens of a GPU laid out contiguously by expert and all experts' products run as
 * one grouped GEMM).  Routing, dispatch and combine (all-to-all exchanges, router
 * weights) are the caller's.
 *
 * Both projections run on one of two kernels: STREAM, for a hundred or so tokens
 * per expert, streams each expert's weights once per 128 of its tokens
 * (weight-bound, as at decode); TILED runs 256-token tiles on the matrix cores (for
 * many tokens per expert).  AUTO takes STREAM when T <= 128 * E.
 *
 *   d_model     d, a multiple of 64.
 *   ffn_expert  F: hidden features of one expert (no multiple constraint).
 *   n_experts   E, 1 <= E <= 1024.
 *   max_tokens  largest T (tokens over all experts) a fwd call may pass.
 *   act         tpm_act (SILU_GATE: W1_e holds F gate then F up columns per row).
 *   in_dtype    TPM_BF16 (the grouped path is bf16 only); out_dtype: dtype of Y.
 * Constraints: TPM_ERR_SHAPE / TPM_ERR_INVALID_ARG as for the shard handle. */
typedef struct tpm_moe_desc {
  int64_t d_model;
  int64_t ffn_expert;
  int64_t n_experts;
  int64_t max_tokens;
  int32_t act;
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t path;  /* tpm_path: AUTO, STREAM or TILED */
} tpm_moe_desc;

typedef struct tpm_moe *tpm_moe_t;

/* Create: W1_dev holds the E first weights back to back ([E][d x 2F] for
 * SILU_GATE, else [E][d x F]), W2_dev the E second weights ([E][F x d]), all
 * row-major bf16.  The handle owns packed copies; waits for `stream`. */
tpm_status tp_moe_create(const tpm_moe_desc *desc, const void *W1_dev, const void *W2_dev,
                         void *stream, tpm_moe_t *out);

/* Y_dev[rows of expert e] = act(X_e W1_e) W2_e for every expert, in two launches.
 *
 *   X_dev       [T x d] bf16: the tokens of expert 0, then those of expert 1, ...
 *   counts_dev  device array of E int32: tokens per expert, in expert order.  Read
 *               on the device (no host synchronization); counts past the T rows
 *               are clamped (rows of X beyond T are never read), negative counts
 *               count as 0, and rows beyond the sum of the counts are left as they
 *               were.
 *   T           rows of X and Y, 0 <= T <= max_tokens (0 is a no-op); on the STREAM
 *               path also ceil(T / 128) + E <= 65535 (TPM_ERR_SHAPE otherwise; AUTO
 *               never streams that many).
 *   Y_dev       [T x d] of out_dtype.
 * Asynchronous on `stream`, allocates nothing; one handle on one stream at a time. */
tpm_status tp_moe_fwd(tpm_moe_t h, const void *X_dev, const int32_t *counts_dev, int64_t T,
                      void *Y_dev, void *stream);

/* Free a grouped-expert handle (waits for the device first).  NULL is OK. */
tpm_status tp_moe_destroy(tpm_moe_t h);

/* Timing hook for profiling.  When `events` is non-NULL, every later fwd call on
 * this handle attaches events[2j] and events[2j+1] to its j-th kernel launch, for
 * j < kernels_per_fwd: they record the start and the end of that kernel's
 * execution (they travel with the kernel's own dispatch, so no extra work is
 * enqueued and the stream's timing is unchanged).  n_events must be at least
 * 2 * kernels_per_fwd.  The events are hipEvent_t created by the caller, passed as
 * void*, and stay owned by the caller.  events = NULL (with n_events = 0) switches
 * the hook off. */
tpm_status tp_mlp_shard_set_timing_events(tpm_shard_t h, void *const *events, int32_t n_events);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* TP_MLP_SHARD_H */
