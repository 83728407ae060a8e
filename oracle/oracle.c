/*
 * Oracle for the tensor-parallel MLP shard: plain, slow, fp64 loops.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The GPU library never links it, and it
 * shares no code, header or constant with the GPU path.
 *
 * What it computes (the pages' definition, restated):
 *
 *   Page "大模型推理系统揭秘（07）Multi-GPU", section 1.2.2 (column/row split
 *   of Y = XW) and section 1.2.3 (the column -> row pairing, Z = sum_i Y_i W2_i):
 *   a column-parallel first projection gives each rank a slice Y_i = X A_i of
 *   the hidden features, the row-parallel second projection turns that slice into
 *   a full-shape partial Z_i = Y_i B_i, and the layer output is the sum of the
 *   partials.
 *
 *   Page "LLM 推理并行化：先找瓶颈，再决定怎么切", section 三.2 (tensor
 *   parallel), the NumPy function: per matched pair of shards the partial is
 *   act(x @ a_shard) @ b_shard (activation tanh by default), and the output is
 *   the element-wise sum of the partials.
 *
 *   Page "大模型推理系统揭秘（07）", section 1.4.3 (expert FFN): the SwiGLU form
 *   W2 [ SiLU(W1 x) (.) (W3 x) ]: SiLU is applied to the gate branch and the
 *   result is multiplied element-wise by the up branch.  SiLU(x) = x / (1 + e^-x)
 *   is the textbook definition (the pages name SiLU but do not define it).
 *
 * Activations (ORC_*):
 *   ORC_TANH      h = tanh(X A)            A is [d x F]
 *   ORC_SILU_GATE h = SiLU(X G) * (X U)    A is [d x 2F]; each row of A holds the
 *                                          F gate weights, then the F up weights
 *                                          (gate and up of one shard cover the same
 *                                          hidden indices)
 *   ORC_IDENTITY  h = X A                  A is [d x F]
 * then P = h B with B [F x N] (N = d for the MLP block; the pages' worked example
 * also uses an output width other than d).  All matrices are row-major, all arithmetic fp64,
 * every sum runs over its index in ascending order.  No blocking, no fusion.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_TANH = 0, ORC_SILU_GATE = 1, ORC_IDENTITY = 2 };
enum { ORC_OK = 0, ORC_BAD_ARG = 1, ORC_NO_MEMORY = 2 };

static double orc_silu(double x) { return x / (1.0 + exp(-x)); }

/* One rank's partial P [M x N]: P[m][n] = sum_j h[m][j] * B[j][n],
 * h[m][j] = act applied to sum_k X[m][k] * A[k][j] (and the up branch for SiLU-gate).
 * Rows m are independent; they are spread over threads, nothing else is reordered.
 * The k-loop is outside the j-loop so each A row is read contiguously; the sum for
 * every (m, j) still runs over k in ascending order. */
int orc_shard_forward(const double *X, int64_t M, int64_t d, const double *A,
                      int64_t F, const double *B, int64_t N, int act, double *P) {
  if (M < 0 || d < 1 || F < 1 || N < 1) return ORC_BAD_ARG;
  if (act != ORC_TANH && act != ORC_SILU_GATE && act != ORC_IDENTITY) return ORC_BAD_ARG;
  if (M == 0) return ORC_OK;
  if (!X || !A || !B || !P) return ORC_BAD_ARG;
  const int64_t ncol = (act == ORC_SILU_GATE) ? 2 * F : F; /* columns of A */
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    double *s = (double *)malloc((size_t)ncol * sizeof(double));
    double *h = (double *)malloc((size_t)F * sizeof(double));
    if (!s || !h) {
      free(s);
      free(h);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    /* first projection: s[j] = sum_k X[m][k] * A[k][j] */
    for (int64_t j = 0; j < ncol; ++j) s[j] = 0.0;
    for (int64_t k = 0; k < d; ++k) {
      const double x = X[m * d + k];
      const double *arow = A + k * ncol;
      for (int64_t j = 0; j < ncol; ++j) s[j] += x * arow[j];
    }
    /* activation, local to the rank */
    for (int64_t j = 0; j < F; ++j) {
      if (act == ORC_TANH)
        h[j] = tanh(s[j]);
      else if (act == ORC_SILU_GATE)
        h[j] = orc_silu(s[j]) * s[F + j]; /* gate branch s[j], up branch s[F+j] */
      else
        h[j] = s[j];
    }
    /* second projection: P[m][n] = sum_j h[j] * B[j][n] */
    double *prow = P + m * N;
    for (int64_t n = 0; n < N; ++n) prow[n] = 0.0;
    for (int64_t j = 0; j < F; ++j) {
      const double hj = h[j];
      const double *brow = B + j * N;
      for (int64_t n = 0; n < N; ++n) prow[n] += hj * brow[n];
    }
    free(s);
    free(h);
  }
  return failed ? ORC_NO_MEMORY : ORC_OK;
}

/* Sum of k rank partials in rank order: Z[e] = ((P_0[e] + P_1[e]) + ...) + P_{k-1}[e]. */
int orc_partials_sum(const double *const *parts, int32_t k, int64_t numel, double *Z) {
  if (k < 1 || numel < 0 || !parts || !Z) return ORC_BAD_ARG;
  for (int32_t i = 0; i < k; ++i)
    if (!parts[i]) return ORC_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < numel; ++e) {
    double acc = 0.0;
    for (int32_t i = 0; i < k; ++i) acc += parts[i][e];
    Z[e] = acc;
  }
  return ORC_OK;
}

/* One projection Y [M x N] = X [M x K] W [K x N] (page "大模型推理系统揭秘（07）
 * Multi-GPU", section 1.2.2: Y = XW, split by columns or by rows of W).  Plain loops:
 * Y[m][n] = sum_k X[m][k] * W[k][n], summed over k in ascending order; rows over threads. */
int orc_matmul(const double *X, int64_t M, int64_t K, const double *W, int64_t N, double *Y) {
  if (M < 0 || K < 1 || N < 1) return ORC_BAD_ARG;
  if (M == 0) return ORC_OK;
  if (!X || !W || !Y) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    double *yrow = Y + m * N;
    for (int64_t n = 0; n < N; ++n) yrow[n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double x = X[m * K + k];
      const double *wrow = W + k * N;
      for (int64_t n = 0; n < N; ++n) yrow[n] += x * wrow[n];
    }
  }
  return ORC_OK;
}

int orc_num_threads(void) {
  int n = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
#endif
  return n;
}
