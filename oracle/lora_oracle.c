/*
 * lora_oracle.c -- plain fp64 CPU oracle for batched multi-adapter LoRA.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * reference that the HIP library is checked against. Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * library never calls it and shares no code, header or constant with it.
 *
 * What it computes (notation: token t carries adapter i = a(t); adapter i has
 * rank r_i, scale s_i, shrink weight A_i [r_i x h_in] and expand weight
 * B_i [h_out x r_i], both row-major):
 *
 *   forward   u_t = A_i x_t                      (shrink, rank r_i)
 *             y_t = y_t + s_i * B_i u_t          (expand)
 *   backward  du_t = s_i * B_i^T dy_t
 *             dx_t = dx_t + A_i^T du_t
 *             dB_i = s_i * sum_{t: a(t)=i} dy_t u_t^T
 *             dA_i =       sum_{t: a(t)=i} du_t x_t^T
 *
 * Sources. LoRA keeps the base model frozen and trains small adapter weights
 * with a rank and a scaling factor ("Trajectory presenta C-LoRA" (vivodigitale.it), "Cos'e C-LoRA e
 * perche serve"; "Technische Samenvatting: PLoRA" (gist.science), "Resultaten", search space of rank and scaling
 * factor). A decode batch mixes tokens of many resident adapters and one
 * kernel launch covers the per-adapter matrix-vector work of the whole batch
 * ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona l'architettura"). Packed training runs
 * the forward and backward of many adapters together over concatenated LoRA
 * tensors ("Technische Samenvatting: PLoRA" (gist.science), "LoRA Execution Engine", "Packed LoRA Kernels" and
 * "Kernelontwerp"). The pages print no formula; the forward above is the
 * standard low-rank update written per token, and the backward is its chain
 * rule. Gradients are fp32 buffers on the GPU side ("Trajectory presenta C-LoRA" (vivodigitale.it),
 * "Come funziona l'architettura": gradient buffers in the AdapterStore); here
 * everything is fp64.
 *
 * Conventions. Adapter id -1 means "no adapter". A segment is a run of tokens
 * [seg_starts[g], seg_starts[g+1]) sharing seg_adapter[g]. Segments with id
 * -1 or rank 0 produce nothing. y and dx accumulate; u and du rows of skipped
 * tokens and columns k >= r_i are left untouched. dA/dB are overwritten
 * (accumulate == 0; adapters without tokens get zeros) or accumulated.
 *
 * Every sum runs in ascending index order; OpenMP splits only independent
 * outputs (tokens, or adapter rows), so results do not depend on the thread
 * count.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Grouping a request-order batch into per-adapter segments (the batch of a
 * decode step mixes tokens of different adapters; "Come funziona
 * l'architettura"). Definition: segment a (a = 0..N-1) holds, in their
 * original order, the tokens with id a; a final segment N holds the tokens
 * with id -1. perm[p] is the original index of the token at sorted position
 * p. seg_starts has N+2 entries, seg_adapter N+1 (the last is -1).
 * Returns 0, or -1 if an id is outside [-1, N).
 */
int oracle_segments_from_ids(const int32_t* ids, int32_t T, int32_t N, int32_t* perm,
                             int32_t* seg_starts, int32_t* seg_adapter) {
  for (int32_t t = 0; t < T; ++t)
    if (ids[t] < -1 || ids[t] >= N) return -1;
  int32_t pos = 0;
  for (int32_t a = 0; a <= N; ++a) {
    int32_t want = (a < N) ? a : -1;
    seg_starts[a] = pos;
    seg_adapter[a] = want;
    for (int32_t t = 0; t < T; ++t)
      if (ids[t] == want) perm[pos++] = t;
  }
  seg_starts[N + 1] = pos;
  return 0;
}

/* Adapter of every token from the segment list (-1 where no LoRA applies). */
static int32_t* token_adapters(int32_t T, int32_t S, const int32_t* seg_starts,
                               const int32_t* seg_adapter, const int32_t* ranks) {
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int32_t t = 0; t < T; ++t) a[t] = -1;
  for (int32_t g = 0; g < S; ++g) {
    int32_t i = seg_adapter[g];
    if (i < 0 || ranks[i] == 0) continue;
    for (int32_t t = seg_starts[g]; t < seg_starts[g + 1]; ++t) a[t] = i;
  }
  return a;
}

/*
 * Forward: shrink then expand, per token.
 *   u[t][k] = sum_d A_i[k][d] * x[t][d]                 (k < r_i)
 *   y[t][j] = y[t][j] + s_i * sum_k B_i[j][k] * u[t][k]  (j < h_out)
 * x [T][h_in], y [T][h_out] (in/out), u [T][ldu] (out).
 */
void oracle_forward(int32_t T, int32_t h_in, int32_t h_out, int32_t S, const int32_t* seg_starts,
                    const int32_t* seg_adapter, const int32_t* ranks, const double* scales,
                    const double* const* A, const double* const* B, const double* x, double* y,
                    double* u, int32_t ldu) {
  int32_t* a = token_adapters(T, S, seg_starts, seg_adapter, ranks);
#pragma omp parallel for schedule(dynamic, 4)
  for (int32_t t = 0; t < T; ++t) {
    int32_t i = a[t];
    if (i < 0) continue;
    const int32_t r = ranks[i];
    const double* Ai = A[i];
    const double* Bi = B[i];
    const double* xt = x + (size_t)t * h_in;
    double* ut = u + (size_t)t * ldu;
    for (int32_t k = 0; k < r; ++k) {
      double acc = 0.0;
      for (int32_t d = 0; d < h_in; ++d) acc += Ai[(size_t)k * h_in + d] * xt[d];
      ut[k] = acc;
    }
    double* yt = y + (size_t)t * h_out;
    for (int32_t j = 0; j < h_out; ++j) {
      double acc = 0.0;
      for (int32_t k = 0; k < r; ++k) acc += Bi[(size_t)j * r + k] * ut[k];
      yt[j] = yt[j] + scales[i] * acc;
    }
  }
  free(a);
}

/*
 * Backward of the forward above, given the forward's u.
 *   du[t][k]   = s_i * sum_j B_i[j][k] * dy[t][j]
 *   dx[t][d]  += sum_k A_i[k][d] * du[t][k]          (skipped if dx == NULL)
 *   dB_i[j][k] = s_i * sum_{t: a(t)=i} dy[t][j] * u[t][k]
 *   dA_i[k][d] =       sum_{t: a(t)=i} du[t][k] * x[t][d]
 * Token sums run over every segment of adapter i in ascending t.
 * dA[i] / dB[i] may be NULL for adapters whose gradient is not wanted.
 */
void oracle_backward(int32_t T, int32_t h_in, int32_t h_out, int32_t S, const int32_t* seg_starts,
                     const int32_t* seg_adapter, const int32_t* ranks, const double* scales,
                     const double* const* A, const double* const* B, int32_t N, const double* x,
                     const double* dy, const double* u, double* du, int32_t ldu, double* dx,
                     double* const* dA, double* const* dB, int32_t accumulate) {
  int32_t* a = token_adapters(T, S, seg_starts, seg_adapter, ranks);

#pragma omp parallel for schedule(dynamic, 4)
  for (int32_t t = 0; t < T; ++t) {
    int32_t i = a[t];
    if (i < 0) continue;
    const int32_t r = ranks[i];
    const double* Bi = B[i];
    const double* dyt = dy + (size_t)t * h_out;
    double* dut = du + (size_t)t * ldu;
    for (int32_t k = 0; k < r; ++k) {
      double acc = 0.0;
      for (int32_t j = 0; j < h_out; ++j) acc += Bi[(size_t)j * r + k] * dyt[j];
      dut[k] = scales[i] * acc;
    }
    if (dx) {
      /* acc[d] sums over k in ascending order; the k loop is outermost only
         so that rows of A_i are walked contiguously. */
      const double* Ai = A[i];
      double* dxt = dx + (size_t)t * h_in;
      double* acc = (double*)calloc((size_t)h_in, sizeof(double));
      for (int32_t k = 0; k < r; ++k)
        for (int32_t d = 0; d < h_in; ++d) acc[d] += Ai[(size_t)k * h_in + d] * dut[k];
      for (int32_t d = 0; d < h_in; ++d) dxt[d] = dxt[d] + acc[d];
      free(acc);
    }
  }

  /* token lists per adapter, ascending */
  int32_t* count = (int32_t*)calloc((size_t)N + 1, sizeof(int32_t));
  for (int32_t t = 0; t < T; ++t)
    if (a[t] >= 0) count[a[t] + 1]++;
  for (int32_t i = 0; i < N; ++i) count[i + 1] += count[i];
  int32_t* list = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  for (int32_t i = 0; i < N; ++i) fill[i] = count[i];
  for (int32_t t = 0; t < T; ++t)
    if (a[t] >= 0) list[fill[a[t]]++] = t;

  /* (adapter, row) work items: dB rows j < h_out, then dA rows k < r_i */
  int64_t total = 0;
  for (int32_t i = 0; i < N; ++i) total += (int64_t)h_out + ranks[i];
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t w = 0; w < total; ++w) {
    int64_t rem = w;
    int32_t i = 0;
    while (rem >= (int64_t)h_out + ranks[i]) { rem -= (int64_t)h_out + ranks[i]; ++i; }
    const int32_t r = ranks[i];
    const int32_t* ti = list + count[i];
    const int32_t nt = count[i + 1] - count[i];
    /* acc[.] sums over the adapter's tokens in ascending t; the token loop
       sits outside the row loop only so that token rows are walked
       contiguously. */
    if (rem < h_out) {
      const int32_t j = (int32_t)rem;
      if (!dB[i] || r == 0) continue;
      double* row = dB[i] + (size_t)j * r;
      double* acc = (double*)calloc((size_t)r, sizeof(double));
      for (int32_t q = 0; q < nt; ++q) {
        const int32_t t = ti[q];
        const double g = dy[(size_t)t * h_out + j];
        for (int32_t k = 0; k < r; ++k) acc[k] += g * u[(size_t)t * ldu + k];
      }
      for (int32_t k = 0; k < r; ++k) row[k] = (accumulate ? row[k] : 0.0) + scales[i] * acc[k];
      free(acc);
    } else {
      const int32_t k = (int32_t)(rem - h_out);
      if (!dA[i]) continue;
      double* row = dA[i] + (size_t)k * h_in;
      double* acc = (double*)calloc((size_t)h_in, sizeof(double));
      for (int32_t q = 0; q < nt; ++q) {
        const int32_t t = ti[q];
        const double g = du[(size_t)t * ldu + k];
        for (int32_t d = 0; d < h_in; ++d) acc[d] += g * x[(size_t)t * h_in + d];
      }
      for (int32_t d = 0; d < h_in; ++d) row[d] = (accumulate ? row[d] : 0.0) + acc[d];
      free(acc);
    }
  }
  free(fill);
  free(list);
  free(count);
  free(a);
}
