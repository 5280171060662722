/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for the gated delta rule forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or constant with the HIP
 * library and is compiled on its own with gcc.
 *
 * Every routine here is the plain definition of the step it names, written out
 * token by token (or tap by tap) in double precision, with no blocking, no
 * chunking and no reordering beyond what the definition states.  Parallelism
 * is only across independent (sequence, head) units or channels.
 *
 * Sources (the pages are pull requests describing GatedDeltaNet context
 * parallelism; the formula itself is the one the method is defined by):
 *   - prime-rl PR "feat: hybrid CP for Qwen3.5 MoE", Summary: the per-head state
 *     S lives in R^{K x V} and is updated sequentially token by token.
 *   - the gated delta rule: S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1}
 *     + beta_t k_t v_t^T, o_t = S_t^T q_t (state stored K x V), with
 *     beta = sigmoid(b) and g = -exp(A_log) * softplus(a + dt_bias).
 *   - LlamaFactory PR "[v1] support GDN Ulysses cp", Design, decisions 5-6:
 *     packed samples (cu_seqlens) must not leak into each other, in the causal
 *     conv1d as well as in the recurrence.
 *   - sglang fork PR "Qwen3.5 cp - #1", PR body: each context segment is an
 *     affine map of its initial state, S_end = M S_start + b, and the (b, M)
 *     pairs are chain-reduced in fp32 across segments.
 *
 * Layouts (row-major, token-major, all double):
 *   q, k      [T, Hqk, K]          v, o        [T, Hv, V]
 *   g, beta   [T, Hv]              s0, sfinal  [N, Hv, K, V]
 *   cu        int64 [N + 1], cu[0] = 0 .. cu[N] = T (packed sample offsets)
 *   v-head h reads qk-head h / (Hv / Hqk) (contiguous groups).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static void set_threads(int n_threads) {
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
}

/* Validates a packed-offsets array: monotone, starts at 0. Returns 0 if fine. */
static int check_cu(const int64_t* cu, int n) {
  if (!cu || n < 0 || cu[0] != 0) return -1;
  for (int i = 0; i < n; ++i)
    if (cu[i + 1] < cu[i]) return -1;
  return 0;
}

/*
 * Token-by-token recurrence (the definition).  For every sequence n and v-head
 * h, starting from S = s0[n,h] (zero when s0 is NULL), each token t does
 *   S <- exp(g_t) S                    (gated decay)
 *   u <- beta_t (v_t - S^T k_t)        (delta-rule correction of the prediction)
 *   S <- S + k_t u^T                   (write)
 *   o_t <- scale * S^T q_t             (read after the write)
 * which multiplies out to S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1}
 * + beta_t k_t v_t^T.  unit_mask (optional, [N*Hv]) restricts the work to the
 * selected (n, h) units; outputs of unselected units are left untouched.
 */
int oracle_gdn_recurrence(const double* q, const double* k, const double* v,
                          const double* g, const double* beta, const double* s0,
                          const int64_t* cu, int N, int Hqk, int Hv, int K, int V,
                          double scale, const unsigned char* unit_mask, double* o,
                          double* sfinal, int n_threads) {
  if (check_cu(cu, N) || Hqk <= 0 || Hv <= 0 || K <= 0 || V <= 0 || Hv % Hqk) return -1;
  set_threads(n_threads);
  const int group = Hv / Hqk;
  const int64_t units = (int64_t)N * Hv;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < units; ++unit) {
    if (unit_mask && !unit_mask[unit]) continue;
    const int n = (int)(unit / Hv), h = (int)(unit % Hv), hq = h / group;
    double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* u = (double*)malloc(sizeof(double) * (size_t)V);
    if (!S || !u) {
      free(S);
      free(u);
#pragma omp atomic write
      err = -2;
      continue;
    }
    if (s0)
      memcpy(S, s0 + (size_t)unit * K * V, sizeof(double) * (size_t)K * V);
    else
      memset(S, 0, sizeof(double) * (size_t)K * V);
    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      const double* kt = k + ((size_t)t * Hqk + hq) * K;
      const double* qt = q + ((size_t)t * Hqk + hq) * K;
      const double* vt = v + ((size_t)t * Hv + h) * V;
      const double decay = exp(g[(size_t)t * Hv + h]);
      const double b = beta[(size_t)t * Hv + h];
      for (int64_t i = 0; i < (int64_t)K * V; ++i) S[i] *= decay;
      for (int j = 0; j < V; ++j) {
        double pred = 0.0;
        for (int i = 0; i < K; ++i) pred += S[(size_t)i * V + j] * kt[i];
        u[j] = b * (vt[j] - pred);
      }
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += kt[i] * u[j];
      if (o) {
        double* ot = o + ((size_t)t * Hv + h) * V;
        for (int j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int i = 0; i < K; ++i) acc += S[(size_t)i * V + j] * qt[i];
          ot[j] = scale * acc;
        }
      }
    }
    if (sfinal) memcpy(sfinal + (size_t)unit * K * V, S, sizeof(double) * (size_t)K * V);
    free(S);
    free(u);
  }
  return err;
}

/*
 * Segment transition matrix by explicit dense products: for tokens [t0, t1) of
 * the packed arrays, M[h] = A_{t1-1} ... A_{t0} with
 * A_t = exp(g_t) (I - beta_t k_t k_t^T), so that the state at the segment end
 * is M S_start + b (b being the recurrence run from a zero state).  O(L K^3):
 * for pinning and small checks only.  M is [Hv, K, K].
 */
int oracle_transition(const double* k, const double* g, const double* beta, int64_t t0,
                      int64_t t1, int Hqk, int Hv, int K, double* M, int n_threads) {
  if (t1 < t0 || Hqk <= 0 || Hv <= 0 || K <= 0 || Hv % Hqk) return -1;
  set_threads(n_threads);
  const int group = Hv / Hqk;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < Hv; ++h) {
    double* P = M + (size_t)h * K * K; /* running product, starts at I */
    double* A = (double*)malloc(sizeof(double) * (size_t)K * K);
    double* R = (double*)malloc(sizeof(double) * (size_t)K * K);
    if (!A || !R) {
      free(A);
      free(R);
#pragma omp atomic write
      err = -2;
      continue;
    }
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < K; ++j) P[(size_t)i * K + j] = (i == j) ? 1.0 : 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      const double* kt = k + ((size_t)t * Hqk + h / group) * K;
      const double e = exp(g[(size_t)t * Hv + h]);
      const double b = beta[(size_t)t * Hv + h];
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < K; ++j)
          A[(size_t)i * K + j] = e * ((i == j ? 1.0 : 0.0) - b * kt[i] * kt[j]);
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < K; ++j) {
          double acc = 0.0;
          for (int l = 0; l < K; ++l) acc += A[(size_t)i * K + l] * P[(size_t)l * K + j];
          R[(size_t)i * K + j] = acc;
        }
      memcpy(P, R, sizeof(double) * (size_t)K * K);
    }
    free(A);
    free(R);
  }
  return err;
}

/*
 * Causal depthwise conv1d (+ optional SiLU), the PyTorch conv1d convention
 * (cross-correlation, left zero padding of W-1, groups = channels), with the
 * history reset at every packed-sample start:
 *   y[t, c] = act( bias[c] + sum_{j=0}^{W-1} w[c, j] * x[t - (W-1) + j, c] ),
 * where x[tau, c] counts as 0 for tau before the start of t's sample, and
 * act(z) = z / (1 + exp(-z)) when apply_silu, else z.
 * x, y [T, C]; w [C, W]; bias [C] or NULL.
 */
int oracle_conv1d(const double* x, const double* w, const double* bias, const int64_t* cu,
                  int N, int C, int W, int apply_silu, double* y, int n_threads) {
  if (check_cu(cu, N) || C <= 0 || W <= 0) return -1;
  set_threads(n_threads);
#pragma omp parallel for schedule(static)
  for (int c = 0; c < C; ++c) {
    for (int n = 0; n < N; ++n) {
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
        double acc = bias ? bias[c] : 0.0;
        for (int j = 0; j < W; ++j) {
          const int64_t tau = t - (W - 1) + j;
          if (tau < cu[n]) continue;
          acc += w[(size_t)c * W + j] * x[(size_t)tau * C + c];
        }
        y[(size_t)t * C + c] = apply_silu ? acc / (1.0 + exp(-acc)) : acc;
      }
    }
  }
  return 0;
}

/*
 * Gates: beta = sigmoid(b) = 1 / (1 + exp(-b)),
 *        g    = -exp(A_log[h]) * softplus(a + dt_bias[h]),
 * softplus(x) = log(1 + exp(x)), evaluated as max(x, 0) + log1p(exp(-|x|)) so
 * that it neither overflows for large x nor loses the tail for very negative x.
 * a, b, g, beta [T, H]; A_log, dt_bias [H].
 */
void oracle_gates(const double* a, const double* b, const double* A_log, const double* dt_bias,
                  int64_t T, int H, double* g, double* beta) {
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      const size_t i = (size_t)t * H + h;
      const double x = a[i] + dt_bias[h];
      const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
      g[i] = -exp(A_log[h]) * sp;
      beta[i] = 1.0 / (1.0 + exp(-b[i]));
    }
}
