/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 reference for the Kimi Delta Attention (KDA) forward pass
 * and its scalar-gate / grouped-value-head variant.  It exists so that the
 * GPU path can be checked against something obviously correct.  Only the
 * test-suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it; the GPU library never links or calls it, and it shares no code,
 * header or constant with the GPU path.
 *
 * What it computes (the recurrence as stated for KDA: a gated delta rule,
 * chunked forward of the KDA operator whose interface FlashKDA documents on
 * the refft.com FlashKDA summary, "stateful/streaming" section):
 *
 *   per chain (batch row or packed sequence, value head h), state S in
 *   R^{K x V}, starting from initial_state (or zeros), for each token t:
 *
 *     qn  = q_t / sqrt(sum(q_t^2) + eps)          (L2 normalisation)
 *     kn  = k_t / sqrt(sum(k_t^2) + eps)
 *     g_t = -exp(A_log[h]) * softplus(g_raw_t)     (per channel, or one
 *                                                   scalar per token-head)
 *     b_t = 1 / (1 + exp(-beta_logit_t))           (sigmoid)
 *     S_t = (I - b_t kn kn^T) Diag(exp(g_t)) S_{t-1} + b_t kn v_t^T
 *     o_t = scale * S_t^T qn
 *
 * Nothing is blocked, reordered or chunked: the state is advanced one token
 * at a time exactly as the definition reads.  Inputs arrive already widened
 * to fp64 (bf16 and fp32 both convert to fp64 exactly), so the oracle sees
 * precisely the values the GPU receives.
 *
 * Layouts (row-major, contiguous):
 *   q, k    [B, T, H_qk, K]
 *   v       [B, T, H, V]
 *   g_raw   [B, T, H, K] (per-channel gate) or [B, T, H] (scalar gate)
 *   beta    [B, T, H]
 *   A_log   [H]
 *   out     [B, T, H, V]
 *   state   [C, H, V, K] with state[c, h, v, kk] = S[kk][v], C = B (dense)
 *           or N (packed sequences).
 * Value head h reads q/k head h / (H / H_qk) (contiguous groups).
 * With cu_seqlens (int32 [N+1]) B must be 1 and sequence n covers tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1; its state is slot n.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_EPS 1e-6

static double softplus(double x) {
  /* log(1 + e^x) without overflow */
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Normalise a K-vector into dst: x / sqrt(sum x^2 + eps). */
static void l2_normalise(const double* x, double* dst, int K) {
  double ss = 0.0;
  for (int i = 0; i < K; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss + KDA_ORACLE_EPS);
  for (int i = 0; i < K; ++i) dst[i] = x[i] * inv;
}

typedef struct {
  const double *q, *k, *v, *g_raw, *beta, *A_log;
  double scale;
  int gate_per_channel;
  int B, T, H_qk, H, K, V;
} kda_problem;

/*
 * Advance one chain through tokens [t0, t1) of batch row b, value head h.
 * S is K x V (S[kk*V + j]); it holds the entering state and is overwritten
 * with the leaving state.  Scratch must hold 4*K + 2*V doubles.
 */
static void run_chain(const kda_problem* P, int b, int h, int t0, int t1, double* S, double* out,
                      double* scratch) {
  const int K = P->K, V = P->V, H = P->H, H_qk = P->H_qk;
  const int group = H / H_qk;
  const int hq = h / group;
  double* qn = scratch;
  double* kn = qn + K;
  double* decay = kn + K;
  double* ktS = decay + K;  /* V entries: kn^T (Diag(e^g) S) */
  double* o = ktS + V;      /* V entries */
  const double a = exp(P->A_log[h]);
  for (int t = t0; t < t1; ++t) {
    const size_t tok = (size_t)b * P->T + t;
    l2_normalise(P->q + (tok * H_qk + hq) * K, qn, K);
    l2_normalise(P->k + (tok * H_qk + hq) * K, kn, K);
    if (P->gate_per_channel) {
      const double* gr = P->g_raw + (tok * H + h) * K;
      for (int i = 0; i < K; ++i) decay[i] = exp(-a * softplus(gr[i]));
    } else {
      const double gd = exp(-a * softplus(P->g_raw[tok * H + h]));
      for (int i = 0; i < K; ++i) decay[i] = gd;
    }
    const double beta = sigmoid(P->beta[tok * H + h]);
    const double* vt = P->v + (tok * H + h) * V;

    /* S' = Diag(exp(g_t)) S_{t-1}: row i of S scales by decay[i]. */
    for (int i = 0; i < K; ++i) {
      double* row = S + (size_t)i * V;
      for (int j = 0; j < V; ++j) row[j] *= decay[i];
    }
    /* kn^T S' */
    for (int j = 0; j < V; ++j) ktS[j] = 0.0;
    for (int i = 0; i < K; ++i) {
      const double* row = S + (size_t)i * V;
      for (int j = 0; j < V; ++j) ktS[j] += kn[i] * row[j];
    }
    /* S_t = S' - beta kn (kn^T S') + beta kn v^T */
    for (int i = 0; i < K; ++i) {
      double* row = S + (size_t)i * V;
      for (int j = 0; j < V; ++j) row[j] += -beta * kn[i] * ktS[j] + beta * kn[i] * vt[j];
    }
    /* o_t = scale * S_t^T qn */
    for (int j = 0; j < V; ++j) o[j] = 0.0;
    for (int i = 0; i < K; ++i) {
      const double* row = S + (size_t)i * V;
      for (int j = 0; j < V; ++j) o[j] += qn[i] * row[j];
    }
    double* ot = out + (tok * H + h) * V;
    for (int j = 0; j < V; ++j) ot[j] = P->scale * o[j];
  }
}

/*
 * Forward over all chains.  chain_mask (optional, length C*H) selects which
 * chains to compute; unselected chains leave out/final_state untouched.
 * Returns 0 on success, nonzero on bad arguments.
 */
int kda_oracle_fwd(const double* q, const double* k, const double* v, const double* g_raw,
                   const double* beta_logits, const double* A_log, double scale,
                   int gate_per_channel, const double* initial_state, double* out,
                   double* final_state, int B, int T, int H_qk, int H, int K, int V,
                   const int32_t* cu_seqlens, int N, const uint8_t* chain_mask, int nthreads) {
  if (B < 0 || T < 0 || H_qk <= 0 || H <= 0 || K <= 0 || V <= 0) return 1;
  if (H % H_qk != 0) return 2;
  if (cu_seqlens && B != 1) return 3;
  kda_problem P = {q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel,
                   B, T, H_qk, H, K, V};
  const int C = cu_seqlens ? N : B;
  const long nchains = (long)C * H;
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel num_threads(nt)
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(4 * K + 2 * V));
    if (!S || !scratch) {
#pragma omp atomic write
      err = 4;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long ch = 0; ch < nchains; ++ch) {
        if (chain_mask && !chain_mask[ch]) continue;
        const int c = (int)(ch / H), h = (int)(ch % H);
        int b, t0, t1;
        if (cu_seqlens) { b = 0; t0 = cu_seqlens[c]; t1 = cu_seqlens[c + 1]; }
        else { b = c; t0 = 0; t1 = T; }
        if (t0 < 0 || t1 < t0 || t1 > T) {
#pragma omp atomic write
          err = 5;
          continue;
        }
        /* S[kk][j] = state[c, h, j, kk] */
        const size_t sbase = ((size_t)c * H + h) * (size_t)V * K;
        for (int kk = 0; kk < K; ++kk)
          for (int j = 0; j < V; ++j)
            S[(size_t)kk * V + j] = initial_state ? initial_state[sbase + (size_t)j * K + kk] : 0.0;
        run_chain(&P, b, h, t0, t1, S, out, scratch);
        if (final_state)
          for (int kk = 0; kk < K; ++kk)
            for (int j = 0; j < V; ++j)
              final_state[sbase + (size_t)j * K + kk] = S[(size_t)kk * V + j];
      }
    }
    free(S);
    free(scratch);
  }
  return err;
}

/*
 * One decode step: each batch row b advances by exactly one token.
 * q, k: [B, H_qk, K]; v: [B, H, V]; g_raw: [B, H, K] or [B, H]; beta: [B, H];
 * state [B, H, V, K] is read and overwritten in place; out [B, H, V].
 * This is the forward recurrence with T = 1 and final_state = initial_state.
 */
int kda_oracle_decode(const double* q, const double* k, const double* v, const double* g_raw,
                      const double* beta_logits, const double* A_log, double scale,
                      int gate_per_channel, double* state, double* out, int B, int H_qk, int H,
                      int K, int V, int nthreads) {
  return kda_oracle_fwd(q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, state, out,
                        state, B, 1, H_qk, H, K, V, NULL, 0, NULL, nthreads);
}
