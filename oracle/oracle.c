/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact scaled-dot-product
 * attention and its gradient.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the GPU library; nothing in the product path calls it.
 *
 * What it computes is the plain definition, written out with every N x N
 * intermediate materialised, one (batch, head) slice at a time:
 *
 *   S = scale * Q K^T                       (Flash Attention notes, section 1,
 *                                            "standard attention", and the
 *                                            attention formula at its top)
 *   S_ij = -inf when causal and key j > query position i
 *   m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i),
 *   P_ij = exp(S_ij - m_i) / l_i            (section 2, 1.3: safe softmax,
 *                                            three passes: max, sum, divide)
 *   O = P V,  LSE_i = m_i + ln l_i          (section 3, part 3: the saved
 *                                            per-row statistic L = m + log l)
 *
 * and, given dO (backward derivation page, parts 3 and 4):
 *
 *   dV = P^T dO                  (conclusion 1 applied to O = P V)
 *   dP = dO V^T                  (same)
 *   D_i = sum_j P_ij dP_ij       (conclusion 2: rowsum(dP o P), by definition)
 *   dS = P o (dP - D)            (conclusion 2, row softmax Jacobian)
 *   dQ = scale * dS K            (conclusion 1 applied to S = scale Q K^T)
 *   dK = scale * dS^T Q
 *
 * The derivation page drops the 1/sqrt(d) factor "for brevity"; the Ascend
 * recompute article writes it into both dQ and dK. Here `scale` multiplies
 * Q K^T in the forward, so the chain rule puts the same factor on dQ and dK.
 *
 * The backward also returns D' = rowsum(dO o O) so that callers can check the
 * identity of the derivation page, part 5, against D computed by definition.
 *
 * Parallelism: OpenMP over independent rows (or columns for dK, dV). Every
 * output element is summed by one thread in a fixed order, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ENOMEM (-1)
#define ORACLE_EINVAL (-2)

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* Scores and softmax for M query rows at absolute positions qpos[] against N
 * keys. Fills S (M x N) and P (M x N), row max m and normaliser l (M each). */
static void scores_and_softmax(int M, const int *qpos, const double *Q, int N,
                               const double *K, int d, double scale, int causal,
                               double *S, double *P, double *m, double *l) {
  long long i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    const double *q = Q + (size_t)i * d;
    double *s = S + (size_t)i * N;
    double *p = P + (size_t)i * N;
    /* S_ij = scale * q_i . k_j, with the causal mask */
    for (int j = 0; j < N; ++j) {
      if (causal && j > qpos[i]) {
        s[j] = -INFINITY;
        continue;
      }
      const double *k = K + (size_t)j * d;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += q[c] * k[c];
      s[j] = scale * acc;
    }
    /* pass 1: row max */
    double mi = -INFINITY;
    for (int j = 0; j < N; ++j)
      if (s[j] > mi) mi = s[j];
    /* pass 2: normaliser; exp(-inf) = 0 for masked entries */
    double li = 0.0;
    for (int j = 0; j < N; ++j) li += exp(s[j] - mi);
    /* pass 3: normalised probabilities */
    for (int j = 0; j < N; ++j) p[j] = exp(s[j] - mi) / li;
    m[i] = mi;
    l[i] = li;
  }
}

/* Forward for M query rows (absolute positions qpos[0..M)) of one slice.
 * Q is M x d, K and V are N x d, O is M x d, LSE is M. P_out, if not NULL,
 * receives P (M x N). Rows whose keys are all masked (only possible when a
 * query position is negative) get LSE = -inf and O = NaN, as the definition
 * gives 0/0 there. */
int oracle_fwd_rows(int M, const int *qpos, const double *Q, int N,
                    const double *K, const double *V, int d, double scale,
                    int causal, double *O, double *LSE, double *P_out) {
  if (M <= 0 || N <= 0 || d <= 0 || !qpos || !Q || !K || !V || !O || !LSE)
    return ORACLE_EINVAL;
  double *S = (double *)malloc(sizeof(double) * (size_t)M * N);
  double *P = P_out ? P_out : (double *)malloc(sizeof(double) * (size_t)M * N);
  double *m = (double *)malloc(sizeof(double) * (size_t)M);
  double *l = (double *)malloc(sizeof(double) * (size_t)M);
  if (!S || !P || !m || !l) {
    free(S);
    if (!P_out) free(P);
    free(m);
    free(l);
    return ORACLE_ENOMEM;
  }
  scores_and_softmax(M, qpos, Q, N, K, d, scale, causal, S, P, m, l);
  long long i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    double *o = O + (size_t)i * d;
    const double *p = P + (size_t)i * N;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    /* O_i = sum_j P_ij V_j */
    for (int j = 0; j < N; ++j) {
      const double pij = p[j];
      const double *v = V + (size_t)j * d;
      for (int c = 0; c < d; ++c) o[c] += pij * v[c];
    }
    LSE[i] = m[i] + log(l[i]);
  }
  free(S);
  if (!P_out) free(P);
  free(m);
  free(l);
  return ORACLE_OK;
}

/* Forward for a whole slice: query i sits at position i. */
int oracle_fwd(int N, const double *Q, const double *K, const double *V, int d,
               double scale, int causal, double *O, double *LSE) {
  if (N <= 0) return ORACLE_EINVAL;
  int *qpos = (int *)malloc(sizeof(int) * (size_t)N);
  if (!qpos) return ORACLE_ENOMEM;
  for (int i = 0; i < N; ++i) qpos[i] = i;
  int rc = oracle_fwd_rows(N, qpos, Q, N, K, V, d, scale, causal, O, LSE, NULL);
  free(qpos);
  return rc;
}

/* Backward for a whole slice (N queries at positions 0..N-1, N keys).
 * Outputs dQ, dK, dV (N x d each), D = rowsum(dP o P) and
 * Dprime = rowsum(dO o O) (N each). dS_out, if not NULL, receives dS (N x N). */
int oracle_bwd(int N, const double *Q, const double *K, const double *V,
               const double *dO, int d, double scale, int causal, double *dQ,
               double *dK, double *dV, double *D, double *Dprime,
               double *dS_out) {
  if (N <= 0 || d <= 0 || !Q || !K || !V || !dO || !dQ || !dK || !dV || !D ||
      !Dprime)
    return ORACLE_EINVAL;
  const size_t NN = (size_t)N * N;
  int *qpos = (int *)malloc(sizeof(int) * (size_t)N);
  double *S = (double *)malloc(sizeof(double) * NN);
  double *P = (double *)malloc(sizeof(double) * NN);
  double *dP = (double *)malloc(sizeof(double) * NN);
  double *dS = dS_out ? dS_out : (double *)malloc(sizeof(double) * NN);
  double *m = (double *)malloc(sizeof(double) * (size_t)N);
  double *l = (double *)malloc(sizeof(double) * (size_t)N);
  double *O = (double *)malloc(sizeof(double) * (size_t)N * d);
  if (!qpos || !S || !P || !dP || !dS || !m || !l || !O) {
    free(qpos);
    free(S);
    free(P);
    free(dP);
    if (!dS_out) free(dS);
    free(m);
    free(l);
    free(O);
    return ORACLE_ENOMEM;
  }
  for (int i = 0; i < N; ++i) qpos[i] = i;

  /* Recompute the forward: S, P and O. */
  scores_and_softmax(N, qpos, Q, N, K, d, scale, causal, S, P, m, l);
  long long i, j;
#pragma omp parallel for schedule(static)
  for (i = 0; i < N; ++i) {
    double *o = O + (size_t)i * d;
    const double *p = P + (size_t)i * N;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int jj = 0; jj < N; ++jj) {
      const double *v = V + (size_t)jj * d;
      for (int c = 0; c < d; ++c) o[c] += p[jj] * v[c];
    }
  }

  /* dP = dO V^T, D = rowsum(dP o P), dS = P o (dP - D), D' = rowsum(dO o O) */
#pragma omp parallel for schedule(static)
  for (i = 0; i < N; ++i) {
    const double *g = dO + (size_t)i * d;
    double *dp = dP + (size_t)i * N;
    const double *p = P + (size_t)i * N;
    double *ds = dS + (size_t)i * N;
    for (int jj = 0; jj < N; ++jj) {
      const double *v = V + (size_t)jj * d;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += g[c] * v[c];
      dp[jj] = acc;
    }
    double Di = 0.0;
    for (int jj = 0; jj < N; ++jj) Di += dp[jj] * p[jj];
    D[i] = Di;
    for (int jj = 0; jj < N; ++jj) ds[jj] = p[jj] * (dp[jj] - Di);
    const double *o = O + (size_t)i * d;
    double Dp = 0.0;
    for (int c = 0; c < d; ++c) Dp += g[c] * o[c];
    Dprime[i] = Dp;
  }

  /* dQ = scale * dS K */
#pragma omp parallel for schedule(static)
  for (i = 0; i < N; ++i) {
    double *gq = dQ + (size_t)i * d;
    const double *ds = dS + (size_t)i * N;
    for (int c = 0; c < d; ++c) gq[c] = 0.0;
    for (int jj = 0; jj < N; ++jj) {
      const double *k = K + (size_t)jj * d;
      for (int c = 0; c < d; ++c) gq[c] += ds[jj] * k[c];
    }
    for (int c = 0; c < d; ++c) gq[c] *= scale;
  }

  /* dV = P^T dO and dK = scale * dS^T Q, one key row j per iteration */
#pragma omp parallel for schedule(static)
  for (j = 0; j < N; ++j) {
    double *gv = dV + (size_t)j * d;
    double *gk = dK + (size_t)j * d;
    for (int c = 0; c < d; ++c) {
      gv[c] = 0.0;
      gk[c] = 0.0;
    }
    for (int ii = 0; ii < N; ++ii) {
      const double pij = P[(size_t)ii * N + j];
      const double dsij = dS[(size_t)ii * N + j];
      const double *g = dO + (size_t)ii * d;
      const double *q = Q + (size_t)ii * d;
      for (int c = 0; c < d; ++c) {
        gv[c] += pij * g[c];
        gk[c] += dsij * q[c];
      }
    }
    for (int c = 0; c < d; ++c) gk[c] *= scale;
  }

  free(qpos);
  free(S);
  free(P);
  free(dP);
  if (!dS_out) free(dS);
  free(m);
  free(l);
  free(O);
  return ORACLE_OK;
}

/* Merge of partial results over disjoint key sets ("Flash Attention" notes,
 * section 2, parts 3.1 and 4.1: the two-block merge of (m, l) and of the
 * unnormalised output O~, which is associative, so blocks may be combined in
 * any grouping).
 *
 * Part s holds, for each of `rows` rows, a normalised output O_s (d values)
 * and its log-normaliser LSE_s. It enters the merge as the block
 * (m = LSE_s, l = 1, O~ = O_s), for which m + log l = LSE_s and O~ / l = O_s.
 * Parts are folded left to right:
 *   m = max(m_A, m_B),  l = l_A e^(m_A - m) + l_B e^(m_B - m),
 *   O~ = O~_A e^(m_A - m) + O~_B e^(m_B - m),
 * and the result is O = O~ / l, LSE = m + log l. A part with LSE_s = -inf
 * (no visible key) contributes nothing; a row whose parts are all -inf gets
 * O = 0 and LSE = -inf.
 * Layout: O_parts [parts][rows][d], LSE_parts [parts][rows]; O [rows][d],
 * LSE [rows]. */
int oracle_lse_merge(int parts, int rows, int d, const double *O_parts,
                     const double *LSE_parts, double *O, double *LSE) {
  if (parts <= 0 || rows <= 0 || d <= 0 || !O_parts || !LSE_parts || !O || !LSE)
    return ORACLE_EINVAL;
  int i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < rows; ++i) {
    double m = -INFINITY, l = 0.0;
    double *acc = O + (size_t)i * d;
    for (int c = 0; c < d; ++c) acc[c] = 0.0;
    for (int s = 0; s < parts; ++s) {
      const double mb = LSE_parts[(size_t)s * rows + i];
      if (mb == -INFINITY) continue;
      const double *ob = O_parts + ((size_t)s * rows + i) * d;
      const double mn = m > mb ? m : mb;
      const double fa = (m == -INFINITY) ? 0.0 : exp(m - mn);
      const double fb = exp(mb - mn);
      l = l * fa + 1.0 * fb;
      for (int c = 0; c < d; ++c) acc[c] = acc[c] * fa + ob[c] * fb;
      m = mn;
    }
    if (l > 0.0) {
      for (int c = 0; c < d; ++c) acc[c] /= l;
      LSE[i] = m + log(l);
    } else {
      LSE[i] = -INFINITY;
    }
  }
  return ORACLE_OK;
}
