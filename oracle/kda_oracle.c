/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the package's smoke check and the
 * benchmark's CPU-baseline leg have an obviously correct result to compare
 * the HIP kernels against.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (per sequence n and head h, all arithmetic in double):
 *
 *   S <- S0 (zero when absent)
 *   for each token t of the sequence:
 *       S <- Diag(exp(log_alpha_t)) S         forget, one rate per key channel
 *       r <- S^T k_t                          read back the decayed state
 *       S <- S + beta_t k_t (v_t - r)^T       erase along k_t, then write v_t
 *       o_t <- S^T q_t                        output reads the updated state
 *
 * The last three lines together are S_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
 * S_{t-1} + beta_t k_t v_t^T, the KDA update:
 *   - "Kimi Linear: An Expressive, Efficient Attention Architecture" deep-read
 *     report (zako-mio knowledge base), section 2.3: a per-channel diagonal
 *     gate Diag(alpha_t) replaces the scalar gate of the gated delta rule; the
 *     three factors are, in order, channel-wise forgetting, targeted erasure
 *     (I - beta k k^T) and the write beta k v^T.  Section 2.2: the delta rule
 *     subtracts the old content along the key before writing.
 *   - zhaixingw.cn news explainer, section on KDA turning the forget gate into
 *     a vector: alpha_t has one entry per key channel (dk entries), and the
 *     scalar-gate (Gated DeltaNet) update applies the gate before the erase.
 *   - The state is dk x dv (key dimension by value dimension); Diag(alpha)
 *     scales rows, i.e. key channels.
 * Reading taken where the pages are loose: the explainer's KDA line writes a
 * transposed state with a read-back of the undecayed state; this oracle
 * follows the ordered component description (decay, erase, write), which
 * reads back the decayed state.  Output is S_t^T q_t with no extra scale.
 *
 * Layouts (row-major, contiguous):
 *   q, k, log_alpha : [T_tot, H, dk]      v, o : [T_tot, H, dv]
 *   beta            : [T_tot, H]          S0, S_T : [N, H, dk, dv]
 *   cu_seqlens      : [N + 1], cu[0] = 0, non-decreasing; sequence n owns
 *                     tokens cu[n] .. cu[n+1]-1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
  int T, H, dk, dv;
  const double *q, *k, *v, *la, *beta; /* already offset to the sequence */
  const double *S0;                    /* [dk, dv] for this (n, h) or NULL */
  double *o;                           /* already offset to the sequence */
  double *S;                           /* [dk, dv] output state for (n, h) */
  int h;
} pair_job;

/* One (sequence, head): the token loop above, with S held in `S`. */
static void run_pair(const pair_job *J) {
  const int H = J->H, dk = J->dk, dv = J->dv, h = J->h;
  double *S = J->S;
  double *r = (double *)malloc(sizeof(double) * (size_t)dv);
  if (J->S0) {
    if (J->S0 != S) memcpy(S, J->S0, sizeof(double) * (size_t)dk * dv);
  } else
    memset(S, 0, sizeof(double) * (size_t)dk * dv);
  for (int t = 0; t < J->T; ++t) {
    const double *qt = J->q + ((size_t)t * H + h) * dk;
    const double *kt = J->k + ((size_t)t * H + h) * dk;
    const double *lat = J->la + ((size_t)t * H + h) * dk;
    const double *vt = J->v + ((size_t)t * H + h) * dv;
    const double bt = J->beta[(size_t)t * H + h];
    double *ot = J->o + ((size_t)t * H + h) * dv;
    /* forget: row i of S (key channel i) is scaled by alpha_t[i] */
    for (int i = 0; i < dk; ++i) {
      const double a = exp(lat[i]);
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
    }
    /* read back the decayed state along k_t */
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) r[j] += S[(size_t)i * dv + j] * kt[i];
    /* erase-then-write: add beta k (v - r)^T */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bt * kt[i] * (vt[j] - r[j]);
    /* output from the updated state */
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];
  }
  free(r);
}

typedef struct {
  pair_job *jobs;
  int njobs;
  int next;
  pthread_mutex_t mu;
} job_queue;

static void *worker(void *arg) {
  job_queue *Q = (job_queue *)arg;
  for (;;) {
    pthread_mutex_lock(&Q->mu);
    const int i = Q->next++;
    pthread_mutex_unlock(&Q->mu);
    if (i >= Q->njobs) break;
    run_pair(&Q->jobs[i]);
  }
  return NULL;
}

/* Returns the number of threads used, or -1 on a bad argument. */
int kda_oracle_prefill(int N, const int32_t *cu_seqlens, int H, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *S0, double *o, double *S_T, int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || !S_T) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  if (cu_seqlens[0] != 0) return -1;
  const int njobs = N * H;
  pair_job *jobs = (pair_job *)calloc((size_t)(njobs > 0 ? njobs : 1), sizeof(pair_job));
  for (int n = 0; n < N; ++n) {
    const size_t t0 = (size_t)cu_seqlens[n];
    for (int h = 0; h < H; ++h) {
      pair_job *J = &jobs[n * H + h];
      J->T = cu_seqlens[n + 1] - cu_seqlens[n];
      J->H = H; J->dk = dk; J->dv = dv; J->h = h;
      J->q = q + t0 * H * dk;
      J->k = k + t0 * H * dk;
      J->la = log_alpha + t0 * H * dk;
      J->v = v + t0 * H * dv;
      J->beta = beta + t0 * H;
      J->o = o + t0 * H * dv;
      J->S0 = S0 ? S0 + ((size_t)n * H + h) * dk * dv : NULL;
      J->S = S_T + ((size_t)n * H + h) * dk * dv;
    }
  }
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > njobs) nthreads = njobs > 0 ? njobs : 1;
  job_queue Q;
  Q.jobs = jobs; Q.njobs = njobs; Q.next = 0;
  pthread_mutex_init(&Q.mu, NULL);
  if (nthreads == 1) {
    worker(&Q);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &Q);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&Q.mu);
  free(jobs);
  return nthreads;
}

/*
 * One decode step for a batch of B independent states: exactly one iteration
 * of the token loop for every (b, h), with S updated in place.
 *   q, k, log_alpha : [B, H, dk]   v, o : [B, H, dv]   beta : [B, H]
 *   S               : [B, H, dk, dv], read as S_{t-1}, written as S_t.
 */
int kda_oracle_decode_step(int B, int H, int dk, int dv, const double *q,
                           const double *k, const double *v,
                           const double *log_alpha, const double *beta,
                           double *S, double *o, int nthreads) {
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const int njobs = B * H;
  pair_job *jobs = (pair_job *)calloc((size_t)(njobs > 0 ? njobs : 1), sizeof(pair_job));
  /* run_pair starts from S0 and writes S; here S0 is S itself (in place) */
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      pair_job *J = &jobs[b * H + h];
      /* batch row b is a one-token sequence whose head stride is H */
      J->T = 1; J->H = H; J->dk = dk; J->dv = dv; J->h = h;
      J->q = q + (size_t)b * H * dk;
      J->k = k + (size_t)b * H * dk;
      J->la = log_alpha + (size_t)b * H * dk;
      J->v = v + (size_t)b * H * dv;
      J->beta = beta + (size_t)b * H;
      J->o = o + (size_t)b * H * dv;
      J->S0 = S + ((size_t)b * H + h) * dk * dv;
      J->S = S + ((size_t)b * H + h) * dk * dv;
    }
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > njobs) nthreads = njobs > 0 ? njobs : 1;
  job_queue Q;
  Q.jobs = jobs; Q.njobs = njobs; Q.next = 0;
  pthread_mutex_init(&Q.mu, NULL);
  if (nthreads == 1) {
    worker(&Q);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &Q);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&Q.mu);
  free(jobs);
  return nthreads;
}
