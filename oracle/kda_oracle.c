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

/*
 * Backward pass (reverse-mode derivative of the token loop above).
 *
 * The pages use the operator inside a trained model (the deep-read report,
 * section 3.4, training recipe) but print no gradient; what follows is the
 * chain rule applied to the four lines of the forward loop, taken in reverse
 * order, for the scalar loss
 *
 *   L = sum_t <dO_t, o_t> + <dS_T, S_T>
 *
 * so that the results are dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta and
 * dL/dS0 for given output and final-state cotangents dO and dS_T (dS_T absent
 * means zero).  With G = dL/dS_t carried backwards from dS_T, one token t is
 * (Sp = S_{t-1}, Sd = Diag(alpha_t) Sp, r = Sd^T k, e = v - r, S_t = Sd +
 * beta k e^T, o_t = S_t^T q):
 *
 *   G   += q dO_t^T              dq_t  = S_t dO_t
 *   de   = beta G^T k            dbeta = k^T G e       dk_t = beta G e
 *   dv_t = de                    dr    = -de
 *   dSd  = G + k dr^T            dk_t += Sd dr
 *   dlog_alpha_t[i] = sum_j dSd[i][j] Sd[i][j]        (d alpha = alpha d log alpha)
 *   G    = Diag(alpha_t) dSd
 *
 * and dS0 = G after the first token.  The states S_{t-1} are needed in
 * reverse order: the forward loop is run once keeping every CKPT-th state,
 * and each CKPT-token span is run forward again from its checkpoint when the
 * reverse sweep reaches it.  The recomputation repeats the forward loop's
 * operations in the same order, so the states are bitwise those of the
 * forward pass; checkpointing only bounds memory.
 */
#define CKPT 64

typedef struct {
  int T, H, dk, dv, h;
  const double *q, *k, *v, *la, *beta, *dO; /* offset to the sequence */
  const double *S0, *dST;                   /* [dk, dv] or NULL */
  double *dq, *dk_, *dv_, *dla, *dbeta;     /* offset to the sequence */
  double *dS0;                              /* [dk, dv] */
} bwd_job;

/* One token of the forward loop: S (= S_{t-1} on entry) becomes S_t; Sd
 * receives Diag(alpha_t) S_{t-1} and e the write residual v - Sd^T k. */
static void fwd_token(int dk, int dv, const double *kt, const double *vt, const double *lat, double bt,
                      double *S, double *Sd, double *e) {
  for (int i = 0; i < dk; ++i) {
    const double a = exp(lat[i]);
    for (int j = 0; j < dv; ++j) Sd[(size_t)i * dv + j] = S[(size_t)i * dv + j] * a;
  }
  for (int j = 0; j < dv; ++j) {
    double r = 0.0;
    for (int i = 0; i < dk; ++i) r += Sd[(size_t)i * dv + j] * kt[i];
    e[j] = vt[j] - r;
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = Sd[(size_t)i * dv + j] + bt * kt[i] * e[j];
}

static void run_pair_bwd(const bwd_job *J) {
  const int H = J->H, dk = J->dk, dv = J->dv, h = J->h, T = J->T;
  const size_t SZ = (size_t)dk * dv;
  const int nck = (T + CKPT - 1) / CKPT;
  /* ck[c] = S_{c CKPT - 1}, the state before token c CKPT */
  double *ck = (double *)malloc(sizeof(double) * SZ * (size_t)(nck > 0 ? nck : 1));
  double *span = (double *)malloc(sizeof(double) * SZ * (CKPT + 1)); /* states before and after each token */
  double *Sd = (double *)malloc(sizeof(double) * SZ);
  double *G = (double *)malloc(sizeof(double) * SZ);
  double *e = (double *)malloc(sizeof(double) * (size_t)dv);
  double *de = (double *)malloc(sizeof(double) * (size_t)dv);
  double *S = span; /* scratch state for the checkpoint sweep */
  if (J->S0) memcpy(S, J->S0, sizeof(double) * SZ);
  else memset(S, 0, sizeof(double) * SZ);
  for (int t = 0; t < T; ++t) {
    if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * SZ, S, sizeof(double) * SZ);
    fwd_token(dk, dv, J->k + ((size_t)t * H + h) * dk, J->v + ((size_t)t * H + h) * dv,
              J->la + ((size_t)t * H + h) * dk, J->beta[(size_t)t * H + h], S, Sd, e);
  }
  if (J->dST) memcpy(G, J->dST, sizeof(double) * SZ);
  else memset(G, 0, sizeof(double) * SZ);
  for (int c = nck - 1; c >= 0; --c) {
    const int t0 = c * CKPT, t1 = t0 + CKPT < T ? t0 + CKPT : T;
    /* span[m] = S_{t0 + m - 1}: the state before token t0 + m */
    memcpy(span, ck + (size_t)c * SZ, sizeof(double) * SZ);
    for (int t = t0; t < t1; ++t) {
      double *nxt = span + (size_t)(t - t0 + 1) * SZ;
      memcpy(nxt, span + (size_t)(t - t0) * SZ, sizeof(double) * SZ);
      fwd_token(dk, dv, J->k + ((size_t)t * H + h) * dk, J->v + ((size_t)t * H + h) * dv,
                J->la + ((size_t)t * H + h) * dk, J->beta[(size_t)t * H + h], nxt, Sd, e);
    }
    for (int t = t1 - 1; t >= t0; --t) {
      const double *qt = J->q + ((size_t)t * H + h) * dk;
      const double *kt = J->k + ((size_t)t * H + h) * dk;
      const double *vt = J->v + ((size_t)t * H + h) * dv;
      const double *lat = J->la + ((size_t)t * H + h) * dk;
      const double *dot = J->dO + ((size_t)t * H + h) * dv;
      const double bt = J->beta[(size_t)t * H + h];
      const double *Sp = span + (size_t)(t - t0) * SZ;     /* S_{t-1} */
      const double *St = span + (size_t)(t - t0 + 1) * SZ; /* S_t */
      double *dqt = J->dq + ((size_t)t * H + h) * dk;
      double *dkt = J->dk_ + ((size_t)t * H + h) * dk;
      double *dvt = J->dv_ + ((size_t)t * H + h) * dv;
      double *dlat = J->dla + ((size_t)t * H + h) * dk;
      /* rebuild Sd and e of this token from S_{t-1} */
      for (int i = 0; i < dk; ++i) {
        const double a = exp(lat[i]);
        for (int j = 0; j < dv; ++j) Sd[(size_t)i * dv + j] = Sp[(size_t)i * dv + j] * a;
      }
      for (int j = 0; j < dv; ++j) {
        double r = 0.0;
        for (int i = 0; i < dk; ++i) r += Sd[(size_t)i * dv + j] * kt[i];
        e[j] = vt[j] - r;
      }
      /* o_t = S_t^T q_t */
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          G[(size_t)i * dv + j] += qt[i] * dot[j];
          acc += St[(size_t)i * dv + j] * dot[j];
        }
        dqt[i] = acc;
      }
      /* S_t = Sd + beta k e^T */
      double db = 0.0;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += G[(size_t)i * dv + j] * kt[i];
        de[j] = bt * acc;
        db += acc * e[j];
      }
      J->dbeta[(size_t)t * H + h] = db;
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += G[(size_t)i * dv + j] * e[j];
        dkt[i] = bt * acc;
      }
      /* e = v - r, r = Sd^T k: dv = de, dr = -de */
      for (int j = 0; j < dv; ++j) dvt[j] = de[j];
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          G[(size_t)i * dv + j] -= kt[i] * de[j]; /* G is now dSd */
          acc -= Sd[(size_t)i * dv + j] * de[j];
        }
        dkt[i] += acc;
      }
      /* Sd = Diag(alpha) S_{t-1} */
      for (int i = 0; i < dk; ++i) {
        const double a = exp(lat[i]);
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          acc += G[(size_t)i * dv + j] * Sd[(size_t)i * dv + j];
          G[(size_t)i * dv + j] *= a;
        }
        dlat[i] = acc;
      }
    }
  }
  memcpy(J->dS0, G, sizeof(double) * SZ);
  free(ck); free(span); free(Sd); free(G); free(e); free(de);
}

typedef struct {
  bwd_job *jobs;
  int njobs;
  int next;
  pthread_mutex_t mu;
} bwd_queue;

static void *bwd_worker(void *arg) {
  bwd_queue *Q = (bwd_queue *)arg;
  for (;;) {
    pthread_mutex_lock(&Q->mu);
    const int i = Q->next++;
    pthread_mutex_unlock(&Q->mu);
    if (i >= Q->njobs) break;
    run_pair_bwd(&Q->jobs[i]);
  }
  return NULL;
}

/* Layouts as for kda_oracle_prefill; dO like o, dS_T and dS0 like S_T; the
 * gradients are laid out like the inputs they belong to.  dS_T and S0 may be
 * NULL (zero).  Returns the number of threads used, or -1 on a bad argument. */
int kda_oracle_backward(int N, const int32_t *cu_seqlens, int H, int dk, int dv,
                        const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *beta, const double *S0,
                        const double *dO, const double *dS_T,
                        double *dq, double *dk_, double *dv_, double *dlog_alpha,
                        double *dbeta, double *dS0, int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || !dS0) return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int njobs = N * H;
  bwd_job *jobs = (bwd_job *)calloc((size_t)(njobs > 0 ? njobs : 1), sizeof(bwd_job));
  for (int n = 0; n < N; ++n) {
    const size_t t0 = (size_t)cu_seqlens[n];
    for (int h = 0; h < H; ++h) {
      bwd_job *J = &jobs[n * H + h];
      const size_t sidx = ((size_t)n * H + h) * dk * dv;
      J->T = cu_seqlens[n + 1] - cu_seqlens[n];
      J->H = H; J->dk = dk; J->dv = dv; J->h = h;
      J->q = q + t0 * H * dk;
      J->k = k + t0 * H * dk;
      J->la = log_alpha + t0 * H * dk;
      J->v = v + t0 * H * dv;
      J->beta = beta + t0 * H;
      J->dO = dO + t0 * H * dv;
      J->S0 = S0 ? S0 + sidx : NULL;
      J->dST = dS_T ? dS_T + sidx : NULL;
      J->dq = dq + t0 * H * dk;
      J->dk_ = dk_ + t0 * H * dk;
      J->dv_ = dv_ + t0 * H * dv;
      J->dla = dlog_alpha + t0 * H * dk;
      J->dbeta = dbeta + t0 * H;
      J->dS0 = dS0 + sidx;
    }
  }
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > njobs) nthreads = njobs > 0 ? njobs : 1;
  bwd_queue Q;
  Q.jobs = jobs; Q.njobs = njobs; Q.next = 0;
  pthread_mutex_init(&Q.mu, NULL);
  if (nthreads == 1) {
    bwd_worker(&Q);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &Q);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&Q.mu);
  free(jobs);
  return nthreads;
}
