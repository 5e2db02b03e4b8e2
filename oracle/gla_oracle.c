/*
 * gla_oracle.c -- plain fp64 CPU oracle of the Simple GLA recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the GPU product path may include,
 * link or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (the plain definition, token by token, in fp64):
 *
 *   Laplace 3B / Trainium2 page ("Beyond the KV cache: training and serving
 *   i14's Laplace 3B linear attention model on AWS Trainium2"), section
 *   "GLA mixer": every head h keeps a dk x dv matrix state that is decayed
 *   and then receives the new key/value outer product at every token, and the
 *   token's output reads that state with the query. The page's formulas are
 *   images that did not survive extraction; the reading used here is
 *
 *       S_t = lambda_h * S_{t-1} + k_t^T v_t          (k_t, q_t: 1 x dk rows)
 *       o_t = scale * q_t S_t                         (readout AFTER update)
 *
 *   with lambda_h a fixed per-head decay (section "Decay scheme": fixed at
 *   initialisation, not learned, geometric across heads).
 *
 * The chunked form used on the GPU is an exact rearrangement of this
 * recurrence (same page, "Challenge 1", chunk-internal output plus state
 * advance); the oracle has no chunks at all.
 *
 * Decode (same page, "Inference optimisation on Trainium2": one fixed state
 * page per sequence that is read, updated and written back per token) is one
 * iteration of the same loop on a state array.
 *
 * Numbers: inputs arrive as fp32 values (bf16 inputs are widened exactly
 * before they get here); every product and sum is done in double. Summation
 * of the readout is in ascending key-dimension index.
 *
 * Parallelism: only across independent (sequence, head) chains; the token
 * loop of each chain is sequential.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

/* One (sequence, head) chain of the recurrence.
 *   q, k : row stride `row_k` floats between consecutive tokens (H*dk)
 *   v    : row stride `row_v` floats (H*dv)
 *   o    : row stride `row_v` doubles
 *   S    : dk*dv doubles, in/out (the running state)
 *   acc  : dv doubles of scratch
 */
static void chain(int64_t ntok, int dk, int dv, const float *q, const float *k,
                  const float *v, int64_t row_k, int64_t row_v, double lam,
                  double scale, double *S, double *o, double *acc) {
  for (int64_t t = 0; t < ntok; ++t) {
    const float *qt = q + t * row_k;
    const float *kt = k + t * row_k;
    const float *vt = v + t * row_v;
    /* state update: decay, then add the outer product k_t^T v_t */
    for (int i = 0; i < dk; ++i) {
      const double ki = (double)kt[i];
      double *Si = S + (int64_t)i * dv;
      for (int j = 0; j < dv; ++j) Si[j] = lam * Si[j] + ki * (double)vt[j];
    }
    /* readout of the updated state: o_t[j] = scale * sum_i q_t[i] S[i][j],
       accumulated over i in ascending order for every j */
    for (int j = 0; j < dv; ++j) acc[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
      const double qi = (double)qt[i];
      const double *Si = S + (int64_t)i * dv;
      for (int j = 0; j < dv; ++j) acc[j] += qi * Si[j];
    }
    if (o) {
      double *ot = o + t * row_v;
      for (int j = 0; j < dv; ++j) ot[j] = scale * acc[j];
    }
  }
}

typedef struct {
  int N, H, dk, dv;
  const int64_t *cu;
  const float *q, *k, *v, *decay;
  const double *s0;
  double scale;
  double *o, *s_final;
  int64_t next; /* next (n,h) work index, taken under the mutex */
  pthread_mutex_t mu;
  int failed;
} job_t;

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  const int dk = J->dk, dv = J->dv, H = J->H;
  const int64_t sz = (int64_t)dk * dv;
  double *S = (double *)malloc(sizeof(double) * (size_t)(sz + dv));
  if (!S) {
    pthread_mutex_lock(&J->mu);
    J->failed = 1;
    pthread_mutex_unlock(&J->mu);
    return NULL;
  }
  double *acc = S + sz;
  const int64_t total = (int64_t)J->N * H;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int64_t w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= total) break;
    const int n = (int)(w / H), h = (int)(w % H);
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
    /* initial state: S0[n,h] or zeros */
    if (J->s0) {
      memcpy(S, J->s0 + ((int64_t)n * H + h) * sz, sizeof(double) * (size_t)sz);
    } else {
      memset(S, 0, sizeof(double) * (size_t)sz);
    }
    const int64_t row_k = (int64_t)H * dk, row_v = (int64_t)H * dv;
    chain(t1 - t0, dk, dv, J->q + t0 * row_k + (int64_t)h * dk,
          J->k + t0 * row_k + (int64_t)h * dk,
          J->v + t0 * row_v + (int64_t)h * dv, row_k, row_v,
          (double)J->decay[h], J->scale, S,
          J->o ? J->o + t0 * row_v + (int64_t)h * dv : NULL, acc);
    if (J->s_final)
      memcpy(J->s_final + ((int64_t)n * H + h) * sz, S,
             sizeof(double) * (size_t)sz);
  }
  free(S);
  return NULL;
}

static int run_threads(job_t *J, int nthreads) {
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads <= 0) nthreads = 1;
  const int64_t total = (int64_t)J->N * J->H;
  if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
  pthread_mutex_init(&J->mu, NULL);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, worker, J) != 0) break;
    ++started;
  }
  if (started == 0) worker(J); /* no thread could start: run inline */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J->mu);
  return J->failed ? -2 : 0;
}

/*
 * Packed variable-length forward. Sequence n owns tokens [cu[n], cu[n+1]) of
 * the packed arrays and starts from s0[n] (or zeros when s0 is NULL).
 *   q, k : [total, H, dk] fp32     v : [total, H, dv] fp32
 *   decay: [H] fp32 (the exact values the GPU receives)
 *   s0   : [N, H, dk, dv] fp64 or NULL (fp64 so that a carried state can be
 *          handed back in without rounding)
 *   o    : [total, H, dv] fp64 or NULL      s_final : [N, H, dk, dv] fp64 or NULL
 * A fixed-length batch [B, T, ...] is the case cu[n] = n*T.
 * Returns 0, -1 on bad arguments, -2 when memory runs out.
 */
int oracle_gla_varlen(int N, const int64_t *cu, int H, int dk, int dv,
                      const float *q, const float *k, const float *v,
                      const float *decay, double scale, const double *s0,
                      double *o, double *s_final, int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu || !decay) return -1;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return -1;
  if (cu[N] > cu[0] && (!q || !k || !v)) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.cu = cu;
  J.q = q; J.k = k; J.v = v; J.decay = decay; J.s0 = s0;
  J.scale = scale; J.o = o; J.s_final = s_final;
  return run_threads(&J, nthreads);
}

/*
 * One decode step for N independent sequences: for each (n, h),
 *   state[n,h] <- decay[h] * state[n,h] + k[n,h]^T v[n,h]   (in place, fp64)
 *   o[n,h,:]   <- scale * q[n,h] state[n,h]                 (after the update)
 *   q, k : [N, H, dk] fp32    v : [N, H, dv] fp32
 *   state: [N, H, dk, dv] fp64 in/out      o : [N, H, dv] fp64
 */
typedef struct {
  int N, H, dk, dv;
  const float *q, *k, *v, *decay;
  double scale;
  double *state, *o;
  int64_t next;
  pthread_mutex_t mu;
  int failed;
} djob_t;

static void *dworker(void *arg) {
  djob_t *J = (djob_t *)arg;
  const int dk = J->dk, dv = J->dv, H = J->H;
  const int64_t sz = (int64_t)dk * dv;
  double *acc = (double *)malloc(sizeof(double) * (size_t)dv);
  if (!acc) {
    pthread_mutex_lock(&J->mu);
    J->failed = 1;
    pthread_mutex_unlock(&J->mu);
    return NULL;
  }
  const int64_t total = (int64_t)J->N * H;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int64_t w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= total) break;
    /* one token of one chain: the same loop body as the forward */
    chain(1, dk, dv, J->q + w * dk, J->k + w * dk, J->v + w * dv, dk, dv,
          (double)J->decay[w % H], J->scale, J->state + w * sz,
          J->o + w * dv, acc);
  }
  free(acc);
  return NULL;
}

int oracle_gla_decode(int N, int H, int dk, int dv, const float *q,
                      const float *k, const float *v, const float *decay,
                      double scale, double *state, double *o, int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !decay || !state || !o ||
      !q || !k || !v)
    return -1;
  djob_t J;
  memset(&J, 0, sizeof(J));
  J.N = N; J.H = H; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.decay = decay; J.scale = scale;
  J.state = state; J.o = o;
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads <= 0) nthreads = 1;
  if (nthreads > (int64_t)N * H) nthreads = (int)((int64_t)N * H > 0 ? (int64_t)N * H : 1);
  pthread_mutex_init(&J.mu, NULL);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, dworker, &J) != 0) break;
    ++started;
  }
  if (started == 0) dworker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return J.failed ? -2 : 0;
}


/*
 * Backward of the same recurrence (gradients by the chain rule, token by
 * token). The page trains the model, and its "Challenge 3" section
 * differentiates through every sequential state update of the chain; here
 * that is written out directly. With upstream gradients dO_t = dL/do_t and
 * dS_fin = dL/dS_final (zero when not given):
 *
 *   forward sweep (recomputes S_t):   dq_t = scale * dO_t S_t^T
 *   backward sweep, R = dS_fin, then for t = T-1 .. 0:
 *       G_t  = R + scale * q_t^T dO_t      (dL/dS_t, all later uses included)
 *       dk_t = v_t G_t^T                   (dk_t[i] = sum_j G_t[i][j] v_t[j])
 *       dv_t = k_t G_t                     (dv_t[j] = sum_i k_t[i] G_t[i][j])
 *       R    = lambda * G_t
 *   dS0 = R after token 0.
 * Sums run over the contracted index in ascending order, in double.
 */
typedef struct {
  int N, H, dk, dv;
  const int64_t *cu;
  const float *q, *k, *v, *decay, *dout;
  const double *s0, *ds_fin;
  double scale;
  double *dq, *dkk, *dvv, *ds0;
  int64_t next;
  pthread_mutex_t mu;
  int failed;
} bjob_t;

static void *bworker(void *arg) {
  bjob_t *J = (bjob_t *)arg;
  const int dk = J->dk, dv = J->dv, H = J->H;
  const int64_t sz = (int64_t)dk * dv;
  double *S = (double *)malloc(sizeof(double) * (size_t)(2 * sz));
  if (!S) {
    pthread_mutex_lock(&J->mu);
    J->failed = 1;
    pthread_mutex_unlock(&J->mu);
    return NULL;
  }
  double *G = S + sz;
  const int64_t total = (int64_t)J->N * H;
  const int64_t row_k = (int64_t)H * dk, row_v = (int64_t)H * dv;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int64_t w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= total) break;
    const int n = (int)(w / H), h = (int)(w % H);
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
    const double lam = (double)J->decay[h];
    /* forward sweep: S_t, then dq_t = scale * dO_t S_t^T */
    if (J->s0)
      memcpy(S, J->s0 + ((int64_t)n * H + h) * sz, sizeof(double) * (size_t)sz);
    else
      memset(S, 0, sizeof(double) * (size_t)sz);
    for (int64_t t = t0; t < t1; ++t) {
      const float *kt = J->k + t * row_k + (int64_t)h * dk;
      const float *vt = J->v + t * row_v + (int64_t)h * dv;
      const float *dot = J->dout + t * row_v + (int64_t)h * dv;
      double *dqt = J->dq + t * row_k + (int64_t)h * dk;
      for (int i = 0; i < dk; ++i) {
        double *Si = S + (int64_t)i * dv;
        const double ki = (double)kt[i];
        for (int j = 0; j < dv; ++j) Si[j] = lam * Si[j] + ki * (double)vt[j];
        double a = 0.0;
        for (int j = 0; j < dv; ++j) a += (double)dot[j] * Si[j];
        dqt[i] = J->scale * a;
      }
    }
    /* backward sweep: R carries dL/dS from the later tokens */
    if (J->ds_fin)
      memcpy(G, J->ds_fin + ((int64_t)n * H + h) * sz, sizeof(double) * (size_t)sz);
    else
      memset(G, 0, sizeof(double) * (size_t)sz);
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const float *qt = J->q + t * row_k + (int64_t)h * dk;
      const float *kt = J->k + t * row_k + (int64_t)h * dk;
      const float *vt = J->v + t * row_v + (int64_t)h * dv;
      const float *dot = J->dout + t * row_v + (int64_t)h * dv;
      double *dkt = J->dkk + t * row_k + (int64_t)h * dk;
      double *dvt = J->dvv + t * row_v + (int64_t)h * dv;
      /* G_t = R + scale * q_t^T dO_t (R is in G on entry) */
      for (int i = 0; i < dk; ++i) {
        double *Gi = G + (int64_t)i * dv;
        const double sq = J->scale * (double)qt[i];
        for (int j = 0; j < dv; ++j) Gi[j] += sq * (double)dot[j];
      }
      for (int i = 0; i < dk; ++i) {
        const double *Gi = G + (int64_t)i * dv;
        double a = 0.0;
        for (int j = 0; j < dv; ++j) a += Gi[j] * (double)vt[j];
        dkt[i] = a;
      }
      for (int j = 0; j < dv; ++j) {
        double a = 0.0;
        for (int i = 0; i < dk; ++i) a += (double)kt[i] * G[(int64_t)i * dv + j];
        dvt[j] = a;
      }
      /* R = lambda * G_t for the token before */
      for (int64_t e = 0; e < sz; ++e) G[e] *= lam;
    }
    if (J->ds0)
      memcpy(J->ds0 + ((int64_t)n * H + h) * sz, G, sizeof(double) * (size_t)sz);
  }
  free(S);
  return NULL;
}

/*
 * Packed variable-length backward: the inputs of oracle_gla_varlen plus
 *   dout   : [total, H, dv] fp32 (dL/do)
 *   ds_fin : [N, H, dk, dv] fp64 or NULL (dL/dS_final; NULL means zero)
 * and outputs dq, dk : [total, H, dk] fp64, dv : [total, H, dv] fp64,
 * ds0 : [N, H, dk, dv] fp64 or NULL.
 * Returns 0, -1 on bad arguments, -2 when memory runs out.
 */
int oracle_gla_bwd_varlen(int N, const int64_t *cu, int H, int dk, int dv,
                          const float *q, const float *k, const float *v,
                          const float *decay, double scale, const double *s0,
                          const float *dout, const double *ds_fin, double *dq,
                          double *dkk, double *dvv, double *ds0, int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu || !decay) return -1;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return -1;
  if (cu[N] > cu[0] && (!q || !k || !v || !dout || !dq || !dkk || !dvv)) return -1;
  bjob_t J;
  memset(&J, 0, sizeof(J));
  J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.cu = cu;
  J.q = q; J.k = k; J.v = v; J.decay = decay; J.dout = dout;
  J.s0 = s0; J.ds_fin = ds_fin; J.scale = scale;
  J.dq = dq; J.dkk = dkk; J.dvv = dvv; J.ds0 = ds0;
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads <= 0) nthreads = 1;
  const int64_t total = (int64_t)N * H;
  if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
  pthread_mutex_init(&J.mu, NULL);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, bworker, &J) != 0) break;
    ++started;
  }
  if (started == 0) bworker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return J.failed ? -2 : 0;
}
