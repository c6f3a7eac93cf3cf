/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the gated delta rule (GDN) and of its
 * per-channel-decay variant (KDA, Kimi Delta Attention).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the HIP
 * path is compared against.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or helper
 * with the HIP library, and the HIP library never calls it.
 *
 * What it computes (token by token, one (batch, head) stream at a time, in fp64):
 *
 *   S <- S0 (or zeros)                        S is d_v x d_k (row = value channel)
 *   for t = 1..T:
 *     GDN:  S <- alpha_t * S                  alpha_t = exp(log_alpha_t), a scalar
 *     KDA:  S <- S * Diag(alpha_t)            alpha_t in (0,1)^{d_k}: column j scaled
 *     r   = S k_t                             read with the decayed state
 *     S  <- S + beta_t (v_t - r) k_t^T        delta correction
 *     o_t = S q_t                             the query reads the updated state
 *     every ckpt_every tokens: snapshot S
 *
 * Sources (pages on the gated delta rule):
 *  - "From Traditional Attention to hybrid ones" (jq-wei.github.io), section 5
 *    "From DeltaNet to Gated DeltaNet": first decay the previous memory by alpha_t,
 *    then apply the delta update to the decayed state; the query reads the updated
 *    state o_t = S_t q_t; the state is d_v x d_k.  Section 7 gives KDA as
 *    S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, D_t = Diag(alpha_t).
 *  - "Attention, Part 4: Linear Attention, Gated DeltaNet and Hybrid Models"
 *    (ishwarj.com), section 6: the order forget -> correct (delta) -> read, with
 *    q, k of shape (H, T, d_k), v of shape (H, T, d_v); "Where alpha and beta come
 *    from": the gate is stored as g = log alpha.
 *  - "Hybrid models: what Gated DeltaNet replaces in the KV cache" (trefon.com),
 *    section "Gated DeltaNet: add decay": S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T)
 *    + beta_t v_t k_t^T, algebraically the same as the loop above; section "What a
 *    recurrent state changes for serving", item 1: a snapshot of the state at
 *    position N is what prefix reuse needs.
 *
 * Inputs are given in their storage type (fp64, fp32 or bf16 bit patterns) and
 * widened exactly to fp64 element by element.  Outputs are fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "gdn_oracle.h"

/* ---- exact widening of one stored element to fp64 ---------------------------- */
static double ora_widen(const void* p, int dtype, int64_t i) {
  if (dtype == ORA_F64) return ((const double*)p)[i];
  if (dtype == ORA_F32) return (double)((const float*)p)[i];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---- one (batch, head) stream of the token loop ------------------------------- */
typedef struct {
  int64_t T, Dk, Dv;
  int kda;
  int in_dtype, s0_dtype;
  const void *q, *k, *v, *beta, *log_alpha, *s0; /* s0 may be NULL (zeros) */
  double *o, *s_final, *s_ckpt;                   /* s_final, s_ckpt may be NULL */
  int64_t ckpt_every;
} ora_fwd_job;

static int ora_stream(const ora_fwd_job* J, int64_t bh) {
  const int64_t T = J->T, Dk = J->Dk, Dv = J->Dv;
  double* S = (double*)malloc(sizeof(double) * (size_t)(Dv * Dk));
  double* kt = (double*)malloc(sizeof(double) * (size_t)Dk);
  double* qt = (double*)malloc(sizeof(double) * (size_t)Dk);
  double* at = (double*)malloc(sizeof(double) * (size_t)Dk);
  if (!S || !kt || !qt || !at) {
    free(S); free(kt); free(qt); free(at);
    return -1;
  }
  for (int64_t i = 0; i < Dv * Dk; ++i)
    S[i] = J->s0 ? ora_widen(J->s0, J->s0_dtype, bh * Dv * Dk + i) : 0.0;

  const int64_t nck = J->ckpt_every > 0 ? T / J->ckpt_every : 0;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t tok = bh * T + t;
    for (int64_t j = 0; j < Dk; ++j) {
      kt[j] = ora_widen(J->k, J->in_dtype, tok * Dk + j);
      qt[j] = ora_widen(J->q, J->in_dtype, tok * Dk + j);
    }
    const double beta = ora_widen(J->beta, J->in_dtype, tok);

    /* 1. forget: GDN scales the whole state, KDA scales key channel j by alpha_j */
    if (J->kda) {
      for (int64_t j = 0; j < Dk; ++j) at[j] = exp(ora_widen(J->log_alpha, J->in_dtype, tok * Dk + j));
      for (int64_t i = 0; i < Dv; ++i)
        for (int64_t j = 0; j < Dk; ++j) S[i * Dk + j] *= at[j];
    } else {
      const double a = exp(ora_widen(J->log_alpha, J->in_dtype, tok));
      for (int64_t i = 0; i < Dv * Dk; ++i) S[i] *= a;
    }

    /* 2. correct: each value row i moves by beta * (v_i - (S k)_i) along k */
    for (int64_t i = 0; i < Dv; ++i) {
      double r = 0.0;
      for (int64_t j = 0; j < Dk; ++j) r += S[i * Dk + j] * kt[j];
      const double err = ora_widen(J->v, J->in_dtype, tok * Dv + i) - r;
      const double w = beta * err;
      for (int64_t j = 0; j < Dk; ++j) S[i * Dk + j] += w * kt[j];
    }

    /* 3. read: o_t = S_t q_t with the updated state */
    for (int64_t i = 0; i < Dv; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < Dk; ++j) acc += S[i * Dk + j] * qt[j];
      J->o[tok * Dv + i] = acc;
    }

    /* snapshot n (1-based) holds the state after token n * ckpt_every */
    if (J->s_ckpt && J->ckpt_every > 0 && (t + 1) % J->ckpt_every == 0) {
      const int64_t n = (t + 1) / J->ckpt_every - 1;
      memcpy(J->s_ckpt + (bh * nck + n) * Dv * Dk, S, sizeof(double) * (size_t)(Dv * Dk));
    }
  }
  if (J->s_final) memcpy(J->s_final + bh * Dv * Dk, S, sizeof(double) * (size_t)(Dv * Dk));
  free(S); free(kt); free(qt); free(at);
  return 0;
}

/* ---- one decode step on one (sequence, head) state, in place ------------------- */
typedef struct {
  int64_t Dk, Dv;
  int kda, in_dtype;
  double* state;
  const void *q, *k, *v, *beta, *log_alpha;
  double* o;
} ora_dec_job;

static int ora_decode_one(const ora_dec_job* J, int64_t nh) {
  const int64_t Dk = J->Dk, Dv = J->Dv;
  double* S = J->state + nh * Dv * Dk;
  const double beta = ora_widen(J->beta, J->in_dtype, nh);
  if (J->kda) {
    for (int64_t j = 0; j < Dk; ++j) {
      const double a = exp(ora_widen(J->log_alpha, J->in_dtype, nh * Dk + j));
      for (int64_t i = 0; i < Dv; ++i) S[i * Dk + j] *= a;
    }
  } else {
    const double a = exp(ora_widen(J->log_alpha, J->in_dtype, nh));
    for (int64_t i = 0; i < Dv * Dk; ++i) S[i] *= a;
  }
  for (int64_t i = 0; i < Dv; ++i) {
    double r = 0.0;
    for (int64_t j = 0; j < Dk; ++j) r += S[i * Dk + j] * ora_widen(J->k, J->in_dtype, nh * Dk + j);
    const double w = beta * (ora_widen(J->v, J->in_dtype, nh * Dv + i) - r);
    for (int64_t j = 0; j < Dk; ++j) S[i * Dk + j] += w * ora_widen(J->k, J->in_dtype, nh * Dk + j);
  }
  for (int64_t i = 0; i < Dv; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < Dk; ++j) acc += S[i * Dk + j] * ora_widen(J->q, J->in_dtype, nh * Dk + j);
    J->o[nh * Dv + i] = acc;
  }
  return 0;
}

/* ---- a plain thread pool over independent units (streams or states) ------------ */
typedef struct {
  int64_t n_units;
  int64_t next; /* guarded by mu */
  int failed;
  pthread_mutex_t mu;
  int (*fn)(const void*, int64_t);
  const void* job;
} ora_pool;

static void* ora_worker(void* arg) {
  ora_pool* P = (ora_pool*)arg;
  for (;;) {
    pthread_mutex_lock(&P->mu);
    const int64_t u = P->next++;
    pthread_mutex_unlock(&P->mu);
    if (u >= P->n_units) break;
    if (P->fn(P->job, u) != 0) {
      pthread_mutex_lock(&P->mu);
      P->failed = 1;
      pthread_mutex_unlock(&P->mu);
    }
  }
  return NULL;
}

static int ora_fwd_thunk(const void* j, int64_t u) { return ora_stream((const ora_fwd_job*)j, u); }
static int ora_dec_thunk(const void* j, int64_t u) { return ora_decode_one((const ora_dec_job*)j, u); }

static int ora_run(int64_t n_units, int nthreads, int (*fn)(const void*, int64_t), const void* job) {
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if ((int64_t)nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
  ora_pool P;
  P.n_units = n_units;
  P.next = 0;
  P.failed = 0;
  P.fn = fn;
  P.job = job;
  pthread_mutex_init(&P.mu, NULL);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -1;
  int started = 0;
  for (int i = 0; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, ora_worker, &P) == 0) ++started;
  if (started == 0) ora_worker(&P); /* no threads available: run inline */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&P.mu);
  return P.failed ? -1 : started;
}

/* ---- exported entry points ---------------------------------------------------- */
int ora_forward(int64_t B, int64_t H, int64_t T, int64_t Dk, int64_t Dv, int kda, int in_dtype,
                const void* q, const void* k, const void* v, const void* beta, const void* log_alpha,
                const void* s0, int s0_dtype, double* o, double* s_final, double* s_ckpt,
                int64_t ckpt_every, int nthreads) {
  if (B <= 0 || H <= 0 || T < 0 || Dk <= 0 || Dv <= 0 || !q || !k || !v || !beta || !log_alpha || !o)
    return -1;
  if (ckpt_every < 0 || (s_ckpt && ckpt_every == 0)) return -1;
  ora_fwd_job J;
  J.T = T; J.Dk = Dk; J.Dv = Dv; J.kda = kda; J.in_dtype = in_dtype; J.s0_dtype = s0_dtype;
  J.q = q; J.k = k; J.v = v; J.beta = beta; J.log_alpha = log_alpha; J.s0 = s0;
  J.o = o; J.s_final = s_final; J.s_ckpt = s_ckpt; J.ckpt_every = ckpt_every;
  return ora_run(B * H, nthreads, ora_fwd_thunk, &J);
}

int ora_decode_step(int64_t N, int64_t H, int64_t Dk, int64_t Dv, int kda, int in_dtype, double* state,
                    const void* q, const void* k, const void* v, const void* beta, const void* log_alpha,
                    double* o, int nthreads) {
  if (N <= 0 || H <= 0 || Dk <= 0 || Dv <= 0 || !state || !q || !k || !v || !beta || !log_alpha || !o)
    return -1;
  ora_dec_job J;
  J.Dk = Dk; J.Dv = Dv; J.kda = kda; J.in_dtype = in_dtype; J.state = state;
  J.q = q; J.k = k; J.v = v; J.beta = beta; J.log_alpha = log_alpha; J.o = o;
  return ora_run(N * H, nthreads, ora_dec_thunk, &J);
}

int ora_hardware_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}
