/*
 * oracle_check.c -- drives the fp64 oracle (oracle/gdn_oracle.c) through every input type,
 * both variants, snapshots, several thread counts and the decode step, so that the oracle
 * can be run under AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.  Each case
 * also checks a property the recurrence fixes exactly:
 *  - a unit key e_j with beta = 1 overwrites: after the step S k = v (the delta rule writes
 *    the correction, so the old association is replaced);
 *  - beta = 0 only forgets: S_T = (prod alpha) S_0 for the scalar gate;
 *  - per-channel gates that are all equal give the scalar-gate result;
 *  - T decode steps equal one forward pass, and the last snapshot equals the final state.
 * Exit status 0 when every check holds; the sanitizers abort on any memory or UB error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/gdn_oracle.h"

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static uint16_t to_bf16(double x) { /* truncation is enough: any bf16 pattern is a valid input */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int fails = 0;
#define CHECK(cond, ...) do { if (!(cond)) { fprintf(stderr, "FAIL: " __VA_ARGS__); fprintf(stderr, "\n"); ++fails; } } while (0)

static double maxdiff(const double* a, const double* b, size_t n) {
  double m = 0.0;
  for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

/* random inputs of one dtype; log_alpha in [-0.3, 0) */
typedef struct { void *q, *k, *v, *beta, *la; } Inputs;
static void* fill(size_t n, int dt, double lo, double hi) {
  size_t es = dt == ORA_F64 ? 8 : dt == ORA_F32 ? 4 : 2;
  void* p = malloc(n * es);
  for (size_t i = 0; i < n; ++i) {
    const double x = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    if (dt == ORA_F64) ((double*)p)[i] = x;
    else if (dt == ORA_F32) ((float*)p)[i] = (float)x;
    else ((uint16_t*)p)[i] = to_bf16(x);
  }
  return p;
}

static void forward_cases(int dt) {
  const int64_t B = 2, H = 3, T = 37, D = 8, every = 12;
  const int64_t nk = T / every;
  for (int kda = 0; kda < 2; ++kda) {
    Inputs in;
    in.q = fill(B * H * T * D, dt, -1, 1);
    in.k = fill(B * H * T * D, dt, -1, 1);
    in.v = fill(B * H * T * D, dt, -1, 1);
    in.beta = fill(B * H * T, dt, 0, 1);
    in.la = fill(B * H * T * (kda ? D : 1), dt, -0.3, 0);
    double* s0 = (double*)fill(B * H * D * D, ORA_F64, -0.1, 0.1);
    double *o = malloc(sizeof(double) * B * H * T * D), *sf = malloc(sizeof(double) * B * H * D * D);
    double* sc = malloc(sizeof(double) * B * H * nk * D * D);
    double *o1 = malloc(sizeof(double) * B * H * T * D), *sf1 = malloc(sizeof(double) * B * H * D * D);
    int n = ora_forward(B, H, T, D, D, kda, dt, in.q, in.k, in.v, in.beta, in.la, s0, ORA_F64, o, sf, sc, every, 3);
    CHECK(n > 0, "forward dt=%d kda=%d returned %d", dt, kda, n);
    n = ora_forward(B, H, T, D, D, kda, dt, in.q, in.k, in.v, in.beta, in.la, s0, ORA_F64, o1, sf1, NULL, 0, 1);
    CHECK(n == 1, "single-thread forward returned %d", n);
    CHECK(maxdiff(o, o1, B * H * T * D) == 0.0 && maxdiff(sf, sf1, B * H * D * D) == 0.0,
          "thread count changed the result (dt=%d kda=%d)", dt, kda);
    /* snapshot positions: rerun the first 2*every tokens and compare with snapshot 1 */
    {
      const int64_t T2 = 2 * every;
      size_t es = dt == ORA_F64 ? 8 : dt == ORA_F32 ? 4 : 2;
      const int64_t la_w = kda ? D : 1;
      char *q2 = malloc(B * H * T2 * D * es), *k2 = malloc(B * H * T2 * D * es), *v2 = malloc(B * H * T2 * D * es);
      char *b2 = malloc(B * H * T2 * es), *l2 = malloc(B * H * T2 * la_w * es);
      for (int64_t bh = 0; bh < B * H; ++bh) {
        memcpy(q2 + bh * T2 * D * es, (char*)in.q + bh * T * D * es, T2 * D * es);
        memcpy(k2 + bh * T2 * D * es, (char*)in.k + bh * T * D * es, T2 * D * es);
        memcpy(v2 + bh * T2 * D * es, (char*)in.v + bh * T * D * es, T2 * D * es);
        memcpy(b2 + bh * T2 * es, (char*)in.beta + bh * T * es, T2 * es);
        memcpy(l2 + bh * T2 * la_w * es, (char*)in.la + bh * T * la_w * es, T2 * la_w * es);
      }
      double* o2 = malloc(sizeof(double) * B * H * T2 * D);
      double* sf2 = malloc(sizeof(double) * B * H * D * D);
      ora_forward(B, H, T2, D, D, kda, dt, q2, k2, v2, b2, l2, s0, ORA_F64, o2, sf2, NULL, 0, 2);
      for (int64_t bh = 0; bh < B * H; ++bh)
        CHECK(maxdiff(sf2 + bh * D * D, sc + (bh * nk + 1) * D * D, D * D) == 0.0, "snapshot 1 of stream %ld",
              (long)bh);
      free(q2); free(k2); free(v2); free(b2); free(l2); free(o2); free(sf2);
    }
    /* decode steps == forward (zero initial state) */
    {
      double* st = calloc(B * H * D * D, sizeof(double));
      double* od = malloc(sizeof(double) * B * H * D);
      size_t es = dt == ORA_F64 ? 8 : dt == ORA_F32 ? 4 : 2;
      const int64_t la_w = kda ? D : 1;
      char *qt = malloc(B * H * D * es), *kt = malloc(B * H * D * es), *vt = malloc(B * H * D * es);
      char *bt = malloc(B * H * es), *lt = malloc(B * H * la_w * es);
      ora_forward(B, H, T, D, D, kda, dt, in.q, in.k, in.v, in.beta, in.la, NULL, ORA_F64, o1, sf1, NULL, 0, 2);
      double err = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        for (int64_t bh = 0; bh < B * H; ++bh) {
          memcpy(qt + bh * D * es, (char*)in.q + (bh * T + t) * D * es, D * es);
          memcpy(kt + bh * D * es, (char*)in.k + (bh * T + t) * D * es, D * es);
          memcpy(vt + bh * D * es, (char*)in.v + (bh * T + t) * D * es, D * es);
          memcpy(bt + bh * es, (char*)in.beta + (bh * T + t) * es, es);
          memcpy(lt + bh * la_w * es, (char*)in.la + (bh * T + t) * la_w * es, la_w * es);
        }
        CHECK(ora_decode_step(B, H, D, D, kda, dt, st, qt, kt, vt, bt, lt, od, 2) > 0, "decode step");
        for (int64_t bh = 0; bh < B * H; ++bh)
          for (int64_t i = 0; i < D; ++i) err = fmax(err, fabs(od[bh * D + i] - o1[(bh * T + t) * D + i]));
      }
      CHECK(err == 0.0 && maxdiff(st, sf1, B * H * D * D) == 0.0, "decode steps != forward (dt=%d kda=%d)", dt, kda);
      free(st); free(od); free(qt); free(kt); free(vt); free(bt); free(lt);
    }
    free(in.q); free(in.k); free(in.v); free(in.beta); free(in.la);
    free(s0); free(o); free(sf); free(sc); free(o1); free(sf1);
  }
}

static void exact_cases(void) {
  enum { T = 5, D = 4 };
  /* overwrite: unit key e_2, beta = 1, any gate -> S k = v after the step */
  double q[T * D], k[T * D], v[T * D], beta[T], la[T], o[T * D], sf[D * D], s0[D * D];
  for (int i = 0; i < T * D; ++i) { q[i] = urand(); v[i] = urand(); k[i] = urand(); }
  for (int i = 0; i < D * D; ++i) s0[i] = urand();
  for (int t = 0; t < T; ++t) { beta[t] = 0.5 * (urand() + 1.0); la[t] = -0.2 * (urand() + 1.0); }
  for (int j = 0; j < D; ++j) k[(T - 1) * D + j] = (j == 2);
  beta[T - 1] = 1.0;
  ora_forward(1, 1, T, D, D, 0, ORA_F64, q, k, v, beta, la, s0, ORA_F64, o, sf, NULL, 0, 1);
  for (int i = 0; i < D; ++i) CHECK(fabs(sf[i * D + 2] - v[(T - 1) * D + i]) < 1e-15, "overwrite row %d", i);
  /* forget only: beta = 0 -> S_T = exp(sum log alpha) S_0 */
  for (int t = 0; t < T; ++t) beta[t] = 0.0;
  ora_forward(1, 1, T, D, D, 0, ORA_F64, q, k, v, beta, la, s0, ORA_F64, o, sf, NULL, 0, 1);
  double g = 0.0;
  for (int t = 0; t < T; ++t) g += la[t];
  for (int i = 0; i < D * D; ++i) CHECK(fabs(sf[i] - exp(g) * s0[i]) < 1e-14, "forget-only element %d", i);
  /* equal per-channel gates == scalar gate */
  double lak[T * D], sf2[D * D], o2[T * D];
  for (int t = 0; t < T; ++t) { beta[t] = 0.5 * (urand() + 1.0); for (int j = 0; j < D; ++j) lak[t * D + j] = la[t]; }
  ora_forward(1, 1, T, D, D, 0, ORA_F64, q, k, v, beta, la, s0, ORA_F64, o, sf, NULL, 0, 1);
  ora_forward(1, 1, T, D, D, 1, ORA_F64, q, k, v, beta, lak, s0, ORA_F64, o2, sf2, NULL, 0, 1);
  CHECK(maxdiff(o, o2, T * D) < 1e-15 && maxdiff(sf, sf2, D * D) < 1e-15, "equal KDA gates != GDN");
  /* bad arguments are refused */
  CHECK(ora_forward(0, 1, T, D, D, 0, ORA_F64, q, k, v, beta, la, NULL, ORA_F64, o, sf, NULL, 0, 1) == -1, "B=0");
  CHECK(ora_forward(1, 1, T, D, D, 0, ORA_F64, q, k, v, beta, la, NULL, ORA_F64, o, sf, sf, 0, 1) == -1,
        "snapshots without a period");
}

int main(void) {
  exact_cases();
  forward_cases(ORA_F64);
  forward_cases(ORA_F32);
  forward_cases(ORA_BF16);
  if (fails) {
    fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  printf("oracle_check: all checks passed\n");
  return 0;
}
