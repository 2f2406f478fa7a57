/* Host driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of
 * the fp64 oracle (oracle/attn_oracle.c, linked in).  Test infrastructure.
 * Runs every exported oracle function on small seeded shapes, including
 * ragged lengths, agent ranges first/middle/last, window 0/1/W and a wrapped
 * decode ring, then checks the closed forms that need no other code:
 * q = 0 gives LSE = ln |visible keys| and O = the mean of the visible values;
 * window 1 gives O = v of the same frame.  Exit status 0 = all good. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_space_fwd(int, int, int, int, int, int, int, int, double, const double*, const double*,
                     const double*, double*, double*);
int oracle_space_bwd(int, int, int, int, int, int, int, int, double, const double*, const double*,
                     const double*, const double*, double*, double*, double*);
int oracle_time_fwd(int, int, int, int, int, int, int, double, const double*, const double*,
                    const double*, double*, double*);
int oracle_time_bwd(int, int, int, int, int, int, int, double, const double*, const double*,
                    const double*, const double*, double*, double*, double*);
int oracle_time_decode_fwd(int, int, int, int, int, int, int, double, int, int, const double*,
                           const double*, const double*, double*, double*);
int oracle_rmsnorm_qkv_fwd(long, int, int, int, int, double, const double*, const double*,
                           const double*, double*, double*, double*, double*);
int oracle_out_proj_fwd(long, int, int, const double*, const double*, const double*, double*);

static unsigned long long rng = 88172645463325252ULL;
static double urand(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double* arr(long n, int random) {
  double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) a[i] = random ? urand() : 0.0;
  return a;
}
static int fails = 0;
static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++fails;
  }
}

static void space_case(int B, int T, int N, int Hq, int Hkv, int D, int ab, int ac) {
  const long nq = (long)B * T * N * Hq * D, nk = (long)B * T * N * Hkv * D, nl = (long)B * T * N * Hq;
  double *q = arr(nq, 1), *k = arr(nk, 1), *v = arr(nk, 1), *o = arr(nq, 0), *l = arr(nl, 0);
  double *d = arr(nq, 1), *dq = arr(nq, 0), *dk = arr(nk, 0), *dv = arr(nk, 0);
  expect(oracle_space_fwd(B, T, N, Hq, Hkv, D, ab, ac, 0.0, q, k, v, o, l) == 0, "space fwd");
  expect(oracle_space_bwd(B, T, N, Hq, Hkv, D, ab, ac, 0.0, q, k, v, d, dq, dk, dv) == 0, "space bwd");
  /* q = 0: LSE = ln |vis|, O = mean of visible values */
  memset(q, 0, sizeof(double) * (size_t)nq);
  expect(oracle_space_fwd(B, T, N, Hq, Hkv, D, ab, ac, 0.0, q, k, v, o, l) == 0, "space fwd q=0");
  const int G = Hq / Hkv;
  for (int i = 0; i < N; ++i) {
    const int agent = i >= ab && i < ab + ac;
    const int nvis = agent ? N : N - ac;
    for (int h = 0; h < Hq; ++h) {
      const long r = ((long)(B - 1) * T + (T - 1)) * N + i;
      expect(fabs(l[r * Hq + h] - log((double)nvis)) < 1e-12, "space q=0 lse");
      double mean = 0.0;
      for (int j = 0; j < N; ++j)
        if (agent || !(j >= ab && j < ab + ac))
          mean += v[((((long)(B - 1) * T + (T - 1)) * N + j) * Hkv + h / G) * D + 1];
      mean /= nvis;
      expect(fabs(o[(r * Hq + h) * D + 1] - mean) < 1e-12, "space q=0 mean");
    }
  }
  free(q); free(k); free(v); free(o); free(l); free(d); free(dq); free(dk); free(dv);
}

static void time_case(int B, int T, int N, int Hq, int Hkv, int D, int W) {
  const long nq = (long)B * T * N * Hq * D, nk = (long)B * T * N * Hkv * D, nl = (long)B * T * N * Hq;
  double *q = arr(nq, 1), *k = arr(nk, 1), *v = arr(nk, 1), *o = arr(nq, 0), *l = arr(nl, 0);
  double *d = arr(nq, 1), *dq = arr(nq, 0), *dk = arr(nk, 0), *dv = arr(nk, 0);
  expect(oracle_time_fwd(B, T, N, Hq, Hkv, D, W, 0.0, q, k, v, o, l) == 0, "time fwd");
  expect(oracle_time_bwd(B, T, N, Hq, Hkv, D, W, 0.0, q, k, v, d, dq, dk, dv) == 0, "time bwd");
  if (W == 1) { /* O = v of the same frame and KV head */
    const int G = Hq / Hkv;
    for (long r = 0; r < (long)B * T * N; ++r)
      for (int h = 0; h < Hq; ++h)
        expect(fabs(o[(r * Hq + h) * D] - v[(r * Hkv + h / G) * D]) < 1e-12, "time window 1");
  }
  memset(q, 0, sizeof(double) * (size_t)nq);
  expect(oracle_time_fwd(B, T, N, Hq, Hkv, D, W, 0.0, q, k, v, o, l) == 0, "time fwd q=0");
  for (int t = 0; t < T; ++t) {
    const int nvis = W > 0 && t + 1 > W ? W : t + 1;
    expect(fabs(l[((long)t * N) * Hq] - log((double)nvis)) < 1e-12, "time q=0 lse");
  }
  /* decode of the last frame from a wrapped ring of C frames */
  const int C = T > 3 ? T - 1 : T, a = T - 1, first = (W > 0 && a - W + 1 > 0) ? a - W + 1 : 0;
  if (a - first + 1 <= C) {
    double *kc = arr((long)B * C * N * Hkv * D, 1), *vc = arr((long)B * C * N * Hkv * D, 1);
    double *qd = arr((long)B * N * Hq * D, 1), *od = arr((long)B * N * Hq * D, 0), *ld = arr((long)B * N * Hq, 0);
    expect(oracle_time_decode_fwd(B, 1, N, Hq, Hkv, D, W, 0.0, C, a, qd, kc, vc, od, ld) == 0, "decode");
    free(kc); free(vc); free(qd); free(od); free(ld);
  }
  free(q); free(k); free(v); free(o); free(l); free(d); free(dq); free(dk); free(dv);
}

int main(void) {
  space_case(1, 2, 16, 4, 2, 32, 15, 1);
  space_case(2, 1, 17, 6, 3, 64, 0, 1);
  space_case(1, 1, 33, 4, 4, 16, 10, 3);
  space_case(1, 1, 5, 2, 1, 8, 0, 0);
  time_case(1, 8, 3, 4, 2, 32, 4);
  time_case(1, 37, 2, 6, 2, 16, 0);
  time_case(2, 9, 2, 2, 1, 8, 1);
  time_case(1, 1, 4, 4, 1, 8, 192);
  /* projections */
  {
    const long M = 7;
    const int dm = 24, Hq = 4, Hkv = 2, D = 4, nout = (Hq + 2 * Hkv) * D;
    double *x = arr(M * dm, 1), *g = arr(dm, 1), *w = arr((long)nout * dm, 1);
    double *q = arr(M * Hq * D, 0), *k = arr(M * Hkv * D, 0), *v = arr(M * Hkv * D, 0), *r = arr(M, 0);
    expect(oracle_rmsnorm_qkv_fwd(M, dm, Hq, Hkv, D, 1e-6, x, g, w, q, k, v, r) == 0, "rmsnorm qkv");
    double *wo = arr((long)dm * Hq * D, 1), *res = arr(M * dm, 1), *y = arr(M * dm, 0);
    expect(oracle_out_proj_fwd(M, dm, Hq * D, q, wo, res, y) == 0, "out proj");
    expect(oracle_out_proj_fwd(M, dm, Hq * D, q, wo, NULL, y) == 0, "out proj no residual");
    free(x); free(g); free(w); free(q); free(k); free(v); free(r); free(wo); free(res); free(y);
  }
  /* invalid arguments are refused, not read */
  expect(oracle_space_fwd(1, 1, 4, 2, 1, 8, 3, 2, 0.0, 0, 0, 0, 0, 0) == -1, "agent range");
  expect(oracle_time_fwd(1, 1, 4, 2, 1, 8, -1, 0.0, 0, 0, 0, 0, 0) == -1, "window < 0");
  expect(oracle_time_decode_fwd(1, 1, 4, 2, 1, 8, 4, 0.0, 3, 10, 0, 0, 0, 0, 0) == -1, "ring too small");
  if (fails) return 1;
  printf("oracle sanitizer driver: ok\n");
  return 0;
}
