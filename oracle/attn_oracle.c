/*
 * CPU fp64 oracle for block-causal attention.  TEST INFRASTRUCTURE ONLY:
 * it is called by tests/, by the smoke check and by the bench's CPU-baseline
 * leg, never by the product path.  It shares no code, header or constant with
 * the HIP library.
 *
 * What it computes is plain masked softmax attention, written out from its
 * definition, one (unit, head) problem at a time, in double precision with a
 * two-pass softmax (exact maximum first, then the sum).
 *
 * Sources (Open Dreamer articles, pro.edgex.exchange fr-FR edition):
 *  - section "Architecture": the backbone alternates space layers (attention
 *    among the tokens of one timestep block) with causal time layers
 *    (attention across frames); world-model tokens cannot read the agent
 *    token.
 *  - section "Configuration d'entraînement": grouped-query attention, 30
 *    query heads over 3 KV heads; time attention uses a 192-step sliding
 *    window.
 * Readings of the points the pages leave open (stated once, used here):
 *  - softmax scale 1/sqrt(D) unless the caller passes one;
 *  - query head h reads KV head h / (Hq/Hkv) (contiguous groups);
 *  - time attention is per token slot: frame t sees frame t' of the same slot
 *    iff t' <= t and (W == 0 or t - t' <= W - 1), so the window counts the
 *    current frame;
 *  - space attention: a query that is not an agent token cannot see agent
 *    keys; an agent query sees every key of its block.
 *
 * Layout: q, o, dout, dq are (B,T,N,Hq,D); k, v, dk, dv are (B,T,N,Hkv,D);
 * lse is (B,T,N,Hq); all row-major, contiguous, double.
 *
 * Return: 0 on success, -1 on bad arguments, -2 if some query would see no
 * key (impossible for valid descriptors; checked anyway).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One attention problem: a unit (a block for space, a slot for time) and a
 * query head.  Positions p = 0..L-1 index tokens (space) or frames (time). */
typedef struct {
  long qpos_stride;   /* elements between consecutive positions, query side */
  long kpos_stride;   /* same, key/value side */
  int L;
  int is_time;
  int window;         /* time only */
  int agent_begin, agent_count; /* space only */
} problem;

static int is_agent(const problem* P, int p) {
  return p >= P->agent_begin && p < P->agent_begin + P->agent_count;
}

/* visibility of key position b to query position a */
static int visible(const problem* P, int a, int b) {
  if (P->is_time) {
    if (b > a) return 0;
    if (P->window > 0 && a - b > P->window - 1) return 0;
    return 1;
  }
  if (is_agent(P, b) && !is_agent(P, a)) return 0;
  return 1;
}

static double dot(const double* x, const double* y, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += x[d] * y[d];
  return s;
}

/* Softmax row of query position a: z[b] = scale*<q_a,k_b> and p[b] (0 where
 * invisible), max first, then the sum.  Returns the log-sum-exp, or NAN if no
 * key is visible. */
static double row_probs(const problem* P, int a, const double* qa, const double* kbase,
                        int D, double scale, double* z, double* p) {
  double m = -INFINITY;
  int any = 0;
  for (int b = 0; b < P->L; ++b) {
    if (visible(P, a, b)) {
      z[b] = scale * dot(qa, kbase + (long)b * P->kpos_stride, D);
      if (z[b] > m) m = z[b];
      any = 1;
    }
  }
  if (!any) return NAN;
  double l = 0.0;
  for (int b = 0; b < P->L; ++b) {
    p[b] = visible(P, a, b) ? exp(z[b] - m) : 0.0;
    l += p[b];
  }
  for (int b = 0; b < P->L; ++b) p[b] /= l;
  return m + log(l);
}

static int check_shape(int B, int T, int N, int Hq, int Hkv, int D) {
  if (B <= 0 || T <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return -1;
  if (Hq % Hkv != 0) return -1;
  return 0;
}

/* Builds the problem for (op, unit) and the element offsets of position 0 of
 * query head h / KV head g.  Space unit u = b*T + t; time unit u = b*N + n. */
static problem make_problem(int is_time, int B, int T, int N, int Hq, int Hkv, int D,
                            int window, int agent_begin, int agent_count, int u,
                            long* q0, long* kv0, long* lse0, long* lse_stride) {
  problem P;
  (void)B;
  P.is_time = is_time;
  P.window = window;
  P.agent_begin = agent_begin;
  P.agent_count = agent_count;
  if (!is_time) {
    P.L = N;
    P.qpos_stride = (long)Hq * D;
    P.kpos_stride = (long)Hkv * D;
    *q0 = (long)u * N * Hq * D;
    *kv0 = (long)u * N * Hkv * D;
    *lse0 = (long)u * N * Hq;
    *lse_stride = Hq;
  } else {
    int b = u / N, n = u % N;
    P.L = T;
    P.qpos_stride = (long)N * Hq * D;
    P.kpos_stride = (long)N * Hkv * D;
    *q0 = ((long)b * T * N + n) * Hq * D;
    *kv0 = ((long)b * T * N + n) * Hkv * D;
    *lse0 = ((long)b * T * N + n) * Hq;
    *lse_stride = (long)N * Hq;
  }
  return P;
}

static int attn_fwd(int is_time, int B, int T, int N, int Hq, int Hkv, int D,
                    int window, int agent_begin, int agent_count, double scale,
                    const double* q, const double* k, const double* v,
                    double* o, double* lse) {
  if (check_shape(B, T, N, Hq, Hkv, D)) return -1;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  const int G = Hq / Hkv;
  const int units = is_time ? B * N : B * T;
  const int L = is_time ? T : N;
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (long job = 0; job < (long)units * Hq; ++job) {
    int u = (int)(job / Hq), h = (int)(job % Hq), g = h / G;
    long q0, kv0, l0, ls;
    problem P = make_problem(is_time, B, T, N, Hq, Hkv, D, window, agent_begin,
                             agent_count, u, &q0, &kv0, &l0, &ls);
    double* z = (double*)malloc(sizeof(double) * L);
    double* p = (double*)malloc(sizeof(double) * L);
    const double* kb = k + kv0 + (long)g * D;
    const double* vb = v + kv0 + (long)g * D;
    for (int a = 0; a < L; ++a) {
      const double* qa = q + q0 + (long)a * P.qpos_stride + (long)h * D;
      double s = row_probs(&P, a, qa, kb, D, scale, z, p);
      if (isnan(s)) { bad = 1; continue; }
      double* oa = o + q0 + (long)a * P.qpos_stride + (long)h * D;
      for (int d = 0; d < D; ++d) oa[d] = 0.0;
      for (int b = 0; b < L; ++b) {
        if (p[b] == 0.0) continue;
        const double* vbb = vb + (long)b * P.kpos_stride;
        for (int d = 0; d < D; ++d) oa[d] += p[b] * vbb[d];
      }
      lse[l0 + (long)a * ls + h] = s;
    }
    free(z);
    free(p);
  }
  return bad ? -2 : 0;
}

/* Gradients of L = sum(O * dO):
 *   Delta_a = <dO_a, o_a>,  dS_ab = p_ab (<dO_a, v_b> - Delta_a),
 *   dQ_a = scale * sum_b dS_ab k_b,
 *   dK_b = scale * sum over heads of the group and queries a of dS_ab q_a,
 *   dV_b = sum over heads of the group and queries a of p_ab dO_a.
 * Parallel over (unit, KV group) so that dK/dV sums stay in one thread. */
static int attn_bwd(int is_time, int B, int T, int N, int Hq, int Hkv, int D,
                    int window, int agent_begin, int agent_count, double scale,
                    const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv) {
  if (check_shape(B, T, N, Hq, Hkv, D)) return -1;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  const int G = Hq / Hkv;
  const int units = is_time ? B * N : B * T;
  const int L = is_time ? T : N;
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (long job = 0; job < (long)units * Hkv; ++job) {
    int u = (int)(job / Hkv), g = (int)(job % Hkv);
    long q0, kv0, l0, ls;
    problem P = make_problem(is_time, B, T, N, Hq, Hkv, D, window, agent_begin,
                             agent_count, u, &q0, &kv0, &l0, &ls);
    double* z = (double*)malloc(sizeof(double) * L);
    double* p = (double*)malloc(sizeof(double) * L);
    double* oa = (double*)malloc(sizeof(double) * D);
    const double* kb = k + kv0 + (long)g * D;
    const double* vb = v + kv0 + (long)g * D;
    double* dkb = dk + kv0 + (long)g * D;
    double* dvb = dv + kv0 + (long)g * D;
    for (int b = 0; b < L; ++b)
      for (int d = 0; d < D; ++d) {
        dkb[(long)b * P.kpos_stride + d] = 0.0;
        dvb[(long)b * P.kpos_stride + d] = 0.0;
      }
    for (int h = g * G; h < (g + 1) * G; ++h) {
      for (int a = 0; a < L; ++a) {
        const double* qa = q + q0 + (long)a * P.qpos_stride + (long)h * D;
        const double* da = dout + q0 + (long)a * P.qpos_stride + (long)h * D;
        double* dqa = dq + q0 + (long)a * P.qpos_stride + (long)h * D;
        double s = row_probs(&P, a, qa, kb, D, scale, z, p);
        if (isnan(s)) { bad = 1; continue; }
        for (int d = 0; d < D; ++d) oa[d] = 0.0;
        for (int b = 0; b < L; ++b) {
          if (p[b] == 0.0) continue;
          for (int d = 0; d < D; ++d) oa[d] += p[b] * vb[(long)b * P.kpos_stride + d];
        }
        double delta = dot(da, oa, D);
        for (int d = 0; d < D; ++d) dqa[d] = 0.0;
        for (int b = 0; b < L; ++b) {
          if (!visible(&P, a, b)) continue;
          const double* kbb = kb + (long)b * P.kpos_stride;
          const double* vbb = vb + (long)b * P.kpos_stride;
          double ds = p[b] * (dot(da, vbb, D) - delta);
          for (int d = 0; d < D; ++d) {
            dqa[d] += scale * ds * kbb[d];
            dkb[(long)b * P.kpos_stride + d] += scale * ds * qa[d];
            dvb[(long)b * P.kpos_stride + d] += p[b] * da[d];
          }
        }
      }
    }
    free(z);
    free(p);
    free(oa);
  }
  return bad ? -2 : 0;
}

/* ---- exported entry points (ctypes) ---- */

int oracle_space_fwd(int B, int T, int N, int Hq, int Hkv, int D, int agent_begin,
                     int agent_count, double scale, const double* q, const double* k,
                     const double* v, double* o, double* lse) {
  if (agent_count < 0 || agent_begin < 0 || agent_begin + agent_count > N) return -1;
  return attn_fwd(0, B, T, N, Hq, Hkv, D, 0, agent_begin, agent_count, scale, q, k, v, o, lse);
}

int oracle_space_bwd(int B, int T, int N, int Hq, int Hkv, int D, int agent_begin,
                     int agent_count, double scale, const double* q, const double* k,
                     const double* v, const double* dout, double* dq, double* dk,
                     double* dv) {
  if (agent_count < 0 || agent_begin < 0 || agent_begin + agent_count > N) return -1;
  return attn_bwd(0, B, T, N, Hq, Hkv, D, 0, agent_begin, agent_count, scale, q, k, v,
                  dout, dq, dk, dv);
}

int oracle_time_fwd(int B, int T, int N, int Hq, int Hkv, int D, int window, double scale,
                    const double* q, const double* k, const double* v, double* o,
                    double* lse) {
  if (window < 0) return -1;
  return attn_fwd(1, B, T, N, Hq, Hkv, D, window, 0, 0, scale, q, k, v, o, lse);
}

int oracle_time_bwd(int B, int T, int N, int Hq, int Hkv, int D, int window, double scale,
                    const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv) {
  if (window < 0) return -1;
  return attn_bwd(1, B, T, N, Hq, Hkv, D, window, 0, 0, scale, q, k, v, dout, dq, dk, dv);
}

/* Rollout decode of time attention.  Open Dreamer articles (pro.edgex.exchange,
 * fr-FR edition), section "Artefacts publiés": the pipeline ships rollout
 * generation and a local rollout harness, and the browser demo streams the
 * generated world frame by frame; section "Architecture": time layers are
 * causal across frames.  Reading: generating frame a runs the same time
 * attention as training, restricted to the query rows of the new frames, with
 * the keys and values of earlier frames taken from a cache.
 *
 * The queries are Tq consecutive frames with absolute indices q_frame0 ..
 * q_frame0 + Tq - 1: q, o are (B,Tq,N,Hq,D), lse (B,Tq,N,Hq).  The cache kc,
 * vc is (B,C,N,Hkv,D) and holds absolute frame f at ring position f % C.
 * Query frame a sees frame f iff f <= a and (W == 0 or a - f <= W - 1), the
 * predicate of oracle_time_fwd.  Every frame some query sees must be in the
 * ring: (last query frame) - (first visible frame) + 1 <= C. */
int oracle_time_decode_fwd(int B, int Tq, int N, int Hq, int Hkv, int D, int window,
                           double scale, int C, int q_frame0, const double* q,
                           const double* kc, const double* vc, double* o, double* lse) {
  if (check_shape(B, Tq, N, Hq, Hkv, D) || window < 0 || C <= 0 || q_frame0 < 0) return -1;
  const int last = q_frame0 + Tq - 1;
  const int first = (window > 0 && q_frame0 - window + 1 > 0) ? q_frame0 - window + 1 : 0;
  if (last - first + 1 > C) return -1;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  const int G = Hq / Hkv;
  problem P;
  P.is_time = 1;
  P.window = window;
  P.agent_begin = 0;
  P.agent_count = 0;
  P.L = last + 1;
#pragma omp parallel for schedule(dynamic)
  for (long job = 0; job < (long)B * N * Hq; ++job) {
    const int h = (int)(job % Hq), g = h / G;
    const int n = (int)((job / Hq) % N), b = (int)(job / ((long)Hq * N));
    double* z = (double*)malloc(sizeof(double) * (last + 1));
    for (int t = 0; t < Tq; ++t) {
      const int a = q_frame0 + t;
      const long qo = (((long)b * Tq + t) * N + n) * Hq * D + (long)h * D;
      double m = -INFINITY;
      for (int f = 0; f <= last; ++f) {
        if (!visible(&P, a, f)) continue;
        const long ko = (((long)b * C + f % C) * N + n) * Hkv * D + (long)g * D;
        z[f] = scale * dot(q + qo, kc + ko, D);
        if (z[f] > m) m = z[f];
      }
      double l = 0.0;
      for (int d = 0; d < D; ++d) o[qo + d] = 0.0;
      for (int f = 0; f <= last; ++f) {
        if (!visible(&P, a, f)) continue;
        const long vo = (((long)b * C + f % C) * N + n) * Hkv * D + (long)g * D;
        const double e = exp(z[f] - m);
        l += e;
        for (int d = 0; d < D; ++d) o[qo + d] += e * vc[vo + d];
      }
      for (int d = 0; d < D; ++d) o[qo + d] /= l;
      lse[(((long)b * Tq + t) * N + n) * Hq + h] = m + log(l);
    }
    free(z);
  }
  return 0;
}

/* ---- projections beside attention ----
 * Open Dreamer articles (pro.edgex.exchange, fr-FR edition), section
 * "Configuration d'entraînement": d_model 1920, 30 query heads over 3 KV
 * heads of width 64; section "Ingénierie de la stabilité", item 3: parameters
 * are kept in fp32, bf16 covers most matmul activations and the attention
 * inputs, normalization layers stay in fp32.  Readings (the pages name no
 * norm and no layout): the norm before the QKV projection is an RMS norm with
 * a learned fp32 gain, applied to the bf16 token rows; weights are bf16
 * copies stored (out_features, in_features); QKV output columns are the Q
 * heads, then the K heads, then the V heads; no biases.  The pages fix no
 * rounding point inside norm-then-projection, so this is the exact product
 * of the given bf16 and fp32 values. */

/* RMS norm then the QKV projection.  x (M, dm); gamma (dm); w ((Hq+2Hkv)*D, dm);
 * q (M, Hq*D), k and v (M, Hkv*D); rstd (M) = 1/sqrt(mean(x^2) + eps).
 *   y = x * rstd * gamma,  [q | k | v] = y w^T. */
int oracle_rmsnorm_qkv_fwd(long M, int dm, int Hq, int Hkv, int D, double eps,
                           const double* x, const double* gamma, const double* w,
                           double* q, double* k, double* v, double* rstd) {
  if (M <= 0 || dm <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || eps < 0.0) return -1;
  const int nq = Hq * D, nkv = Hkv * D, nout = nq + 2 * nkv;
#pragma omp parallel for schedule(static)
  for (long m = 0; m < M; ++m) {
    const double* xm = x + m * dm;
    double ss = 0.0;
    for (int c = 0; c < dm; ++c) ss += xm[c] * xm[c];
    const double r = 1.0 / sqrt(ss / dm + eps);
    rstd[m] = r;
    double* y = (double*)malloc(sizeof(double) * dm);
    for (int c = 0; c < dm; ++c) y[c] = xm[c] * r * gamma[c];
    for (int n = 0; n < nout; ++n) {
      const double acc = dot(y, w + (long)n * dm, dm);
      if (n < nq) q[m * nq + n] = acc;
      else if (n < nq + nkv) k[m * nkv + (n - nq)] = acc;
      else v[m * nkv + (n - nq - nkv)] = acc;
    }
    free(y);
  }
  return 0;
}

/* Output projection with the residual add: o (M, din); w (dm, din);
 * residual (M, dm) or NULL;  y = residual + o w^T, (M, dm). */
int oracle_out_proj_fwd(long M, int dm, int din, const double* o, const double* w,
                        const double* residual, double* y) {
  if (M <= 0 || dm <= 0 || din <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (long m = 0; m < M; ++m)
    for (int n = 0; n < dm; ++n)
      y[m * dm + n] = (residual ? residual[m * dm + n] : 0.0) + dot(o + m * din, w + (long)n * din, din);
  return 0;
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
