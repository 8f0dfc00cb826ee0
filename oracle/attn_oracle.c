/*
 * attn_oracle.c -- plain CPU oracle for causal grouped-query attention with a
 * per-query document-start mask: the forward row log-sum-exp (and output) and
 * the backward pass (dQ, dK, dV).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * What it computes (the definitions it writes out, in fp64 arithmetic):
 *
 *   Page "llm.istanbul -- 10_backward_attention.wgsl", header comment and
 *   kernel attention_backward (Pass 0 / Pass A / Pass B / Final):
 *     - group map:   q_per_group = H / KV,  kv_h = h / q_per_group
 *     - row layout:  Q, dO, dQ  [S, H, d]   (row base s*H*d + h*d)
 *                    K, V, dK, dV [S, KV, d] (row base j*KV*d + kv_h*d)
 *                    LSE [S, H]             (index s*H + h)
 *     - mask:        key j is visible to query s  iff  seg[s] <= j <= s
 *                    (seg[s] is the start of the query's document; seg == 0
 *                    everywhere is plain causal attention)
 *     - P[s,j]  = exp(scale * q_s . k_j - LSE[s,h])
 *     - dP[s,j] = dO_s . v_j
 *     - D[s]    = sum over visible j of P[s,j] * dP[s,j]
 *     - dS[s,j] = scale * P[s,j] * (dP[s,j] - D[s])
 *     - dQ_s   += sum_j dS[s,j] * k_j
 *     - dK_j   += sum over (s, h in the group of kv_h) of dS[s,j] * q_s
 *     - dV_j   += sum over (s, h in the group of kv_h) of P[s,j] * dO_s
 *   All three outputs accumulate ("+=" contract of the header comment).
 *
 *   Forward (page "tang 0.2.0 -- src/gpu/llm.rs", causal_attention_fused:
 *   row max, exp-sum, weighted V), extended with the same document mask and
 *   with the natural-log LSE = m + ln(sum_j exp(x_j - m)) that the backward
 *   consumes.  A row with no visible key (seg[s] > s) gets LSE = -inf, O = 0.
 *
 * Ordering: phase 1 walks rows (s, h) and produces D and dQ; phase 2 walks
 * keys (j, kv_h) and produces dK and dV (the key-major ordering of the
 * attention_backward_short_dKdV kernel on the same page).  Every output
 * element is written by exactly one thread in a fixed summation order, so
 * results are bitwise identical for any thread count.
 *
 * Precision: inputs are widened to double, all arithmetic is double, and the
 * float entry points round once at the end: out = (float)((double)init + g).
 * No -ffast-math.
 *
 * The _o entry points take the forward output O and read the row term off it
 * (D = dO . O, see bwd_row); the others compute D = sum_j P * dP.
 *
 * The _decode entry points are the single-query backward over a KV history
 * with stored probabilities (page "rullama 0.5.0", pass 1 and pass 2 of 2);
 * see oracle_attn_bwd_decode_f64.
 *
 * Parity status: every function here is pinned by the CPU tests (finite
 * differences, sum_j dS = 0, masked-key zeros, plain-causal equality with an
 * independent dense implementation, packed == per-document, GQA == replicated
 * MHA, closed forms, linearity / "+="; for the _o entry points: agreement with
 * D = sum_j P * dP at the exact forward output, and the closed-form effect of
 * a perturbed O on each gradient; for the _decode entry points: finite
 * differences through the decode forward, equality with the backward above
 * for the last row of a causal problem, the T = 1 closed form, the history
 * sums of dK and dV).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ */
/* problem description shared by the worker threads                    */
/* ------------------------------------------------------------------ */
typedef struct {
  const double *Q, *K, *V, *dO, *LSE;
  const uint32_t *seg; /* NULL means all zeros */
  int S, H, KV, d;
  double scale;
  const double *O; /* forward output [S,H,d]: when given, D = dO . O (see bwd_row) */
} problem_t;

static long first_key(const problem_t *p, long s) { return p->seg ? (long)p->seg[s] : 0; }

static double dot(const double *a, const double *b, int n) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

static const double *q_row(const problem_t *p, const double *base, long s, int h) {
  return base + ((size_t)s * p->H + h) * p->d;
}
static const double *kv_row(const problem_t *p, const double *base, long j, int kvh) {
  return base + ((size_t)j * p->KV + kvh) * p->d;
}
static int kv_head_of(const problem_t *p, int h) { return h / (p->H / p->KV); }

/* P[s,j] of the given head, recomputed from the stored LSE */
static double prob(const problem_t *p, long s, int h, long j) {
  int kvh = kv_head_of(p, h);
  double x = p->scale * dot(q_row(p, p->Q, s, h), kv_row(p, p->K, j, kvh), p->d);
  return exp(x - p->LSE[(size_t)s * p->H + h]);
}
/* dP[s,j] = dO_s . v_j */
static double dprob(const problem_t *p, long s, int h, long j) {
  return dot(q_row(p, p->dO, s, h), kv_row(p, p->V, j, kv_head_of(p, h)), p->d);
}

/* ------------------------------------------------------------------ */
/* tiny static thread pool: item i goes to thread i % T                */
/* ------------------------------------------------------------------ */
typedef struct {
  void (*fn)(void *ctx, long item);
  void *ctx;
  long n_items;
  int tid, nthreads;
} job_t;

static void *run_job(void *arg) {
  job_t *j = (job_t *)arg;
  for (long i = j->tid; i < j->n_items; i += j->nthreads) j->fn(j->ctx, i);
  return NULL;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static void parallel_for(long n_items, int nthreads, void (*fn)(void *, long), void *ctx) {
  nthreads = resolve_threads(nthreads);
  if (nthreads > 256) nthreads = 256;
  if ((long)nthreads > n_items) nthreads = n_items > 0 ? (int)n_items : 1;
  pthread_t th[256];
  job_t jobs[256];
  int spawned[256] = {0};
  for (int t = 0; t < nthreads; ++t) jobs[t] = (job_t){fn, ctx, n_items, t, nthreads};
  for (int t = 1; t < nthreads; ++t)
    spawned[t] = pthread_create(&th[t], NULL, run_job, &jobs[t]) == 0;
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (spawned[t])
      pthread_join(th[t], NULL);
    else
      run_job(&jobs[t]); /* could not spawn: same items, same result */
  }
}

/* ------------------------------------------------------------------ */
/* forward                                                             */
/* ------------------------------------------------------------------ */
typedef struct {
  const problem_t *p;
  double *O, *LSE;
} fwd_ctx_t;

/* One row (s, h): LSE into *lse and, when o != NULL, O into o[0..d). */
static void fwd_one(const problem_t *p, long s, int h, double *o, double *lse_out) {
  int kvh = kv_head_of(p, h);
  int d = p->d;
  if (o) memset(o, 0, sizeof(double) * d);
  long lo = first_key(p, s);
  if (lo > s) { /* no visible key */
    *lse_out = -INFINITY;
    return;
  }
  const double *q = q_row(p, p->Q, s, h);
  double m = -INFINITY;
  for (long j = lo; j <= s; ++j) {
    double x = p->scale * dot(q, kv_row(p, p->K, j, kvh), d);
    if (x > m) m = x;
  }
  double sum = 0.0;
  for (long j = lo; j <= s; ++j) sum += exp(p->scale * dot(q, kv_row(p, p->K, j, kvh), d) - m);
  double lse = m + log(sum);
  *lse_out = lse;
  if (!o) return;
  for (long j = lo; j <= s; ++j) {
    double w = exp(p->scale * dot(q, kv_row(p, p->K, j, kvh), d) - lse);
    const double *v = kv_row(p, p->V, j, kvh);
    for (int i = 0; i < d; ++i) o[i] += w * v[i];
  }
}

static void fwd_row(void *vctx, long item) {
  fwd_ctx_t *c = (fwd_ctx_t *)vctx;
  const problem_t *p = c->p;
  long s = item / p->H;
  int h = (int)(item % p->H);
  size_t r = (size_t)s * p->H + h;
  fwd_one(p, s, h, c->O ? c->O + r * p->d : NULL, &c->LSE[r]);
}

static int check_dims(int S, int H, int KV, int d) {
  if (S < 0 || H < 1 || KV < 1 || d < 1) return 1;
  if (H % KV != 0) return 1;
  return 0;
}

/* O [S,H,d] (may be NULL) and LSE [S,H], fp64 in and out */
int oracle_attn_fwd_f64(const double *Q, const double *K, const double *V, const uint32_t *seg,
                        double *O, double *LSE, int S, int H, int KV, int d, double scale,
                        int nthreads) {
  if (check_dims(S, H, KV, d)) return 1;
  problem_t p = {Q, K, V, NULL, NULL, seg, S, H, KV, d, scale};
  fwd_ctx_t c = {&p, O, LSE};
  parallel_for((long)S * H, nthreads, fwd_row, &c);
  return 0;
}

/* ------------------------------------------------------------------ */
/* backward                                                            */
/* ------------------------------------------------------------------ */
typedef struct {
  const problem_t *p;
  double *D;         /* [S,H]  row term (always produced) */
  double *rowsum_dS; /* [S,H]  sum_j dS (debug hook, may be NULL) */
  double *dQ;        /* [S,H,d] gradient of this call (may be NULL) */
  double *dK, *dV;   /* [S,KV,d] gradients of this call (may be NULL) */
  const unsigned char *row_needed; /* phase-1 filter, NULL = all rows */
  const unsigned char *dq_needed;  /* rows that also get dQ, NULL = all */
  const unsigned char *key_needed; /* phase-2 filter, NULL = all keys */
} bwd_ctx_t;

/* Phase 1 for row (s, h): P and dP over the visible keys, D, and
 * dQ_s = sum_j dS[s,j] k_j. */
static void bwd_row(void *vctx, long item) {
  bwd_ctx_t *c = (bwd_ctx_t *)vctx;
  const problem_t *p = c->p;
  long s = item / p->H;
  int h = (int)(item % p->H);
  if (c->row_needed && !c->row_needed[s]) return;
  int kvh = kv_head_of(p, h);
  int d = p->d;
  size_t r = (size_t)s * p->H + h;
  long lo = first_key(p, s);
  long n = s - lo + 1; /* visible keys; n <= 0 is an empty row */
  double *P = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? 2 * n : 1));
  double *dP = P + (n > 0 ? n : 0);
  double D = 0.0;
  for (long j = lo; j <= s; ++j) {
    P[j - lo] = prob(p, s, h, j);
    dP[j - lo] = dprob(p, s, h, j);
    D += P[j - lo] * dP[j - lo];
  }
  /* With the forward output given, the row term is read off it instead:
   * sum_j P_j (dO . v_j) = dO . (sum_j P_j v_j) = dO . O, where O is the
   * forward's probability-weighted sum of V (page "tang 0.2.0 --
   * src/gpu/llm.rs", causal_attention_fused). */
  if (p->O) D = dot(q_row(p, p->dO, s, h), q_row(p, p->O, s, h), p->d);
  c->D[r] = D;
  int want_dq = c->dQ && (!c->dq_needed || c->dq_needed[s]);
  double *dq = want_dq ? c->dQ + r * d : NULL;
  if (dq) memset(dq, 0, sizeof(double) * d);
  double rs = 0.0;
  for (long j = lo; j <= s && (dq || c->rowsum_dS); ++j) {
    double ds = p->scale * P[j - lo] * (dP[j - lo] - D);
    rs += ds;
    if (dq) {
      const double *k = kv_row(p, p->K, j, kvh);
      for (int i = 0; i < d; ++i) dq[i] += ds * k[i];
    }
  }
  if (c->rowsum_dS) c->rowsum_dS[r] = rs;
  free(P);
}

/* Phase 2 for key (j, kv_h): dK_j and dV_j over every query that sees j,
 * queries ascending, heads of the group ascending. */
static void bwd_key(void *vctx, long item) {
  bwd_ctx_t *c = (bwd_ctx_t *)vctx;
  const problem_t *p = c->p;
  long j = item / p->KV;
  int kvh = (int)(item % p->KV);
  if (c->key_needed && !c->key_needed[j]) return;
  int d = p->d, g = p->H / p->KV;
  double *dk = c->dK + ((size_t)j * p->KV + kvh) * d;
  double *dv = c->dV + ((size_t)j * p->KV + kvh) * d;
  memset(dk, 0, sizeof(double) * d);
  memset(dv, 0, sizeof(double) * d);
  for (long s = j; s < p->S; ++s) {
    if (first_key(p, s) > j) continue; /* key j lies before the query's document */
    for (int h = kvh * g; h < (kvh + 1) * g; ++h) {
      double P = prob(p, s, h, j);
      double ds = p->scale * P * (dprob(p, s, h, j) - c->D[(size_t)s * p->H + h]);
      const double *q = q_row(p, p->Q, s, h);
      const double *go = q_row(p, p->dO, s, h);
      for (int i = 0; i < d; ++i) {
        dk[i] += ds * q[i];
        dv[i] += P * go[i];
      }
    }
  }
}

/* Gradients of this call (no accumulation), fp64 in and out.  O (may be
 * NULL) is the forward output: when given, D = dO . O.  D_out and rowsum_dS
 * are optional debug outputs [S,H]. */
int oracle_attn_bwd_o_f64(const double *Q, const double *K, const double *V, const double *O,
                          const double *dO, const double *LSE, const uint32_t *seg, double *dQ,
                          double *dK, double *dV, double *D_out, double *rowsum_dS, int S, int H,
                          int KV, int d, double scale, int nthreads) {
  if (check_dims(S, H, KV, d)) return 1;
  if (S == 0) return 0;
  problem_t p = {Q, K, V, dO, LSE, seg, S, H, KV, d, scale, O};
  double *D = D_out ? D_out : (double *)malloc(sizeof(double) * (size_t)S * H);
  if (!D) return 2;
  bwd_ctx_t c = {&p, D, rowsum_dS, dQ, dK, dV, NULL, NULL, NULL};
  parallel_for((long)S * H, nthreads, bwd_row, &c);
  if (dK && dV) parallel_for((long)S * KV, nthreads, bwd_key, &c);
  if (!D_out) free(D);
  return 0;
}

int oracle_attn_bwd_f64(const double *Q, const double *K, const double *V, const double *dO,
                        const double *LSE, const uint32_t *seg, double *dQ, double *dK,
                        double *dV, double *D_out, double *rowsum_dS, int S, int H, int KV,
                        int d, double scale, int nthreads) {
  return oracle_attn_bwd_o_f64(Q, K, V, NULL, dO, LSE, seg, dQ, dK, dV, D_out, rowsum_dS, S, H,
                               KV, d, scale, nthreads);
}

/* ------------------------------------------------------------------ */
/* float entry points                                                  */
/* ------------------------------------------------------------------ */
static double *widen(const float *x, size_t n) {
  double *y = (double *)malloc(sizeof(double) * (n ? n : 1));
  if (!y) return NULL;
  for (size_t i = 0; i < n; ++i) y[i] = (double)x[i];
  return y;
}

/* Forward for selected rows only: LSE_sel [n_rows, H] (and O_sel [n_rows, H, d]
 * when not NULL) for query rows rows[0..n_rows), fp32 inputs, fp64 math,
 * fp32-rounded outputs. */
typedef struct {
  const problem_t *p;
  const int32_t *rows;
  float *O_sel, *LSE_sel;
} fwd_rows_ctx_t;

static void fwd_sel_row(void *vctx, long item) {
  fwd_rows_ctx_t *c = (fwd_rows_ctx_t *)vctx;
  const problem_t *p = c->p;
  long i = item / p->H;
  int h = (int)(item % p->H);
  int d = p->d;
  size_t r = (size_t)i * p->H + h;
  double lse;
  double *o = c->O_sel ? (double *)malloc(sizeof(double) * d) : NULL;
  fwd_one(p, c->rows[i], h, o, &lse);
  c->LSE_sel[r] = (float)lse;
  if (o) {
    for (int k = 0; k < d; ++k) c->O_sel[r * d + k] = (float)o[k];
    free(o);
  }
}

int oracle_attn_fwd_rows(const float *Q, const float *K, const float *V, const uint32_t *seg,
                         const int32_t *rows, int n_rows, float *O_sel, float *LSE_sel, int S,
                         int H, int KV, int d, float scale, int nthreads) {
  if (check_dims(S, H, KV, d) || n_rows < 0) return 1;
  for (int i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= S) return 1;
  size_t nq = (size_t)S * H * d, nk = (size_t)S * KV * d;
  double *q = widen(Q, nq), *k = widen(K, nk), *v = widen(V, nk);
  int rc = 2;
  if (q && k && v) {
    problem_t p = {q, k, v, NULL, NULL, seg, S, H, KV, d, (double)scale};
    fwd_rows_ctx_t c = {&p, rows, O_sel, LSE_sel};
    parallel_for((long)n_rows * H, nthreads, fwd_sel_row, &c);
    rc = 0;
  }
  free(q); free(k); free(v);
  return rc;
}

/* fp32 inputs; O (may be NULL) and LSE are overwritten with fp32-rounded
 * fp64 results. */
int oracle_attn_fwd(const float *Q, const float *K, const float *V, const uint32_t *seg, float *O,
                    float *LSE, int S, int H, int KV, int d, float scale, int nthreads) {
  if (check_dims(S, H, KV, d)) return 1;
  size_t nq = (size_t)S * H * d, nk = (size_t)S * KV * d, nr = (size_t)S * H;
  double *q = widen(Q, nq), *k = widen(K, nk), *v = widen(V, nk);
  double *o = O ? (double *)malloc(sizeof(double) * (nq ? nq : 1)) : NULL;
  double *l = (double *)malloc(sizeof(double) * (nr ? nr : 1));
  int rc = 2;
  if (q && k && v && l && (!O || o)) {
    rc = oracle_attn_fwd_f64(q, k, v, seg, o, l, S, H, KV, d, (double)scale, nthreads);
    for (size_t i = 0; i < nr; ++i) LSE[i] = (float)l[i];
    if (O)
      for (size_t i = 0; i < nq; ++i) O[i] = (float)o[i];
  }
  free(q); free(k); free(v); free(o); free(l);
  return rc;
}

/* fp32 inputs; dQ, dK, dV are accumulated: out = fp32(fp64(out) + gradient).
 * O (may be NULL) is the forward output: when given, D = dO . O. */
int oracle_attn_bwd_o(const float *Q, const float *K, const float *V, const float *O,
                      const float *dO, const float *LSE, const uint32_t *seg, float *dQ,
                      float *dK, float *dV, int S, int H, int KV, int d, float scale,
                      int nthreads) {
  if (check_dims(S, H, KV, d)) return 1;
  if (S == 0) return 0;
  size_t nq = (size_t)S * H * d, nk = (size_t)S * KV * d, nr = (size_t)S * H;
  double *q = widen(Q, nq), *k = widen(K, nk), *v = widen(V, nk), *g = widen(dO, nq);
  double *l = widen(LSE, nr);
  double *o = O ? widen(O, nq) : NULL;
  double *gq = (double *)malloc(sizeof(double) * nq);
  double *gk = (double *)malloc(sizeof(double) * nk);
  double *gv = (double *)malloc(sizeof(double) * nk);
  int rc = 2;
  if (q && k && v && g && l && gq && gk && gv && (o || !O)) {
    rc = oracle_attn_bwd_o_f64(q, k, v, o, g, l, seg, gq, gk, gv, NULL, NULL, S, H, KV, d,
                               (double)scale, nthreads);
    for (size_t i = 0; i < nq; ++i) dQ[i] = (float)((double)dQ[i] + gq[i]);
    for (size_t i = 0; i < nk; ++i) {
      dK[i] = (float)((double)dK[i] + gk[i]);
      dV[i] = (float)((double)dV[i] + gv[i]);
    }
  }
  free(q); free(k); free(v); free(g); free(l); free(o); free(gq); free(gk); free(gv);
  return rc;
}

int oracle_attn_bwd(const float *Q, const float *K, const float *V, const float *dO,
                    const float *LSE, const uint32_t *seg, float *dQ, float *dK, float *dV, int S,
                    int H, int KV, int d, float scale, int nthreads) {
  return oracle_attn_bwd_o(Q, K, V, NULL, dO, LSE, seg, dQ, dK, dV, S, H, KV, d, scale, nthreads);
}

/* ------------------------------------------------------------------ */
/* rotary position embedding (RoPE) of interleaved column pairs         */
/* ------------------------------------------------------------------ */
/* Page "llm.istanbul -- 10_backward_attention.wgsl", kernels rope_q_backward
 * and rope_k_backward: for position s, head h and column pair (2p, 2p+1) of
 * X [S, NH, d], angle = (s + pos_offset) * base^(-2p/d).  The forward
 * rotation maps (x0, x1) to (x0 c - x1 s, x0 s + x1 c); the backward applies
 * its transpose, (g0, g1) -> (g0 c + g1 s, -g0 s + g1 c).  In place, fp64. */
int oracle_rope_f64(double *X, int S, int NH, int d, double base, long pos_offset, int backward) {
  if (S < 0 || NH < 1 || d < 2 || (d & 1) || !(base > 0.0)) return 1;
  for (long t = 0; t < S; ++t)
    for (int h = 0; h < NH; ++h)
      for (int pr = 0; pr < d / 2; ++pr) {
        double freq = pow(base, -2.0 * pr / (double)d);
        double ang = (double)(t + pos_offset) * freq;
        double c = cos(ang), sn = sin(ang);
        double *x = X + ((size_t)t * NH + h) * d + 2 * pr;
        double x0 = x[0], x1 = x[1];
        if (backward) {
          x[0] = x0 * c + x1 * sn;
          x[1] = -x0 * sn + x1 * c;
        } else {
          x[0] = x0 * c - x1 * sn;
          x[1] = x0 * sn + x1 * c;
        }
      }
  return 0;
}

/* The backward followed by the page's RoPE backward on dQ (n_heads) and dK
 * (n_kv_heads), in place: dQ = fp32(R^T(fp64(dQ) + gradient)), the same for
 * dK, and dV = fp32(fp64(dV) + gradient).  O may be NULL (see
 * oracle_attn_bwd_o).  Q and K are the rotated inputs the forward used. */
int oracle_attn_bwd_rope(const float *Q, const float *K, const float *V, const float *O,
                         const float *dO, const float *LSE, const uint32_t *seg, float *dQ,
                         float *dK, float *dV, int S, int H, int KV, int d, float scale,
                         double rope_base, long pos_offset, int nthreads) {
  if (check_dims(S, H, KV, d) || (d & 1) || !(rope_base > 0.0)) return 1;
  if (S == 0) return 0;
  size_t nq = (size_t)S * H * d, nk = (size_t)S * KV * d, nr = (size_t)S * H;
  double *q = widen(Q, nq), *k = widen(K, nk), *v = widen(V, nk), *g = widen(dO, nq);
  double *l = widen(LSE, nr);
  double *o = O ? widen(O, nq) : NULL;
  double *gq = (double *)malloc(sizeof(double) * nq);
  double *gk = (double *)malloc(sizeof(double) * nk);
  double *gv = (double *)malloc(sizeof(double) * nk);
  int rc = 2;
  if (q && k && v && g && l && gq && gk && gv && (o || !O)) {
    rc = oracle_attn_bwd_o_f64(q, k, v, o, g, l, seg, gq, gk, gv, NULL, NULL, S, H, KV, d,
                               (double)scale, nthreads);
    if (rc == 0) {
      for (size_t i = 0; i < nq; ++i) gq[i] += (double)dQ[i];
      for (size_t i = 0; i < nk; ++i) gk[i] += (double)dK[i];
      oracle_rope_f64(gq, S, H, d, rope_base, pos_offset, 1);
      oracle_rope_f64(gk, S, KV, d, rope_base, pos_offset, 1);
      for (size_t i = 0; i < nq; ++i) dQ[i] = (float)gq[i];
      for (size_t i = 0; i < nk; ++i) {
        dK[i] = (float)gk[i];
        dV[i] = (float)((double)dV[i] + gv[i]);
      }
    }
  }
  free(q); free(k); free(v); free(g); free(l); free(o); free(gq); free(gk); free(gv);
  return rc;
}

/* Selected rows only, for checks at sizes where the full backward is slow:
 * dQ for query rows q_rows[0..nq) -> dQ_sel [nq, H, d]; dK and dV for key rows
 * k_rows[0..nk) -> dK_sel, dV_sel [nk, KV, d].  Outputs are the fp64
 * gradients of this call (no accumulation).  D is computed only for the rows
 * the selection needs. */
int oracle_attn_bwd_rows_o(const float *Q, const float *K, const float *V, const float *O,
                           const float *dO, const float *LSE, const uint32_t *seg,
                           const int32_t *q_rows, int nq, const int32_t *k_rows, int nk,
                           double *dQ_sel, double *dK_sel, double *dV_sel, int S, int H, int KV,
                           int d, float scale, int nthreads) {
  if (check_dims(S, H, KV, d) || nq < 0 || nk < 0) return 1;
  for (int i = 0; i < nq; ++i)
    if (q_rows[i] < 0 || q_rows[i] >= S) return 1;
  for (int i = 0; i < nk; ++i)
    if (k_rows[i] < 0 || k_rows[i] >= S) return 1;
  if (S == 0) return 0;
  size_t n_q = (size_t)S * H * d, n_k = (size_t)S * KV * d, nr = (size_t)S * H;
  double *q = widen(Q, n_q), *k = widen(K, n_k), *v = widen(V, n_k), *g = widen(dO, n_q);
  double *l = widen(LSE, nr);
  double *o = O ? widen(O, n_q) : NULL;
  double *D = (double *)calloc(nr, sizeof(double));
  double *gq = (double *)calloc(n_q, sizeof(double));
  double *gk = (double *)calloc(n_k, sizeof(double));
  double *gv = (double *)calloc(n_k, sizeof(double));
  unsigned char *row_needed = (unsigned char *)calloc((size_t)S, 1);
  unsigned char *dq_needed = (unsigned char *)calloc((size_t)S, 1);
  unsigned char *key_needed = (unsigned char *)calloc((size_t)S, 1);
  int rc = 2;
  if (q && k && v && g && l && D && gq && gk && gv && row_needed && dq_needed && key_needed &&
      (o || !O)) {
    problem_t p = {q, k, v, g, l, seg, S, H, KV, d, (double)scale, o};
    for (int i = 0; i < nq; ++i) row_needed[q_rows[i]] = dq_needed[q_rows[i]] = 1;
    for (int i = 0; i < nk; ++i) {
      long j = k_rows[i];
      key_needed[j] = 1;
      for (long s = j; s < S; ++s)
        if (first_key(&p, s) <= j) row_needed[s] = 1;
    }
    bwd_ctx_t c = {&p, D, NULL, gq, gk, gv, row_needed, dq_needed, key_needed};
    parallel_for((long)S * H, nthreads, bwd_row, &c);
    parallel_for((long)S * KV, nthreads, bwd_key, &c);
    for (int i = 0; i < nq; ++i)
      memcpy(dQ_sel + (size_t)i * H * d, gq + (size_t)q_rows[i] * H * d, sizeof(double) * H * d);
    for (int i = 0; i < nk; ++i) {
      memcpy(dK_sel + (size_t)i * KV * d, gk + (size_t)k_rows[i] * KV * d,
             sizeof(double) * KV * d);
      memcpy(dV_sel + (size_t)i * KV * d, gv + (size_t)k_rows[i] * KV * d,
             sizeof(double) * KV * d);
    }
    rc = 0;
  }
  free(q); free(k); free(v); free(g); free(l); free(o); free(D); free(gq); free(gk); free(gv);
  free(row_needed); free(dq_needed); free(key_needed);
  return rc;
}

int oracle_attn_bwd_rows(const float *Q, const float *K, const float *V, const float *dO,
                         const float *LSE, const uint32_t *seg, const int32_t *q_rows, int nq,
                         const int32_t *k_rows, int nk, double *dQ_sel, double *dK_sel,
                         double *dV_sel, int S, int H, int KV, int d, float scale,
                         int nthreads) {
  return oracle_attn_bwd_rows_o(Q, K, V, NULL, dO, LSE, seg, q_rows, nq, k_rows, nk, dQ_sel,
                                dK_sel, dV_sel, S, H, KV, d, scale, nthreads);
}

/* ------------------------------------------------------------------ */
/* single-query backward over a KV history (one decode step)            */
/* ------------------------------------------------------------------ */
/* Page "rullama 0.5.0 -- src/backend/dispatch/training.rs",
 * attention_backward_dq_chained and attention_backward_dkv_chained (pass 1
 * and pass 2 of 2): one query per head attends to every one of the T keys of
 * a KV history, and the forward's probabilities P[h][j] are given (the stored
 * "probs"; nothing is recomputed).  Layouts: q, dO, dq [H, d]; P and the
 * staged score gradients [H, T]; K, V, dK, dV [T, KV, d].  Per head h, with
 * kv_h = h / (H/KV):
 *   dP[j] = dO_h . v_j
 *   D     = sum_j P[h][j] * dP[j]
 *   dS[j] = P[h][j] * (dP[j] - D)             (pass 1's staged d_scores)
 *   dq_h += scale * sum_j dS[j] * k_j          (pass 1)
 *   dK_j += scale * sum_{h in group} dS[j] * q_h   (pass 2, key-major)
 *   dV_j += sum_{h in group} P[h][j] * dO_h        (pass 2)
 * Plain loops in a fixed order, fp64.  The _f64 entry writes the gradients
 * (no accumulation) and optionally dS; the float entry adds into its outputs
 * and rounds once: out = (float)((double)init + gradient). */
int oracle_attn_bwd_decode_f64(const double *q, const double *K, const double *V,
                               const double *P, const double *dO, double *dq, double *dK,
                               double *dV, double *dS_out, int T, int H, int KV, int d,
                               double scale) {
  if (T < 0 || H < 1 || KV < 1 || d < 1 || H % KV != 0) return 1;
  const int g = H / KV;
  double *ds = (double *)malloc(sizeof(double) * ((size_t)H * T + 1));
  if (!ds) return 2;
  memset(dq, 0, sizeof(double) * (size_t)H * d);
  memset(dK, 0, sizeof(double) * (size_t)T * KV * d);
  memset(dV, 0, sizeof(double) * (size_t)T * KV * d);
  /* pass 1: score gradients and dq, head by head */
  for (int h = 0; h < H; ++h) {
    const int kvh = h / g;
    const double *doh = dO + (size_t)h * d;
    double D = 0.0;
    for (long j = 0; j < T; ++j) {
      const double dp = dot(doh, V + ((size_t)j * KV + kvh) * d, d);
      ds[(size_t)h * T + j] = dp; /* dP for now */
      D += P[(size_t)h * T + j] * dp;
    }
    for (long j = 0; j < T; ++j) {
      const size_t k = (size_t)h * T + j;
      ds[k] = P[k] * (ds[k] - D);
    }
    for (long j = 0; j < T; ++j) {
      const double *kj = K + ((size_t)j * KV + kvh) * d;
      const double w = scale * ds[(size_t)h * T + j];
      for (int c = 0; c < d; ++c) dq[(size_t)h * d + c] += w * kj[c];
    }
  }
  /* pass 2: key-major dK and dV, the group's heads in order */
  for (long j = 0; j < T; ++j)
    for (int kvh = 0; kvh < KV; ++kvh) {
      double *dk = dK + ((size_t)j * KV + kvh) * d;
      double *dv = dV + ((size_t)j * KV + kvh) * d;
      for (int hh = 0; hh < g; ++hh) {
        const int h = kvh * g + hh;
        const double wk = scale * ds[(size_t)h * T + j], wv = P[(size_t)h * T + j];
        for (int c = 0; c < d; ++c) {
          dk[c] += wk * q[(size_t)h * d + c];
          dv[c] += wv * dO[(size_t)h * d + c];
        }
      }
    }
  if (dS_out) memcpy(dS_out, ds, sizeof(double) * (size_t)H * T);
  free(ds);
  return 0;
}

int oracle_attn_bwd_decode(const float *q, const float *K, const float *V, const float *P,
                           const float *dO, float *dq, float *dK, float *dV, int T, int H, int KV,
                           int d, float scale) {
  if (T < 0 || H < 1 || KV < 1 || d < 1 || H % KV != 0) return 1;
  const size_t nq = (size_t)H * d, nk = (size_t)T * KV * d, np_ = (size_t)H * T;
  double *q64 = widen(q, nq), *K64 = widen(K, nk), *V64 = widen(V, nk), *P64 = widen(P, np_);
  double *dO64 = widen(dO, nq);
  double *gq = (double *)malloc(sizeof(double) * (nq + 1));
  double *gk = (double *)malloc(sizeof(double) * (nk + 1));
  double *gv = (double *)malloc(sizeof(double) * (nk + 1));
  int rc = 2;
  if (q64 && K64 && V64 && P64 && dO64 && gq && gk && gv) {
    rc = oracle_attn_bwd_decode_f64(q64, K64, V64, P64, dO64, gq, gk, gv, NULL, T, H, KV, d,
                                    (double)scale);
    if (rc == 0) {
      for (size_t i = 0; i < nq; ++i) dq[i] = (float)((double)dq[i] + gq[i]);
      for (size_t i = 0; i < nk; ++i) {
        dK[i] = (float)((double)dK[i] + gk[i]);
        dV[i] = (float)((double)dV[i] + gv[i]);
      }
    }
  }
  free(q64); free(K64); free(V64); free(P64); free(dO64); free(gq); free(gk); free(gv);
  return rc;
}
