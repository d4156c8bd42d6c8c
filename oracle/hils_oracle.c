/*
 * HiLS-Attention forward pass and its backward -- float64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library: it is a plain, slow, loop-by-loop restatement of the
 * method as the pages define it, in float64, so that a reader can hold each
 * function against its equation.
 *
 * Sources (the pages about arXiv 2607.02980, "Hierarchical Sparse Attention
 * Done Right: Toward Infinite Context Modeling"):
 *   [p1] picx.dev summary -- Methodology section 1 (Eq. 7, Eq. 8),
 *        section 2 (Eq. 10 and the definition of Z-hat under it),
 *        section 3 (Q-Cal, GQA adaptation).
 *   [p3] rcap.io explainer -- the per-query pseudo-code (score every chunk,
 *        arg-top-K, hierarchical softmax per chunk, sliding-window term) and
 *        the recipe (chunk 64, window 512).
 *
 * Readings where the pages leave a step open (all recorded with the build's
 * design notes):
 *   R1  window and chunks partition [0, i] exactly: w0 = max(0, i-W+1),
 *       n_i = floor(w0 / S) complete chunks lie before the window, and the
 *       window is the token range [n_i*S, i].
 *   R2  one joint normaliser: Z-hat_i = sum over selected chunks of
 *       exp(s-hat_{i,c}) + sum over window tokens of exp(s_{i,j}).
 *   R3  selection per GQA group by the maximum over the group's heads.
 *   R4  each head fuses its chunks with its own s-hat_{i,c}.
 *   R5  one landmark query per (query head, chunk): k'_c, b'_c per query head.
 *   R7  q-hat only in chunk scoring and Z-hat; token logits use the raw q.
 *   R8  Q-Cal: q-hat = q + slice_h(W_up (W_down h_i)), W_down [r, D_h],
 *       W_up [H_q*d, r] shared by all heads.
 *   R10 top-K order: score descending, chunk index ascending; pad -1.
 *   R11 a decode query sits at position seq_len-1.
 *   R13 tau = 1/sqrt(d) unless a scale is given; causal including j = i.
 *
 * Data types of inputs: 0 = bf16 bit patterns (uint16), 1 = f32, 2 = f64.
 * Every value is widened exactly to double on load.  Sums run sequentially
 * in ascending index order; threads split only independent output units.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int B, T, Hq, Hkv, d, S, K, W, r, Dh;
  double scale; /* 0 -> 1/sqrt(d) */
} orc_cfg;

enum { DT_BF16 = 0, DT_F32 = 1, DT_F64 = 2 };

static double ld(const void *p, int dt, size_t i) {
  if (dt == DT_F64) return ((const double *)p)[i];
  if (dt == DT_F32) return (double)((const float *)p)[i];
  uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double tau_of(const orc_cfg *c) {
  return c->scale > 0 ? c->scale : 1.0 / sqrt((double)c->d);
}

/* R1: number of complete chunks that lie before query i's window. */
int orc_eligible_chunks(int i, int W, int S) {
  int w0 = i - W + 1;
  if (w0 < 0) w0 = 0;
  return w0 / S;
}

/* ------------------------------------------------------------------------ */
/* a tiny fork/join helper over independent units                            */
typedef void (*unit_fn)(void *ctx, long unit);
typedef struct { unit_fn fn; void *ctx; long lo, hi; } span_t;

static void *run_span(void *a) {
  span_t *s = (span_t *)a;
  for (long u = s->lo; u < s->hi; ++u) s->fn(s->ctx, u);
  return 0;
}

static void parallel_for(long n, int nthreads, unit_fn fn, void *ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  pthread_t th[256];
  span_t sp[256];
  int ok[256];
  long per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    sp[t].fn = fn; sp[t].ctx = ctx;
    sp[t].lo = t * per; sp[t].hi = (t + 1) * per < n ? (t + 1) * per : n;
    ok[t] = pthread_create(&th[t], 0, run_span, &sp[t]) == 0;
    if (!ok[t]) run_span(&sp[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], 0);
}

/* ------------------------------------------------------------------------ */
/* Landmark chunk summary, [p1] Methodology 1, Eq. 8:
 *   p_j  = softmax_j( q'_c . k_j / sqrt(d) )   over the chunk's S keys
 *   k'_c = sum_j p_j k_j
 *   b'_c = - sum_j p_j log p_j                  (entropy; 0 log 0 = 0)
 * One landmark query per query head (R5); the keys are the KV head's.
 * k [B,Hkv,T,d], q_lm [B,Hq,C,d]  ->  k_sum [B,Hq,C,d], b_sum [B,Hq,C]   */
typedef struct {
  const orc_cfg *c; const void *k; int kdt; const void *qlm; int qdt;
  int c0, c1; double *ksum, *bsum;
} sum_ctx;

static void summary_unit(void *vctx, long unit) {
  sum_ctx *x = (sum_ctx *)vctx;
  const orc_cfg *c = x->c;
  int C = c->T / c->S, G = c->Hq / c->Hkv;
  int b = (int)(unit / c->Hq), h = (int)(unit % c->Hq), g = h / G;
  double tau = tau_of(c);
  double *logit = (double *)malloc(sizeof(double) * c->S);
  double *p = (double *)malloc(sizeof(double) * c->S);
  for (int ch = x->c0; ch < x->c1; ++ch) {
    size_t qoff = (((size_t)b * c->Hq + h) * C + ch) * c->d;
    for (int j = 0; j < c->S; ++j) {
      size_t koff = (((size_t)b * c->Hkv + g) * c->T + (size_t)ch * c->S + j) * c->d;
      double acc = 0;
      for (int e = 0; e < c->d; ++e) acc += ld(x->qlm, x->qdt, qoff + e) * ld(x->k, x->kdt, koff + e);
      logit[j] = tau * acc;
    }
    double m = logit[0];
    for (int j = 1; j < c->S; ++j) if (logit[j] > m) m = logit[j];
    double den = 0;
    for (int j = 0; j < c->S; ++j) den += exp(logit[j] - m);
    for (int j = 0; j < c->S; ++j) p[j] = exp(logit[j] - m) / den;
    size_t so = (((size_t)b * c->Hq + h) * C + ch);
    for (int e = 0; e < c->d; ++e) {
      double acc = 0;
      for (int j = 0; j < c->S; ++j) {
        size_t koff = (((size_t)b * c->Hkv + g) * c->T + (size_t)ch * c->S + j) * c->d;
        acc += p[j] * ld(x->k, x->kdt, koff + e);
      }
      x->ksum[so * c->d + e] = acc;
    }
    double ent = 0;
    for (int j = 0; j < c->S; ++j)
      if (p[j] > 0) ent -= p[j] * log(p[j]);
    x->bsum[so] = ent;
  }
  free(logit);
  free(p);
}

int orc_summary(const orc_cfg *c, const void *k, int kdt, const void *q_lm, int qdt,
                int c0, int c1, double *k_sum, double *b_sum, int nthreads) {
  sum_ctx x = {c, k, kdt, q_lm, qdt, c0, c1, k_sum, b_sum};
  parallel_for((long)c->B * c->Hq, nthreads, summary_unit, &x);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Low-rank query calibration, [p1] Methodology 3 (Q-Cal):
 *   q-hat_i = q_i + W_up W_down h_i ; head h takes rows h*d .. h*d+d-1 (R8).
 * q [B,Hq,nq,d], h [B,nq,Dh], W_down [r,Dh], W_up [Hq*d,r] -> q-hat [B,Hq,nq,d]
 * With r == 0, q-hat = q.                                                     */
typedef struct {
  const orc_cfg *c; const void *q; int qdt; const void *h; int hdt;
  const void *wd; const void *wu; int wdt; int nq; double *qhat;
} qcal_ctx;

static void qcal_unit(void *vctx, long unit) {
  qcal_ctx *x = (qcal_ctx *)vctx;
  const orc_cfg *c = x->c;
  int r = c->r, Dh = c->Dh, d = c->d, nq = x->nq;
  int b = (int)(unit / nq), t = (int)(unit % nq);
  double *u = (double *)malloc(sizeof(double) * (r > 0 ? r : 1));
  for (int a = 0; a < r; ++a) { /* u = W_down h_i */
    double acc = 0;
    for (int e = 0; e < Dh; ++e)
      acc += ld(x->wd, x->wdt, (size_t)a * Dh + e) * ld(x->h, x->hdt, ((size_t)b * nq + t) * Dh + e);
    u[a] = acc;
  }
  for (int hh = 0; hh < c->Hq; ++hh) /* q-hat = q + W_up u, head slice */
    for (int e = 0; e < d; ++e) {
      size_t o = (((size_t)b * c->Hq + hh) * nq + t) * d + e;
      double res = 0;
      for (int a = 0; a < r; ++a) res += ld(x->wu, x->wdt, ((size_t)hh * d + e) * r + a) * u[a];
      x->qhat[o] = ld(x->q, x->qdt, o) + res;
    }
  free(u);
}

int orc_qcal(const orc_cfg *c, const void *q, int qdt, const void *h, int hdt,
             const void *w_down, const void *w_up, int wdt, int nq, double *qhat, int nthreads) {
  qcal_ctx x = {c, q, qdt, h, hdt, w_down, w_up, wdt, nq, qhat};
  parallel_for((long)c->B * nq, nthreads, qcal_unit, &x);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Chunk scores, [p1] Eq. 7 read through Eq. 10's definition of s-hat:
 *   s_{i,c} = q-hat_i . k'_c * tau + b'_c   for the n_i eligible chunks (R1);
 *   -inf for chunks that are not eligible.
 * qhat [B,Hq,nq,d] (double), qpos [B,nq], k_sum [B,Hq,C,d], b_sum [B,Hq,C]
 *   -> s [B,Hq,nq,C]                                                        */
typedef struct {
  const orc_cfg *c; const double *qhat; const int *qpos; int nq;
  const void *ks; int ksdt; const void *bs; int bsdt; double *s;
} score_ctx;

static void score_unit(void *vctx, long unit) {
  score_ctx *x = (score_ctx *)vctx;
  const orc_cfg *c = x->c;
  int C = c->T / c->S;
  int t = (int)(unit % x->nq), h = (int)((unit / x->nq) % c->Hq), b = (int)(unit / ((long)x->nq * c->Hq));
  int i = x->qpos[(size_t)b * x->nq + t];
  int n = orc_eligible_chunks(i, c->W, c->S);
  if (n > C) n = C;
  double tau = tau_of(c);
  const double *qv = x->qhat + (((size_t)b * c->Hq + h) * x->nq + t) * c->d;
  double *out = x->s + (((size_t)b * c->Hq + h) * x->nq + t) * C;
  for (int ch = 0; ch < C; ++ch) {
    if (ch >= n) { out[ch] = -INFINITY; continue; }
    size_t so = ((size_t)b * c->Hq + h) * C + ch;
    double acc = 0;
    for (int e = 0; e < c->d; ++e) acc += qv[e] * ld(x->ks, x->ksdt, so * c->d + e);
    out[ch] = tau * acc + ld(x->bs, x->bsdt, so);
  }
}

int orc_scores(const orc_cfg *c, const double *qhat, const int *qpos, int nq,
               const void *k_sum, int ksdt, const void *b_sum, int bsdt, double *s,
               int nthreads) {
  score_ctx x = {c, qhat, qpos, nq, k_sum, ksdt, b_sum, bsdt, s};
  parallel_for((long)c->B * c->Hq * nq, nthreads, score_unit, &x);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Top-K chunk selection, [p3] pseudo-code (arg-top-K of the chunk scores) with
 * [p1] Methodology 3 (GQA adaptation): sigma_c = max over the group's heads of
 * s_{i,c,h}; keep the min(K, n_i) best by (sigma desc, c asc) (R3, R10).
 *   idx [B,Hkv,nq,K] (pad -1), tsc [B,Hq,nq,K] = each head's own s of the
 *   selected chunks (pad -inf), sigma [B,Hkv,nq,C] if non-NULL.             */
int orc_select(const orc_cfg *c, const double *s, const int *qpos, int nq, int *idx,
               double *tsc, double *sigma_out) {
  int C = c->T / c->S, G = c->Hq / c->Hkv, K = c->K;
  double *sig = (double *)malloc(sizeof(double) * (C > 0 ? C : 1));
  char *taken = (char *)malloc(C > 0 ? C : 1);
  for (int b = 0; b < c->B; ++b)
    for (int g = 0; g < c->Hkv; ++g)
      for (int t = 0; t < nq; ++t) {
        int i = qpos[(size_t)b * nq + t];
        int n = orc_eligible_chunks(i, c->W, c->S);
        if (n > C) n = C;
        for (int ch = 0; ch < C; ++ch) {
          double m = -INFINITY;
          for (int hh = g * G; hh < (g + 1) * G; ++hh) {
            double v = s[(((size_t)b * c->Hq + hh) * nq + t) * C + ch];
            if (v > m) m = v;
          }
          sig[ch] = ch < n ? m : -INFINITY;
          taken[ch] = 0;
        }
        if (sigma_out) memcpy(sigma_out + (((size_t)b * c->Hkv + g) * nq + t) * C, sig, sizeof(double) * C);
        int keep = n < K ? n : K;
        for (int k = 0; k < K; ++k) {
          /* k-th pick: the best chunk not taken yet; a strict '>' keeps the
             lower index among equal scores */
          int ch = -1;
          if (k < keep)
            for (int cand = 0; cand < n; ++cand)
              if (!taken[cand] && (ch < 0 || sig[cand] > sig[ch])) ch = cand;
          if (ch >= 0) taken[ch] = 1;
          idx[(((size_t)b * c->Hkv + g) * nq + t) * K + k] = ch;
          for (int hh = g * G; hh < (g + 1) * G; ++hh)
            tsc[(((size_t)b * c->Hq + hh) * nq + t) * K + k] =
                ch >= 0 ? s[(((size_t)b * c->Hq + hh) * nq + t) * C + ch] : -INFINITY;
        }
      }
  free(sig);
  free(taken);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Hierarchical softmax fusion, [p1] Methodology 2, Eq. 10, with the window
 * of [p3]'s pseudo-code and [p1]'s joint normaliser (R2):
 *   for j in a selected chunk c:  w_ij = exp(s_ij) / Z_{i,c} * Zhat_{i,c} / Zhat_i
 *   for j in the window:          w_ij = exp(s_ij) / Zhat_i
 *   Zhat_{i,c} = exp(alpha_c),  Zhat_i = sum_c Zhat_{i,c} + sum_{j in window} exp(s_ij)
 *   o_i = sum_j w_ij v_j
 * s_ij = tau q_i . k_j with the raw q (R7); alpha_c = the head's own chunk
 * score s-hat_{i,c} (R4), or log Z_{i,c} itself in exact-mass mode (a test
 * mode that replaces the surrogate with the true chunk mass).  Every
 * exponential is taken relative to a common shift, which cancels in w_ij.
 * q [B,Hq,nq,d] raw, k/v [B,Hkv,T,d], qpos [B,nq], idx [B,Hkv,nq,K],
 * tsc [B,Hq,nq,K] -> o [B,Hq,nq,d]; wsum [B,Hq,nq] = sum_j w_ij if non-NULL. */
typedef struct {
  const orc_cfg *c; const void *q; int qdt; const void *k; const void *v; int kvdt;
  const int *qpos; int nq; const int *idx; const double *tsc; int exact;
  double *o; double *wsum;
} fuse_ctx;

static void fuse_unit(void *vctx, long unit) {
  fuse_ctx *x = (fuse_ctx *)vctx;
  const orc_cfg *c = x->c;
  int d = c->d, S = c->S, K = c->K, G = c->Hq / c->Hkv;
  int t = (int)(unit % x->nq), h = (int)((unit / x->nq) % c->Hq), b = (int)(unit / ((long)x->nq * c->Hq));
  int g = h / G;
  int i = x->qpos[(size_t)b * x->nq + t];
  int n = orc_eligible_chunks(i, c->W, c->S);
  double tau = tau_of(c);
  size_t qoff = (((size_t)b * c->Hq + h) * x->nq + t) * d;
  size_t kvbase = ((size_t)b * c->Hkv + g) * c->T;
  int w_lo = n * S, w_hi = i; /* window tokens [w_lo, w_hi] (R1) */
  int nw = w_hi - w_lo + 1;
  int kk = K > 0 ? K : 1;
  double *lam = (double *)malloc(sizeof(double) * ((size_t)(K > 0 ? K : 0) * S + (nw > 0 ? nw : 1)));
  double *chunk_max = (double *)malloc(sizeof(double) * kk);
  double *chunk_z = (double *)malloc(sizeof(double) * kk);
  double *alpha = (double *)malloc(sizeof(double) * kk);
  int *chunk = (int *)malloc(sizeof(int) * kk);
  int nsel = 0;
  /* token logits of the selected chunks and their masses Z_{i,c} */
  for (int k = 0; k < K; ++k) {
    int ch = x->idx[(((size_t)b * c->Hkv + g) * x->nq + t) * K + k];
    if (ch < 0) continue;
    double *l = lam + (size_t)nsel * S;
    for (int j = 0; j < S; ++j) {
      size_t koff = (kvbase + (size_t)ch * S + j) * d;
      double acc = 0;
      for (int e = 0; e < d; ++e) acc += ld(x->q, x->qdt, qoff + e) * ld(x->k, x->kvdt, koff + e);
      l[j] = tau * acc;
    }
    double m = l[0];
    for (int j = 1; j < S; ++j) if (l[j] > m) m = l[j];
    double z = 0;
    for (int j = 0; j < S; ++j) z += exp(l[j] - m);
    chunk[nsel] = ch;
    chunk_max[nsel] = m;
    chunk_z[nsel] = z; /* Z_{i,c} = exp(m) * z */
    alpha[nsel] = x->exact ? m + log(z) : x->tsc[(((size_t)b * c->Hq + h) * x->nq + t) * K + k];
    ++nsel;
  }
  /* window logits */
  double *lw = lam + (size_t)nsel * S;
  for (int j = 0; j < nw; ++j) {
    size_t koff = (kvbase + (size_t)(w_lo + j)) * d;
    double acc = 0;
    for (int e = 0; e < d; ++e) acc += ld(x->q, x->qdt, qoff + e) * ld(x->k, x->kvdt, koff + e);
    lw[j] = tau * acc;
  }
  /* common shift M and the joint normaliser Zhat_i (times exp(-M)) */
  double M = -INFINITY;
  for (int a = 0; a < nsel; ++a) if (alpha[a] > M) M = alpha[a];
  for (int j = 0; j < nw; ++j) if (lw[j] > M) M = lw[j];
  double zhat = 0;
  for (int a = 0; a < nsel; ++a) zhat += exp(alpha[a] - M);
  for (int j = 0; j < nw; ++j) zhat += exp(lw[j] - M);
  double *out = x->o + qoff;
  for (int e = 0; e < d; ++e) out[e] = 0;
  double wtot = 0;
  for (int a = 0; a < nsel; ++a) {
    double inter = exp(alpha[a] - M) / zhat; /* Zhat_{i,c} / Zhat_i */
    const double *l = lam + (size_t)a * S;
    for (int j = 0; j < S; ++j) {
      double w = exp(l[j] - chunk_max[a]) / chunk_z[a] * inter; /* exp(s_ij)/Z_{i,c} * ... */
      size_t voff = (kvbase + (size_t)chunk[a] * S + j) * d;
      for (int e = 0; e < d; ++e) out[e] += w * ld(x->v, x->kvdt, voff + e);
      wtot += w;
    }
  }
  for (int j = 0; j < nw; ++j) {
    double w = exp(lw[j] - M) / zhat;
    size_t voff = (kvbase + (size_t)(w_lo + j)) * d;
    for (int e = 0; e < d; ++e) out[e] += w * ld(x->v, x->kvdt, voff + e);
    wtot += w;
  }
  if (x->wsum) x->wsum[((size_t)b * c->Hq + h) * x->nq + t] = wtot;
  free(lam); free(chunk_max); free(chunk_z); free(alpha); free(chunk);
}

int orc_fuse(const orc_cfg *c, const void *q, int qdt, const void *k, const void *v, int kvdt,
             const int *qpos, int nq, const int *idx, const double *tsc, int exact_mass,
             double *o, double *wsum, int nthreads) {
  fuse_ctx x = {c, q, qdt, k, v, kvdt, qpos, nq, idx, tsc, exact_mass, o, wsum};
  parallel_for((long)c->B * c->Hq * nq, nthreads, fuse_unit, &x);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Full causal softmax attention for the given query rows (the dense
 * comparator the pages measure against): o_i = sum_{j<=i} softmax_j(s_ij) v_j. */
typedef struct {
  const orc_cfg *c; const void *q; int qdt; const void *k; const void *v; int kvdt;
  const int *qpos; int nq; double *o;
} dense_ctx;

static void dense_unit(void *vctx, long unit) {
  dense_ctx *x = (dense_ctx *)vctx;
  const orc_cfg *c = x->c;
  int d = c->d, G = c->Hq / c->Hkv;
  int t = (int)(unit % x->nq), h = (int)((unit / x->nq) % c->Hq), b = (int)(unit / ((long)x->nq * c->Hq));
  int i = x->qpos[(size_t)b * x->nq + t];
  double tau = tau_of(c);
  size_t qoff = (((size_t)b * c->Hq + h) * x->nq + t) * d;
  size_t kvbase = ((size_t)b * c->Hkv + h / G) * c->T;
  double *l = (double *)malloc(sizeof(double) * ((size_t)i + 1));
  double m = -INFINITY;
  for (int j = 0; j <= i; ++j) {
    double acc = 0;
    for (int e = 0; e < d; ++e) acc += ld(x->q, x->qdt, qoff + e) * ld(x->k, x->kvdt, (kvbase + j) * d + e);
    l[j] = tau * acc;
    if (l[j] > m) m = l[j];
  }
  double z = 0;
  for (int j = 0; j <= i; ++j) z += exp(l[j] - m);
  double *out = x->o + qoff;
  for (int e = 0; e < d; ++e) out[e] = 0;
  for (int j = 0; j <= i; ++j) {
    double w = exp(l[j] - m) / z;
    for (int e = 0; e < d; ++e) out[e] += w * ld(x->v, x->kvdt, (kvbase + j) * d + e);
  }
  free(l);
}

int orc_causal_attention(const orc_cfg *c, const void *q, int qdt, const void *k, const void *v,
                         int kvdt, const int *qpos, int nq, double *o, int nthreads) {
  dense_ctx x = {c, q, qdt, k, v, kvdt, qpos, nq, o};
  parallel_for((long)c->B * c->Hq * nq, nthreads, dense_unit, &x);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Storage rounding of a float64 value to bf16 (round to nearest, ties to
 * even, 8 significant bits), used where the stored k' is bf16.             */
static uint16_t round_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0) return sign;
  int e;
  frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
  int q = e - 8;                /* quantum exponent: 8 significant bits */
  if (q < -133) q = -133;       /* bf16 subnormal spacing is 2^-133 */
  double m = nearbyint(ldexp(a, -q)); /* ties to even under the default mode */
  double y = ldexp(m, q);
  if (y >= 0x1p128) return sign | 0x7F80; /* rounds past the largest finite bf16 */
  float f = (float)y;           /* exact: y has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

void orc_round_bf16(const double *x, uint16_t *out, long n) {
  for (long i = 0; i < n; ++i) out[i] = round_to_bf16(x[i]);
}

/* ======================================================================== */
/* Backward pass of the forward above, for a FIXED selection.
 *
 * The pages train chunk selection through the forward weights: the score
 * s-hat of each selected chunk sits inside the joint softmax of Eq. 10
 * ([p1] Methodology 2), so the loss reaches s-hat, hence k'_c and b'_c,
 * hence (Eq. 8, [p1] Methodology 1) the landmark query q'_c and the chunk's
 * keys, and (Q-Cal, [p1] Methodology 3) the calibration weights.  The top-K
 * choice itself is a discrete step and carries no gradient.  Given dO =
 * dL/dO for every output row, this returns the exact gradients of
 * L = sum(dO * O) with respect to q, k, v, the landmark queries and, with
 * Q-Cal, h, W_down and W_up.
 *
 * Per row (b, h, i), with the entries of the row's selection list (c >= 0)
 * and the window tokens j, and logZ = log( sum_c e^{s_c} + sum_j e^{l_j} ):
 *   w_c = e^{s_c - logZ},  u_j = e^{l_j - logZ},  o = sum_c w_c o_c + sum_j u_j v_j
 *   Delta = dO . o
 *   ds_c           = w_c (dO . o_c - Delta)                  (joint softmax)
 *   dl_j (chunk c) = w_c P_cj (dO . v_j - dO . o_c)          (chunk softmax)
 *   dl_j (window)  = u_j (dO . v_j - Delta)
 *   dv_j += w_c P_cj dO  or  u_j dO
 *   dq += tau sum_j dl_j k_j,    dk_j += tau dl_j q          (l_j = tau q.k_j)
 *   dq-hat += tau ds_c k'_c,  dk'_c += tau ds_c q-hat,  db'_c += ds_c
 * Summary (Eq. 8) per (b, h, c), l_j = tau q'_c.k_j, p = softmax(l),
 * k' = sum_j p_j k_j, b' = -sum_j p_j log p_j = LSE(l) - E_p[l]:
 *   dl_j = p_j ( dk'.(k_j - k') - db' (l_j - E_p[l]) )
 *   dq'_c += tau sum_j dl_j k_j,   dk_j += p_j dk' + tau dl_j q'_c
 * The stored k' (rounded to the storage type in the forward) enters s-hat
 * as given; the rounding is taken as the identity in the chain.
 * Q-Cal: q-hat_h = q_h + (W_up u)[h d : h d + d], u = W_down h_i:
 *   dq_h += dq-hat_h,   du = sum_h W_up[h d + e, :]^T dq-hat_h[e],
 *   dW_up[h d + e, a] += dq-hat_h[e] u_a,  dW_down += du h_i^T,  dh_i = W_down^T du.
 *
 * Inputs as in the forward: q [B,Hq,T,d], k, v [B,Hkv,T,d], q_lm
 * [B,Hq,C,d], h [B,T,Dh], w_down [r,Dh], w_up [Hq*d, r], idx [B,Hkv,T,K],
 * k_sum [B,Hq,C,d] (stored), b_sum [B,Hq,C], dO [B,Hq,T,d].  Outputs are
 * float64, overwritten: dq, dk, dv, dq_lm and (r > 0) dh, dw_down, dw_up. */
typedef struct {
  const orc_cfg *c;
  const void *q; int qdt; const void *k; const void *v; int kvdt; const void *qlm; int lmdt;
  const int *idx; const void *ksum; int ksdt; const void *bsum; int bsdt; const void *dout; int dodt;
  const double *qhat; /* [B,Hq,T,d] */
  double *dq, *dk, *dv, *dqlm, *dqhat, *dks, *dbs;
} bwd_ctx;

/* one (b, g) pair: every row of its heads, then its chunk summaries */
static void bwd_pair_unit(void *vctx, long unit) {
  bwd_ctx *x = (bwd_ctx *)vctx;
  const orc_cfg *c = x->c;
  int d = c->d, S = c->S, K = c->K, T = c->T, C = c->T / c->S, G = c->Hq / c->Hkv;
  int b = (int)(unit / c->Hkv), g = (int)(unit % c->Hkv);
  double tau = tau_of(c);
  size_t kvbase = ((size_t)b * c->Hkv + g) * T;
  int kk = K > 0 ? K : 1;
  double *lam = (double *)malloc(sizeof(double) * ((size_t)kk * S + T));
  double *P = (double *)malloc(sizeof(double) * (size_t)kk * S);
  double *ob = (double *)malloc(sizeof(double) * (size_t)kk * d);
  double *s_hat = (double *)malloc(sizeof(double) * kk);
  int *chunk = (int *)malloc(sizeof(int) * kk);
  double *o = (double *)malloc(sizeof(double) * d);
  double *dO = (double *)malloc(sizeof(double) * d);
  double *qv = (double *)malloc(sizeof(double) * d);
  for (int hh = 0; hh < G; ++hh) {
    int h = g * G + hh;
    for (int i = 0; i < T; ++i) {
      size_t qoff = (((size_t)b * c->Hq + h) * T + i) * d;
      int n = orc_eligible_chunks(i, c->W, S);
      int w_lo = n * S, nw = i - w_lo + 1;
      for (int e = 0; e < d; ++e) { qv[e] = ld(x->q, x->qdt, qoff + e); dO[e] = ld(x->dout, x->dodt, qoff + e); }
      const double *qh = x->qhat + qoff;
      /* the selected chunks: s-hat from the stored summaries, token logits,
       * chunk softmax P_c and chunk output o_c */
      int nsel = 0;
      for (int k = 0; k < K; ++k) {
        int ch = x->idx[(kvbase + i) * K + k];
        if (ch < 0) continue;
        size_t so = ((size_t)b * c->Hq + h) * C + ch;
        double acc = 0;
        for (int e = 0; e < d; ++e) acc += qh[e] * ld(x->ksum, x->ksdt, so * d + e);
        s_hat[nsel] = tau * acc + ld(x->bsum, x->bsdt, so);
        double *l = lam + (size_t)nsel * S, *p = P + (size_t)nsel * S;
        for (int j = 0; j < S; ++j) {
          size_t koff = (kvbase + (size_t)ch * S + j) * d;
          double a2 = 0;
          for (int e = 0; e < d; ++e) a2 += qv[e] * ld(x->k, x->kvdt, koff + e);
          l[j] = tau * a2;
        }
        double m = l[0];
        for (int j = 1; j < S; ++j) if (l[j] > m) m = l[j];
        double z = 0;
        for (int j = 0; j < S; ++j) z += exp(l[j] - m);
        for (int j = 0; j < S; ++j) p[j] = exp(l[j] - m) / z;
        double *oc = ob + (size_t)nsel * d;
        for (int e = 0; e < d; ++e) {
          double a3 = 0;
          for (int j = 0; j < S; ++j) a3 += p[j] * ld(x->v, x->kvdt, (kvbase + (size_t)ch * S + j) * d + e);
          oc[e] = a3;
        }
        chunk[nsel++] = ch;
      }
      /* window logits and the joint log-normaliser */
      double *lw = lam + (size_t)nsel * S;
      for (int j = 0; j < nw; ++j) {
        size_t koff = (kvbase + (size_t)(w_lo + j)) * d;
        double a2 = 0;
        for (int e = 0; e < d; ++e) a2 += qv[e] * ld(x->k, x->kvdt, koff + e);
        lw[j] = tau * a2;
      }
      double M = -INFINITY;
      for (int a = 0; a < nsel; ++a) if (s_hat[a] > M) M = s_hat[a];
      for (int j = 0; j < nw; ++j) if (lw[j] > M) M = lw[j];
      double z = 0;
      for (int a = 0; a < nsel; ++a) z += exp(s_hat[a] - M);
      for (int j = 0; j < nw; ++j) z += exp(lw[j] - M);
      double logZ = M + log(z);
      /* the output row and Delta = dO . o */
      for (int e = 0; e < d; ++e) o[e] = 0;
      for (int a = 0; a < nsel; ++a) {
        double w = exp(s_hat[a] - logZ);
        for (int e = 0; e < d; ++e) o[e] += w * ob[(size_t)a * d + e];
      }
      for (int j = 0; j < nw; ++j) {
        double u = exp(lw[j] - logZ);
        for (int e = 0; e < d; ++e) o[e] += u * ld(x->v, x->kvdt, (kvbase + (size_t)(w_lo + j)) * d + e);
      }
      double Delta = 0;
      for (int e = 0; e < d; ++e) Delta += dO[e] * o[e];
      double *dq = x->dq + qoff, *dqh = x->dqhat + qoff;
      /* chunk terms */
      for (int a = 0; a < nsel; ++a) {
        int ch = chunk[a];
        double w = exp(s_hat[a] - logZ);
        const double *oc = ob + (size_t)a * d, *p = P + (size_t)a * S;
        double dOo = 0;
        for (int e = 0; e < d; ++e) dOo += dO[e] * oc[e];
        double ds = w * (dOo - Delta);
        size_t so = ((size_t)b * c->Hq + h) * C + ch;
        for (int e = 0; e < d; ++e) {
          dqh[e] += tau * ds * ld(x->ksum, x->ksdt, so * d + e);
          x->dks[so * d + e] += tau * ds * qh[e];
        }
        x->dbs[so] += ds;
        for (int j = 0; j < S; ++j) {
          size_t koff = (kvbase + (size_t)ch * S + j) * d;
          double dOv = 0;
          for (int e = 0; e < d; ++e) dOv += dO[e] * ld(x->v, x->kvdt, koff + e);
          double dl = w * p[j] * (dOv - dOo);
          for (int e = 0; e < d; ++e) {
            dq[e] += tau * dl * ld(x->k, x->kvdt, koff + e);
            x->dk[koff + e] += tau * dl * qv[e];
            x->dv[koff + e] += w * p[j] * dO[e];
          }
        }
      }
      /* window terms */
      for (int j = 0; j < nw; ++j) {
        size_t koff = (kvbase + (size_t)(w_lo + j)) * d;
        double u = exp(lw[j] - logZ);
        double dOv = 0;
        for (int e = 0; e < d; ++e) dOv += dO[e] * ld(x->v, x->kvdt, koff + e);
        double dl = u * (dOv - Delta);
        for (int e = 0; e < d; ++e) {
          dq[e] += tau * dl * ld(x->k, x->kvdt, koff + e);
          x->dk[koff + e] += tau * dl * qv[e];
          x->dv[koff + e] += u * dO[e];
        }
      }
      /* q-hat = q + calibration: dq also receives dq-hat */
      for (int e = 0; e < d; ++e) dq[e] += dqh[e];
    }
    /* the chunk summaries of head h (Eq. 8) */
    double *l = lam, *p = P;
    double *kp = ob; /* unrounded k' of the chunk */
    for (int ch = 0; ch < C; ++ch) {
      size_t so = ((size_t)b * c->Hq + h) * C + ch;
      size_t lmo = so * d;
      for (int j = 0; j < S; ++j) {
        size_t koff = (kvbase + (size_t)ch * S + j) * d;
        double acc = 0;
        for (int e = 0; e < d; ++e) acc += ld(x->qlm, x->lmdt, lmo + e) * ld(x->k, x->kvdt, koff + e);
        l[j] = tau * acc;
      }
      double m = l[0];
      for (int j = 1; j < S; ++j) if (l[j] > m) m = l[j];
      double z = 0;
      for (int j = 0; j < S; ++j) z += exp(l[j] - m);
      double El = 0;
      for (int j = 0; j < S; ++j) { p[j] = exp(l[j] - m) / z; El += p[j] * l[j]; }
      for (int e = 0; e < d; ++e) {
        double acc = 0;
        for (int j = 0; j < S; ++j) acc += p[j] * ld(x->k, x->kvdt, (kvbase + (size_t)ch * S + j) * d + e);
        kp[e] = acc;
      }
      const double *dkp = x->dks + so * d;
      double dbp = x->dbs[so];
      for (int j = 0; j < S; ++j) {
        size_t koff = (kvbase + (size_t)ch * S + j) * d;
        double proj = 0;
        for (int e = 0; e < d; ++e) proj += dkp[e] * (ld(x->k, x->kvdt, koff + e) - kp[e]);
        double dl = p[j] * (proj - dbp * (l[j] - El));
        for (int e = 0; e < d; ++e) {
          x->dqlm[lmo + e] += tau * dl * ld(x->k, x->kvdt, koff + e);
          x->dk[koff + e] += p[j] * dkp[e] + tau * dl * ld(x->qlm, x->lmdt, lmo + e);
        }
      }
    }
  }
  free(lam); free(P); free(ob); free(s_hat); free(chunk); free(o); free(dO); free(qv);
}

/* Q-Cal weight gradients: one unit per output row of dW_up (Hq*d rows),
 * then per row of dW_down (r rows), then per token of dh (B*T rows). */
typedef struct {
  const orc_cfg *c; const void *h; int hdt; const void *wd; const void *wu; int wdt;
  const double *u, *du, *dqhat; double *dh, *dwd, *dwu;
} qcal_bwd_ctx;

static void dwu_unit(void *vctx, long row) { /* row = h*d + e */
  qcal_bwd_ctx *x = (qcal_bwd_ctx *)vctx;
  const orc_cfg *c = x->c;
  int d = c->d, hh = (int)(row / d), e = (int)(row % d);
  for (int a = 0; a < c->r; ++a) {
    double acc = 0;
    for (int b = 0; b < c->B; ++b)
      for (int i = 0; i < c->T; ++i)
        acc += x->dqhat[(((size_t)b * c->Hq + hh) * c->T + i) * d + e] * x->u[((size_t)b * c->T + i) * c->r + a];
    x->dwu[(size_t)row * c->r + a] = acc;
  }
}
static void dwd_unit(void *vctx, long a) {
  qcal_bwd_ctx *x = (qcal_bwd_ctx *)vctx;
  const orc_cfg *c = x->c;
  for (int f = 0; f < c->Dh; ++f) {
    double acc = 0;
    for (int b = 0; b < c->B; ++b)
      for (int i = 0; i < c->T; ++i)
        acc += x->du[((size_t)b * c->T + i) * c->r + a] * ld(x->h, x->hdt, ((size_t)b * c->T + i) * c->Dh + f);
    x->dwd[(size_t)a * c->Dh + f] = acc;
  }
}
static void dh_unit(void *vctx, long tok) {
  qcal_bwd_ctx *x = (qcal_bwd_ctx *)vctx;
  const orc_cfg *c = x->c;
  for (int f = 0; f < c->Dh; ++f) {
    double acc = 0;
    for (int a = 0; a < c->r; ++a) acc += x->du[(size_t)tok * c->r + a] * ld(x->wd, x->wdt, (size_t)a * c->Dh + f);
    x->dh[(size_t)tok * c->Dh + f] = acc;
  }
}

int orc_backward(const orc_cfg *c, const void *q, int qdt, const void *k, const void *v, int kvdt,
                 const void *q_lm, int lmdt, const void *h, int hdt, const void *w_down, const void *w_up,
                 int wdt, const int *idx, const void *k_sum, int ksdt, const void *b_sum, int bsdt,
                 const void *dout, int dodt, double *dq, double *dk, double *dv, double *dq_lm, double *dh,
                 double *dw_down, double *dw_up, int nthreads) {
  int d = c->d, C = c->T / c->S;
  size_t nq = (size_t)c->B * c->Hq * c->T * d, nkv = (size_t)c->B * c->Hkv * c->T * d;
  size_t nlm = (size_t)c->B * c->Hq * C * d, ns = (size_t)c->B * c->Hq * C;
  double *qhat = (double *)malloc(sizeof(double) * (nq ? nq : 1));
  double *dqhat = (double *)calloc(nq ? nq : 1, sizeof(double));
  double *dks = (double *)calloc(nlm ? nlm : 1, sizeof(double));
  double *dbs = (double *)calloc(ns ? ns : 1, sizeof(double));
  double *u = 0;
  /* q-hat = q + slice_h(W_up (W_down h_i)) */
  if (c->r > 0) {
    u = (double *)malloc(sizeof(double) * (size_t)c->B * c->T * c->r);
    for (size_t tok = 0; tok < (size_t)c->B * c->T; ++tok)
      for (int a = 0; a < c->r; ++a) {
        double acc = 0;
        for (int f = 0; f < c->Dh; ++f) acc += ld(w_down, wdt, (size_t)a * c->Dh + f) * ld(h, hdt, tok * c->Dh + f);
        u[tok * c->r + a] = acc;
      }
  }
  for (int b = 0; b < c->B; ++b)
    for (int hh = 0; hh < c->Hq; ++hh)
      for (int i = 0; i < c->T; ++i) {
        size_t off = (((size_t)b * c->Hq + hh) * c->T + i) * d;
        for (int e = 0; e < d; ++e) {
          double acc = 0;
          if (c->r > 0)
            for (int a = 0; a < c->r; ++a)
              acc += ld(w_up, wdt, ((size_t)hh * d + e) * c->r + a) * u[((size_t)b * c->T + i) * c->r + a];
          qhat[off + e] = ld(q, qdt, off + e) + acc;
        }
      }
  memset(dq, 0, sizeof(double) * nq);
  memset(dk, 0, sizeof(double) * nkv);
  memset(dv, 0, sizeof(double) * nkv);
  memset(dq_lm, 0, sizeof(double) * nlm);
  bwd_ctx x = {c, q, qdt, k, v, kvdt, q_lm, lmdt, idx, k_sum, ksdt, b_sum, bsdt, dout, dodt,
               qhat, dq, dk, dv, dq_lm, dqhat, dks, dbs};
  parallel_for((long)c->B * c->Hkv, nthreads, bwd_pair_unit, &x);
  if (c->r > 0) {
    double *du = (double *)malloc(sizeof(double) * (size_t)c->B * c->T * c->r);
    for (int b = 0; b < c->B; ++b)
      for (int i = 0; i < c->T; ++i)
        for (int a = 0; a < c->r; ++a) {
          double acc = 0;
          for (int hh = 0; hh < c->Hq; ++hh)
            for (int e = 0; e < d; ++e)
              acc += ld(w_up, wdt, ((size_t)hh * d + e) * c->r + a) * dqhat[(((size_t)b * c->Hq + hh) * c->T + i) * d + e];
          du[((size_t)b * c->T + i) * c->r + a] = acc;
        }
    qcal_bwd_ctx y = {c, h, hdt, w_down, w_up, wdt, u, du, dqhat, dh, dw_down, dw_up};
    parallel_for((long)c->Hq * d, nthreads, dwu_unit, &y);
    parallel_for((long)c->r, nthreads, dwd_unit, &y);
    parallel_for((long)c->B * c->T, nthreads, dh_unit, &y);
    free(du);
    free(u);
  }
  free(qhat); free(dqhat); free(dks); free(dbs);
  return 0;
}
