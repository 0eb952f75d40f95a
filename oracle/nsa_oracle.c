/*
 * nsa_oracle.c -- plain, slow, fp64 CPU reference of the NSA forward pass
 * (compression + selection + sliding window + gates) and of the gradient of
 * the selection branch.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may build, load or call it.  It shares no code, header,
 * table or helper with the HIP library, and nothing here is ever used to
 * compute a product result.
 *
 * Sources (web pages; cited by title and section):
 *   [SIC]  "Sparsity is Cool: Reverse-Engineering MoBA and NSA" (wiki summary
 *          of Tilde Research's blog post), sections Method, Key claims.
 *   [DSA]  "DeepSeek's Native Sparse Attention" (newsletter #44), section
 *          "How Does Native Sparse Attention Work?" (COMPRESSION, SELECTION,
 *          SLIDING WINDOW bullets and the gate paragraph after them).
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 * All arithmetic is in double precision; nothing is rounded to a narrower
 * type.  Every loop runs in the order of the definition (per batch entry,
 * query position, query head, then key), with no blocking or fusion; OpenMP
 * only splits independent (batch, position) rows across host threads.
 *
 * Layouts (row-major, contiguous):
 *   q, out, o_cmp, o_sel, o_win, dq : [B][T][Hq][D]
 *   k, v, dk, dv                    : [B][T][Hkv][D]
 *   gates                           : [B][T][Hq][3]  (cmp, sel, win)
 *   lse_sel, lse_win, lse_cmp       : [B][Hq][T]  (lse_cmp = -inf where no
 *                                     compressed block is visible)
 *   dgates                          : [B][T][Hq][3]
 *   indices                         : [B][Hkv][T][top_k]  ascending, -1 pad
 *   scores (nullable)               : [B][Hkv][T][nblk]   nblk = ceil(T/blk)
 *   gap (nullable)                  : [B][Hkv][T]
 * Query head h belongs to KV group h / (Hq/Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int B, T, Hq, Hkv, D;
  int blk;     /* compression block = selection block (both non-overlapping) */
  int top_k;   /* total selected blocks, forced ones included               */
  int window;  /* sliding-window length W: keys t-W < s <= t                 */
  double scale;/* softmax scale tau                                          */
} oparams;

static size_t qidx(const oparams* p, int b, int t, int h, int d) {
  return (((size_t)b * p->T + t) * p->Hq + h) * p->D + d;
}
static size_t kidx(const oparams* p, int b, int t, int g, int d) {
  return (((size_t)b * p->T + t) * p->Hkv + g) * p->D + d;
}

/* ---- Step 1: compression by mean-pooling ---------------------------------
 * [DSA] COMPRESSION: consecutive tokens of a block are summarised into one key
 * and one value; [SIC] Method: the summary is a mean-pool (no MLP), block 64.
 * Reading: blocks do not overlap (stride = block); only complete blocks exist
 * (j < floor(T/blk)). */
static void pool(const oparams* p, const double* x, double* xc) {
  int nc = p->T / p->blk;
  for (int b = 0; b < p->B; ++b)
    for (int j = 0; j < nc; ++j)
      for (int g = 0; g < p->Hkv; ++g)
        for (int d = 0; d < p->D; ++d) {
          double s = 0.0;
          for (int i = 0; i < p->blk; ++i) s += x[kidx(p, b, j * p->blk + i, g, d)];
          xc[(((size_t)b * nc + j) * p->Hkv + g) * p->D + d] = s / p->blk;
        }
}

int nsa_oracle_pool(int B, int T, int Hkv, int D, int blk, const double* x, double* xc) {
  oparams p = {B, T, Hkv, Hkv, D, blk, 1, 1, 1.0};
  if (B < 1 || T < 1 || Hkv < 1 || D < 1 || blk < 1) return -2;
  pool(&p, x, xc);
  return 0;
}

/* Softmax attention of one query vector over an explicit list of keys.
 * Writes o = sum_s softmax(tau q.k_s) v_s and returns lse = log sum exp. */
static double attend(const oparams* p, const double* qv, const double* k, const double* v,
                     int b, int g, const int* keys, int nkeys, double* o, double* logit) {
  int D = p->D;
  double m = -INFINITY;
  for (int i = 0; i < nkeys; ++i) {
    double s = 0.0;
    const double* kv = k + kidx(p, b, keys[i], g, 0);
    for (int d = 0; d < D; ++d) s += qv[d] * kv[d];
    logit[i] = p->scale * s;
    if (logit[i] > m) m = logit[i];
  }
  double l = 0.0;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int i = 0; i < nkeys; ++i) {
    double e = exp(logit[i] - m);
    l += e;
    const double* vv = v + kidx(p, b, keys[i], g, 0);
    for (int d = 0; d < D; ++d) o[d] += e * vv[d];
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  return m + log(l);
}

typedef struct { double s; int j; } cand;
/* Order for block selection: higher importance first, lower index on ties. */
static int cand_cmp(const void* a, const void* b) {
  const cand* x = (const cand*)a;
  const cand* y = (const cand*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}
static int int_cmp(const void* a, const void* b) {
  int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

/* Selected block set I(t, g) from the importance scores S[j] (j < n_c(t)).
 * [DSA] SELECTION: blocks are ranked by reusing the compression-branch
 * attention scores; [SIC] Method: block 64, top-k 16; [SIC] Key claims: the
 * first block is always included.
 * Readings: forced set F = {0, own block}; k counts F; candidates are the
 * earlier complete blocks 1..own-1; ties go to the lower block index; with at
 * most k-|F| candidates, all of them are taken.  Output ascending, -1 padded.
 * Returns the number of valid entries; *gap receives S_(m) - S_(m+1) over the
 * candidates (INFINITY when every candidate is taken). */
static int select_blocks(const oparams* p, int t, const double* S, int* out, double* gap,
                         cand* buf) {
  int own = t / p->blk;
  int n = 0;
  out[n++] = 0;
  if (own != 0) out[n++] = own;
  int m = p->top_k - n;
  int ncand = own > 1 ? own - 1 : 0;
  if (ncand <= m) {
    for (int j = 1; j < own; ++j) out[n++] = j;
    *gap = INFINITY;
  } else {
    for (int j = 1; j < own; ++j) { buf[j - 1].s = S[j]; buf[j - 1].j = j; }
    qsort(buf, (size_t)ncand, sizeof(cand), cand_cmp);
    for (int i = 0; i < m; ++i) out[n++] = buf[i].j;
    *gap = (m > 0 ? buf[m - 1].s : INFINITY) - buf[m].s;
  }
  qsort(out, (size_t)n, sizeof(int), int_cmp);
  for (int i = n; i < p->top_k; ++i) out[i] = -1;
  return n;
}

/* ---- Full forward ---------------------------------------------------------
 * indices: if indices_in != 0 the given table is used instead of Step 4
 * (the oracle's own earlier table, e.g. to freeze the selection).
 * rows/nrows: if rows != NULL only those query positions are computed (the
 * pooled blocks are still built from the whole sequence); other rows of the
 * outputs are left untouched. */
int nsa_oracle_forward(int B, int T, int Hq, int Hkv, int D, int blk, int top_k, int window,
                       double scale, const double* q, const double* k, const double* v,
                       const double* gates, double* out, double* o_cmp, double* o_sel,
                       double* o_win, double* lse_sel, double* lse_win, double* lse_cmp,
                       int32_t* indices, int indices_in, double* scores, double* gap,
                       const int32_t* rows, int nrows, int nthreads) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || blk < 1 || Hq % Hkv) return -2;
  if (top_k < 2 || window < 1) return -2;
  oparams p = {B, T, Hq, Hkv, D, blk, top_k, window, scale};
  int G = Hq / Hkv;
  int nc_all = T / blk;
  int nblk = (T + blk - 1) / blk;
  double* kc = (double*)malloc(sizeof(double) * (size_t)B * (nc_all ? nc_all : 1) * Hkv * D);
  double* vc = (double*)malloc(sizeof(double) * (size_t)B * (nc_all ? nc_all : 1) * Hkv * D);
  if (!kc || !vc) { free(kc); free(vc); return -1; }
  pool(&p, k, kc);
  pool(&p, v, vc);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)(nblk + 1));
    double* pr = (double*)malloc(sizeof(double) * (size_t)G * (nc_all + 1));
    double* logit = (double*)malloc(sizeof(double) * (size_t)T);
    int* keys = (int*)malloc(sizeof(int) * (size_t)T);
    int* wkeys = (int*)malloc(sizeof(int) * (size_t)T);
    int* sel = (int*)malloc(sizeof(int) * (size_t)top_k);
    cand* buf = (cand*)malloc(sizeof(cand) * (size_t)(nblk + 1));
    double* oc = (double*)malloc(sizeof(double) * (size_t)D);
    double* os = (double*)malloc(sizeof(double) * (size_t)D);
    double* ow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!S || !pr || !logit || !keys || !wkeys || !sel || !buf || !oc || !os || !ow) {
#pragma omp atomic write
      err = 1;
    } else {
      /* rows (optional): only these query positions are computed. */
      int nt = rows ? nrows : T;
#pragma omp for schedule(dynamic, 16) collapse(2)
      for (int b = 0; b < B; ++b)
        for (int ti = 0; ti < nt; ++ti)
          for (int g = 0; g < Hkv; ++g) {
            int t = rows ? rows[ti] : ti;
            if (t < 0 || t >= T) continue;
            int ncv = (t + 1) / blk; /* complete blocks visible to t (reading) */
            /* Step 2: compressed attention per head; Step 3: importance.   */
            for (int j = 0; j <= nblk; ++j) S[j] = 0.0;
            for (int hh = 0; hh < G; ++hh) {
              int h = g * G + hh;
              const double* qv = q + qidx(&p, b, t, h, 0);
              double* prh = pr + (size_t)hh * (nc_all + 1);
              for (int d = 0; d < D; ++d) oc[d] = 0.0;
              if (ncv > 0) {
                double m = -INFINITY;
                for (int j = 0; j < ncv; ++j) {
                  const double* kcj = kc + (((size_t)b * nc_all + j) * Hkv + g) * D;
                  double s = 0.0;
                  for (int d = 0; d < D; ++d) s += qv[d] * kcj[d];
                  prh[j] = scale * s;
                  if (prh[j] > m) m = prh[j];
                }
                double l = 0.0;
                for (int j = 0; j < ncv; ++j) { prh[j] = exp(prh[j] - m); l += prh[j]; }
                if (lse_cmp) lse_cmp[((size_t)b * Hq + h) * T + t] = m + log(l);
                for (int j = 0; j < ncv; ++j) {
                  prh[j] /= l;
                  const double* vcj = vc + (((size_t)b * nc_all + j) * Hkv + g) * D;
                  for (int d = 0; d < D; ++d) oc[d] += prh[j] * vcj[d];
                  S[j] += prh[j];
                }
              }
              if (lse_cmp && ncv == 0) lse_cmp[((size_t)b * Hq + h) * T + t] = -INFINITY;
              if (o_cmp)
                for (int d = 0; d < D; ++d) o_cmp[qidx(&p, b, t, h, d)] = oc[d];
              if (out)
                for (int d = 0; d < D; ++d)
                  out[qidx(&p, b, t, h, d)] = gates[(((size_t)b * T + t) * Hq + h) * 3 + 0] * oc[d];
            }
            if (scores)
              for (int j = 0; j < nblk; ++j)
                scores[(((size_t)b * Hkv + g) * T + t) * nblk + j] = j < ncv ? S[j] : 0.0;
            /* Step 4: block selection. */
            int32_t* irow = indices + (((size_t)b * Hkv + g) * T + t) * top_k;
            int nsel;
            double gp = INFINITY;
            if (indices_in) {
              nsel = 0;
              for (int i = 0; i < top_k; ++i) {
                sel[i] = irow[i];
                if (irow[i] >= 0) ++nsel;
              }
            } else {
              nsel = select_blocks(&p, t, S, sel, &gp, buf);
              for (int i = 0; i < top_k; ++i) irow[i] = sel[i];
            }
            if (gap) gap[((size_t)b * Hkv + g) * T + t] = gp;
            /* Step 5: selection attention over the original tokens of the
             * selected blocks, one joint softmax, causal (s <= t). */
            int nk = 0;
            for (int i = 0; i < nsel; ++i)
              for (int s = sel[i] * blk; s < (sel[i] + 1) * blk && s <= t && s < T; ++s)
                keys[nk++] = s;
            /* Step 6 keys: the window t-W < s <= t. */
            int w0 = t - window + 1 > 0 ? t - window + 1 : 0;
            for (int hh = 0; hh < G; ++hh) {
              int h = g * G + hh;
              const double* qv = q + qidx(&p, b, t, h, 0);
              double lse = attend(&p, qv, k, v, b, g, keys, nk, os, logit);
              if (lse_sel) lse_sel[((size_t)b * Hq + h) * T + t] = lse;
              int nw = 0;
              for (int s = w0; s <= t; ++s) wkeys[nw++] = s;
              double lsw = attend(&p, qv, k, v, b, g, wkeys, nw, ow, logit);
              if (lse_win) lse_win[((size_t)b * Hq + h) * T + t] = lsw;
              if (o_sel)
                for (int d = 0; d < D; ++d) o_sel[qidx(&p, b, t, h, d)] = os[d];
              if (o_win)
                for (int d = 0; d < D; ++d) o_win[qidx(&p, b, t, h, d)] = ow[d];
              /* Step 7: gated combination. [DSA]: the branch outputs are mixed
               * by learned gates; the gate values are inputs here. */
              if (out) {
                const double* gt = gates + (((size_t)b * T + t) * Hq + h) * 3;
                for (int d = 0; d < D; ++d)
                  out[qidx(&p, b, t, h, d)] += gt[1] * os[d] + gt[2] * ow[d];
              }
            }
          }
    }
    free(S); free(pr); free(logit); free(keys); free(wkeys); free(sel); free(buf); free(oc); free(os); free(ow);
  }
  free(kc);
  free(vc);
  return err ? -1 : 0;
}

/* ---- Gradient of the selection branch --------------------------------------
 * The selected blocks and the gates are held fixed.  dout is the gradient of
 * the combined output; the selection branch receives g_sel * dout.  With
 * P_s = exp(tau q.k_s - lse), dP_s = dO_s . v_s, Delta = dO_s . o_sel and
 * dS_s = P_s (dP_s - Delta) (softmax Jacobian):
 *   dq   = tau sum_s dS_s k_s
 *   dk_s += tau dS_s q,   dv_s += P_s dO_s     (summed over the group's heads)
 * [SIC] Method describes the kernel problem (each query has its own key
 * subset); this is the plain definition, scattered in query order. */
int nsa_oracle_select_bwd(int B, int T, int Hq, int Hkv, int D, int blk, int top_k,
                          double scale, const double* q, const double* k, const double* v,
                          const double* gates, const int32_t* indices, const double* dout,
                          double* dq, double* dk, double* dv, int nthreads) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || blk < 1 || Hq % Hkv) return -2;
  oparams p = {B, T, Hq, Hkv, D, blk, top_k, 1, scale};
  int G = Hq / Hkv;
  memset(dk, 0, sizeof(double) * (size_t)B * T * Hkv * D);
  memset(dv, 0, sizeof(double) * (size_t)B * T * Hkv * D);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
  /* (b, g) pairs own disjoint dk/dv rows, so they may run in parallel; inside
   * one pair the scatter runs in query order. */
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      int* keys = (int*)malloc(sizeof(int) * (size_t)T);
      double* logit = (double*)malloc(sizeof(double) * (size_t)T);
      double* os = (double*)malloc(sizeof(double) * (size_t)D);
      double* dos = (double*)malloc(sizeof(double) * (size_t)D);
      if (!keys || !logit || !os || !dos) {
#pragma omp atomic write
        err = 1;
      } else {
        for (int t = 0; t < T; ++t) {
          const int32_t* irow = indices + (((size_t)b * Hkv + g) * T + t) * top_k;
          int nk = 0;
          for (int i = 0; i < top_k; ++i) {
            int j = irow[i];
            if (j < 0) continue;
            for (int s = j * blk; s < (j + 1) * blk && s <= t && s < T; ++s) keys[nk++] = s;
          }
          for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            const double* qv = q + qidx(&p, b, t, h, 0);
            double lse = attend(&p, qv, k, v, b, g, keys, nk, os, logit);
            double gs = gates[(((size_t)b * T + t) * Hq + h) * 3 + 1];
            double delta = 0.0;
            for (int d = 0; d < D; ++d) {
              dos[d] = gs * dout[qidx(&p, b, t, h, d)];
              delta += dos[d] * os[d];
            }
            double* dqv = dq + qidx(&p, b, t, h, 0);
            for (int d = 0; d < D; ++d) dqv[d] = 0.0;
            for (int i = 0; i < nk; ++i) {
              const double* kv = k + kidx(&p, b, keys[i], g, 0);
              const double* vv = v + kidx(&p, b, keys[i], g, 0);
              double P = exp(logit[i] - lse);
              double dP = 0.0;
              for (int d = 0; d < D; ++d) dP += dos[d] * vv[d];
              double dS = P * (dP - delta);
              double* dkv = dk + kidx(&p, b, keys[i], g, 0);
              double* dvv = dv + kidx(&p, b, keys[i], g, 0);
              for (int d = 0; d < D; ++d) {
                dqv[d] += scale * dS * kv[d];
                dkv[d] += scale * dS * qv[d];
                dvv[d] += P * dos[d];
              }
            }
          }
        }
      }
      free(keys); free(logit); free(os); free(dos);
    }
  return err ? -1 : 0;
}

/* ---- Gradient of all three branches and of the gates ------------------------
 * The selected blocks are held fixed (top-k is piecewise constant, so no
 * gradient flows through the importance scores).  out = g_c o_cmp + g_s o_sel
 * + g_w o_win, so
 *   dgates[t,h] = (dout . o_cmp, dout . o_sel, dout . o_win)
 * and each branch receives g_branch * dout.  Every branch is a softmax
 * attention, so its gradient is the softmax Jacobian written out as in
 * nsa_oracle_select_bwd, over its own keys:
 *   selection : the tokens s <= t of the selected blocks;
 *   window    : t - W < s <= t;
 *   compression: the pooled keys Kc_j, Vc_j of the complete blocks with
 *               64 (j + 1) - 1 <= t; their gradients dKc_j, dVc_j flow back
 *               through the mean-pool as dk_s += dKc_j / blk, dv_s += dVc_j /
 *               blk for the blk tokens s of block j ([DSA] COMPRESSION; [SIC]
 *               Method: the pool is a plain mean).
 * Scattered in query order, per (batch, KV group). */
static void softmax_bwd(const oparams* p, int b, int g, const double* qv, const double* k,
                        const double* v, const int* keys, int nkeys, const double* dob,
                        double* dqv, double* dk, double* dv, double* logit, double* ob) {
  int D = p->D;
  double lse = attend(p, qv, k, v, b, g, keys, nkeys, ob, logit);
  double delta = 0.0;
  for (int d = 0; d < D; ++d) delta += dob[d] * ob[d];
  for (int i = 0; i < nkeys; ++i) {
    const double* kv = k + kidx(p, b, keys[i], g, 0);
    const double* vv = v + kidx(p, b, keys[i], g, 0);
    double P = exp(logit[i] - lse);
    double dP = 0.0;
    for (int d = 0; d < D; ++d) dP += dob[d] * vv[d];
    double dS = P * (dP - delta);
    double* dkv = dk + kidx(p, b, keys[i], g, 0);
    double* dvv = dv + kidx(p, b, keys[i], g, 0);
    for (int d = 0; d < D; ++d) {
      dqv[d] += p->scale * dS * kv[d];
      dkv[d] += p->scale * dS * qv[d];
      dvv[d] += P * dob[d];
    }
  }
}

int nsa_oracle_backward(int B, int T, int Hq, int Hkv, int D, int blk, int top_k, int window,
                        double scale, const double* q, const double* k, const double* v,
                        const double* gates, const int32_t* indices, const double* dout,
                        double* dq, double* dk, double* dv, double* dgates, int nthreads) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || blk < 1 || Hq % Hkv) return -2;
  if (top_k < 1 || window < 1) return -2;
  oparams p = {B, T, Hq, Hkv, D, blk, top_k, window, scale};
  int G = Hq / Hkv;
  int nc = T / blk;
  /* pooled keys / values as [B][nc][Hkv][D]: the layout of k with T -> nc */
  oparams pc = p;
  pc.T = nc > 0 ? nc : 1;
  double* kc = (double*)calloc((size_t)B * pc.T * Hkv * D, sizeof(double));
  double* vc = (double*)calloc((size_t)B * pc.T * Hkv * D, sizeof(double));
  double* dkc = (double*)calloc((size_t)B * pc.T * Hkv * D, sizeof(double));
  double* dvc = (double*)calloc((size_t)B * pc.T * Hkv * D, sizeof(double));
  if (!kc || !vc || !dkc || !dvc) { free(kc); free(vc); free(dkc); free(dvc); return -1; }
  if (nc > 0) { pool(&p, k, kc); pool(&p, v, vc); }
  memset(dq, 0, sizeof(double) * (size_t)B * T * Hq * D);
  memset(dk, 0, sizeof(double) * (size_t)B * T * Hkv * D);
  memset(dv, 0, sizeof(double) * (size_t)B * T * Hkv * D);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      int* keys = (int*)malloc(sizeof(int) * (size_t)(T + 1));
      double* logit = (double*)malloc(sizeof(double) * (size_t)(T + 1));
      double* ob = (double*)malloc(sizeof(double) * (size_t)D);
      double* dob = (double*)malloc(sizeof(double) * (size_t)D);
      if (!keys || !logit || !ob || !dob) {
#pragma omp atomic write
        err = 1;
      } else {
        for (int t = 0; t < T; ++t) {
          const int32_t* irow = indices + (((size_t)b * Hkv + g) * T + t) * top_k;
          for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            const double* qv = q + qidx(&p, b, t, h, 0);
            const double* dov = dout + qidx(&p, b, t, h, 0);
            const double* gt = gates + (((size_t)b * T + t) * Hq + h) * 3;
            double* dqv = dq + qidx(&p, b, t, h, 0);
            double* dg = dgates + (((size_t)b * T + t) * Hq + h) * 3;
            /* compression: pooled keys j with 64 (j + 1) - 1 <= t */
            int ncv = (t + 1) / blk;
            for (int j = 0; j < ncv; ++j) keys[j] = j;
            for (int d = 0; d < D; ++d) dob[d] = gt[0] * dov[d];
            if (ncv > 0) {
              softmax_bwd(&pc, b, g, qv, kc, vc, keys, ncv, dob, dqv, dkc, dvc, logit, ob);
            } else {
              for (int d = 0; d < D; ++d) ob[d] = 0.0;
            }
            double s0 = 0.0;
            for (int d = 0; d < D; ++d) s0 += dov[d] * ob[d];
            dg[0] = s0;
            /* selection */
            int nk = 0;
            for (int i = 0; i < top_k; ++i) {
              int j = irow[i];
              if (j < 0) continue;
              for (int s = j * blk; s < (j + 1) * blk && s <= t && s < T; ++s) keys[nk++] = s;
            }
            for (int d = 0; d < D; ++d) dob[d] = gt[1] * dov[d];
            softmax_bwd(&p, b, g, qv, k, v, keys, nk, dob, dqv, dk, dv, logit, ob);
            double s1 = 0.0;
            for (int d = 0; d < D; ++d) s1 += dov[d] * ob[d];
            dg[1] = s1;
            /* window */
            int nw = 0;
            for (int s = t - window + 1 > 0 ? t - window + 1 : 0; s <= t; ++s) keys[nw++] = s;
            for (int d = 0; d < D; ++d) dob[d] = gt[2] * dov[d];
            softmax_bwd(&p, b, g, qv, k, v, keys, nw, dob, dqv, dk, dv, logit, ob);
            double s2 = 0.0;
            for (int d = 0; d < D; ++d) s2 += dov[d] * ob[d];
            dg[2] = s2;
          }
        }
        /* the mean-pool's gradient: every token of block j gets dKc_j / blk */
        for (int j = 0; j < nc; ++j)
          for (int i = 0; i < blk; ++i)
            for (int d = 0; d < D; ++d) {
              dk[kidx(&p, b, j * blk + i, g, d)] += dkc[kidx(&pc, b, j, g, d)] / blk;
              dv[kidx(&p, b, j * blk + i, g, d)] += dvc[kidx(&pc, b, j, g, d)] / blk;
            }
      }
      free(keys); free(logit); free(ob); free(dob);
    }
  free(kc); free(vc); free(dkc); free(dvc);
  return err ? -1 : 0;
}
