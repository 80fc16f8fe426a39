/*
 * HSTU pointwise attention: CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file; it exists so that tests, the smoke check and the CPU baseline
 * timing of the benchmark have a plain, obviously correct fp64 definition to
 * compare the HIP kernels against. It shares no code, header or constant with
 * the HIP library.
 *
 * What it computes (sources: the HSTU blog page "Meta HSTU: 生成式推荐系统的实践",
 * section 3 "HSTU 架构" (the layer formula), 3.1 "Pointwise Attention" (phi2 is
 * SiLU, no softmax), 3.2 "Relative Attention Bias" (position and time biases),
 * 4.2/4.3 (M-FALCON candidate mask and history K/V caching); the MTGR pages
 * "MTGR：美团外卖生成式推荐..." section 2 "方法详解" (Group LayerNorm, dynamic
 * hybrid mask) and the fmread.com MTGR report, section 三.1 "动态掩码策略"):
 *
 *   per sequence b, head h, local rows i and keys j in [0, L):
 *     s_ij = <q_i, k_j> + rab_p[min(|pos(i)-pos(j)|, n_pos-1)]
 *                       + rab_t[bucket(t_i - t_j)]
 *     a_ij = vis(i,j) ? SiLU(s_ij) / n_max : 0
 *     o_i  = sum_j a_ij v_j                        (ascending j)
 *   per token: x = concat_h o_i^h, n = Norm(x), y = n * u.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - vis: rows in the prefix [0,P) see keys [0,P); rows in [P,E) see j <= i;
 *     candidate rows [E,L) (E = L - C) see j < E and themselves.
 *   - pos(i) = i for i < E, and every candidate sits at position E.
 *   - bucket(dt) = min(n_tb-1, floor(log2(max(1,|dt|)))), dt in int64 seconds.
 *   - Norm is over the full width D = H*d of a token; LN uses the population
 *     variance and eps; GLN indexes the affine (gamma, beta) by token group.
 *   - rab tables are shared by all heads; a NULL table (or NULL timestamps)
 *     turns its term off.
 *
 * Pins (tests under tests/ marked "not gpu"): closed form for L = 1, library
 * routines (torch matmul / silu / layer_norm / tril) for the dense special
 * cases, bit patterns of the attention matrix read out with Q = 0 and one-hot
 * V, the exact invariants (Q = 0, masked-pair perturbation, candidate
 * permutation, microbatching, cached K/V), hand-written mask fixtures, integer
 * bucket boundaries, and for the backward: torch autograd of a dense
 * formulation plus central finite differences of oracle_fwd itself.
 *
 * All arithmetic is fp64; inputs arrive as fp64 arrays (bf16 and fp32 decode
 * exactly into fp64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { NORM_NONE = 0, NORM_LN = 1, NORM_GLN = 2 };

/* floor(log2(x)) for x >= 1, by repeated halving. */
static int floor_log2_u64(uint64_t x) {
  int n = 0;
  while (x > 1) {
    x >>= 1;
    n++;
  }
  return n;
}

int oracle_time_bucket(int64_t dt, int n_tb) {
  uint64_t a = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
  if (a < 1) a = 1;
  int b = floor_log2_u64(a);
  return b < n_tb - 1 ? b : n_tb - 1;
}

int oracle_classify_tiles_tf(int L, int P, int C, int r0, int nrows, int BN, int nkt,
                             int time_filter, int8_t *kind);

/* Visibility of key j from row i inside one sequence of length L with a
 * bidirectional prefix of P tokens and a candidate tail of C tokens. */
int oracle_visible(int i, int j, int L, int P, int C) {
  int E = L - C;
  if (j < 0 || j >= L || i < 0 || i >= L) return 0;
  if (i < P) return j < P;
  if (i < E) return j <= i;
  return j < E || j == i;
}

/* The same with MTGR's timestamp filter for candidates (MTGR deep read,
 * section 2: exposure samples are filtered by timestamp to stay causal): when
 * time_filter is set, a candidate row i (i >= E) sees a key j of the causal
 * segment [P, E) only if t_j < t_i; everything else is as above. */
static int visible_t(int i, int j, int L, int P, int C, const int64_t *ts, int time_filter) {
  int v = oracle_visible(i, j, L, P, C);
  int E = L - C;
  if (v && time_filter && i >= E && j >= P && j < E) return ts[j] < ts[i];
  return v;
}

static int position_of(int i, int E) { return i < E ? i : E; }

static double silu(double x) { return x / (1.0 + exp(-x)); }

/* The logit of pair (i, j) of one head of one sequence frame. */
typedef struct {
  int L, P, C, d;
  const double *q; long q_stride;  /* rows of the frame (row i at q + i*q_stride) */
  const double *k; long k_stride;
  const double *v; long v_stride;
  const int64_t *ts;               /* frame timestamps or NULL */
  const double *rab_p; int n_pos;
  const double *rab_t; int n_tb;
  double inv_nmax;
  int time_filter;                 /* candidates see causal keys only if earlier (needs ts) */
} frame_t;

static double logit(const frame_t *f, int i, int j, int *pidx, int *tidx) {
  const double *qi = f->q + (long)i * f->q_stride;
  const double *kj = f->k + (long)j * f->k_stride;
  double s = 0.0;
  for (int c = 0; c < f->d; c++) s += qi[c] * kj[c];
  int E = f->L - f->C;
  *pidx = -1;
  *tidx = -1;
  if (f->rab_p) {
    int dp = position_of(i, E) - position_of(j, E);
    if (dp < 0) dp = -dp;
    int idx = dp < f->n_pos - 1 ? dp : f->n_pos - 1;
    s += f->rab_p[idx];
    *pidx = idx;
  }
  if (f->rab_t && f->ts) {
    int idx = oracle_time_bucket(f->ts[i] - f->ts[j], f->n_tb);
    s += f->rab_t[idx];
    *tidx = idx;
  }
  return s;
}

/* o_i = sum over visible j (ascending) of SiLU(s_ij)/n_max * v_j. */
static void attend_row(const frame_t *f, int i, double *out) {
  for (int c = 0; c < f->d; c++) out[c] = 0.0;
  for (int j = 0; j < f->L; j++) {
    if (!visible_t(i, j, f->L, f->P, f->C, f->ts, f->time_filter)) continue;
    int pi, ti;
    double a = silu(logit(f, i, j, &pi, &ti)) * f->inv_nmax;
    const double *vj = f->v + (long)j * f->v_stride;
    for (int c = 0; c < f->d; c++) out[c] += a * vj[c];
  }
}

/* Norm(x) * u for one token of width D. Writes y, and the statistics. */
static void norm_token(int mode, int D, const double *x, const double *u, double eps,
                       const double *gamma, const double *beta, double *y,
                       double *mean_out, double *rstd_out) {
  if (mode == NORM_NONE) {
    for (int c = 0; c < D; c++) y[c] = x[c] * u[c];
    *mean_out = 0.0;
    *rstd_out = 1.0;
    return;
  }
  double mu = 0.0;
  for (int c = 0; c < D; c++) mu += x[c];
  mu /= D;
  double var = 0.0;
  for (int c = 0; c < D; c++) var += (x[c] - mu) * (x[c] - mu);
  var /= D;
  double rstd = 1.0 / sqrt(var + eps);
  for (int c = 0; c < D; c++) {
    double n = (x[c] - mu) * rstd;
    if (gamma) n *= gamma[c];
    if (beta) n += beta[c];
    y[c] = n * u[c];
  }
  *mean_out = mu;
  *rstd_out = rstd;
}

static int check_common(int B, int H, int d, const int32_t *offsets, const int32_t *prefix_len,
                        const int32_t *cand_len) {
  if (B < 0 || H <= 0 || d <= 0 || !offsets) return 1;
  if (offsets[0] != 0) return 2;
  for (int b = 0; b < B; b++) {
    int L = offsets[b + 1] - offsets[b];
    if (L < 0) return 3;
    int P = prefix_len ? prefix_len[b] : 0, C = cand_len ? cand_len[b] : 0;
    if (P < 0 || C < 0 || P + C > L) return 4;
  }
  return 0;
}

/*
 * Forward. Layouts: Q, K, V, U are [T, H, d] (token-major, U read as [T, D]);
 * Y and O are [T, D] with D = H*d; mean, rstd are [T]. row_sel (or NULL)
 * restricts the computation to tokens whose flag is nonzero; other rows of
 * Y/O/mean/rstd are left untouched. group[T] picks the affine row for GLN.
 * Returns 0 on success, nonzero on invalid input.
 */
int oracle_fwd(int B, int H, int d, const int32_t *offsets, const int32_t *prefix_len,
               const int32_t *cand_len, const double *Q, const double *K, const double *V,
               const double *U, const int64_t *ts, const double *rab_p, int n_pos,
               const double *rab_t, int n_tb, double n_max, int norm, double eps,
               const uint8_t *group, int n_groups, const double *gamma, const double *beta,
               const uint8_t *row_sel, double *Y, double *O, double *mean, double *rstd,
               int time_filter, int nthreads) {
  int err = check_common(B, H, d, offsets, prefix_len, cand_len);
  if (err) return err;
  if (n_max <= 0) return 5;
  if (time_filter && !ts) return 9;
  if (norm == NORM_GLN && (!group || n_groups <= 0)) return 6;
  const int D = H * d;
  const long T = offsets[B];
  if (norm == NORM_GLN)
    for (long t = 0; t < T; t++)
      if (group[t] >= n_groups) return 8;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < (long)B * H; bh++) {
    int b = (int)(bh / H), h = (int)(bh % H);
    long base = offsets[b];
    frame_t f;
    f.L = offsets[b + 1] - offsets[b];
    f.P = prefix_len ? prefix_len[b] : 0;
    f.C = cand_len ? cand_len[b] : 0;
    f.d = d;
    f.q = Q + (base * H + h) * d; f.q_stride = (long)H * d;
    f.k = K + (base * H + h) * d; f.k_stride = (long)H * d;
    f.v = V + (base * H + h) * d; f.v_stride = (long)H * d;
    f.ts = ts ? ts + base : NULL;
    f.rab_p = rab_p; f.n_pos = n_pos;
    f.rab_t = rab_t; f.n_tb = n_tb;
    f.inv_nmax = 1.0 / n_max;
    f.time_filter = time_filter;
    for (int i = 0; i < f.L; i++) {
      if (row_sel && !row_sel[base + i]) continue;
      attend_row(&f, i, O + (base + i) * D + (long)h * d);
    }
  }
#pragma omp parallel for schedule(static)
  for (long t = 0; t < T; t++) {
    if (row_sel && !row_sel[t]) continue;
    int g = (norm == NORM_GLN) ? group[t] : 0;
    norm_token(norm, D, O + t * D, U + t * D, eps, gamma ? gamma + (long)g * D : NULL,
               beta ? beta + (long)g * D : NULL, Y + t * D, mean + t, rstd + t);
  }
  return 0;
}

/*
 * Backward of oracle_fwd with respect to Q, K, V, U, the rab tables and the
 * affine parameters, given dY [T, D]. The forward is recomputed internally.
 * drab_p_abs / drab_t_abs (or NULL) receive the sums of |dS| that enter each
 * table entry.
 * Every gradient output is overwritten. dgamma/dbeta ([n_groups, D]) may be
 * NULL; they are only produced when gamma/beta are given. Timestamps have no
 * gradient.
 */
int oracle_bwd(int B, int H, int d, const int32_t *offsets, const int32_t *prefix_len,
               const int32_t *cand_len, const double *Q, const double *K, const double *V,
               const double *U, const int64_t *ts, const double *rab_p, int n_pos,
               const double *rab_t, int n_tb, double n_max, int norm, double eps,
               const uint8_t *group, int n_groups, const double *gamma, const double *beta,
               const double *dY, double *dQ, double *dK, double *dV, double *dU,
               double *drab_p, double *drab_t, double *dgamma, double *dbeta,
               double *drab_p_abs, double *drab_t_abs, int time_filter, int nthreads) {
  int err = check_common(B, H, d, offsets, prefix_len, cand_len);
  if (err) return err;
  if (time_filter && !ts) return 9;
  const int D = H * d;
  const long T = offsets[B];
  const int G = (norm == NORM_GLN) ? n_groups : 1;
  double *O = (double *)calloc((size_t)T * D + 1, sizeof(double));
  double *Yt = (double *)calloc((size_t)T * D + 1, sizeof(double));
  double *mean = (double *)calloc((size_t)T + 1, sizeof(double));
  double *rstd = (double *)calloc((size_t)T + 1, sizeof(double));
  double *dO = (double *)calloc((size_t)T * D + 1, sizeof(double));
  if (!O || !Yt || !mean || !rstd || !dO) {
    free(O); free(Yt); free(mean); free(rstd); free(dO);
    return 7;
  }
  err = oracle_fwd(B, H, d, offsets, prefix_len, cand_len, Q, K, V, U, ts, rab_p, n_pos, rab_t,
                   n_tb, n_max, norm, eps, group, n_groups, gamma, beta, NULL, Yt, O, mean, rstd,
                   time_filter, nthreads);
  if (err) {
    free(O); free(Yt); free(mean); free(rstd); free(dO);
    return err;
  }
  int nth = 1;
#ifdef _OPENMP
  nth = omp_get_max_threads();
#endif
  /* Per-thread partial sums for the parameters shared across tokens. */
  double *pg = (double *)calloc((size_t)nth * G * D + 1, sizeof(double));
  double *pb = (double *)calloc((size_t)nth * G * D + 1, sizeof(double));
  double *pp = (double *)calloc((size_t)nth * (n_pos > 0 ? n_pos : 1), sizeof(double));
  double *pt = (double *)calloc((size_t)nth * (n_tb > 0 ? n_tb : 1), sizeof(double));
  /* sums of |dS| per table entry: the scale against which the cancelling
   * sums drab_p / drab_t are measured */
  double *ppa = (double *)calloc((size_t)nth * (n_pos > 0 ? n_pos : 1), sizeof(double));
  double *pta = (double *)calloc((size_t)nth * (n_tb > 0 ? n_tb : 1), sizeof(double));

  /* Norm backward, per token:
   *   dU = n * dY,  dN = dY * u
   *   LN: xhat = (x - mu) * rstd, g = dN * gamma,
   *       dx = rstd * (g - mean(g) - xhat * mean(g * xhat)),
   *       dgamma += dN * xhat, dbeta += dN.   NONE: dx = dN. */
#pragma omp parallel
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double *ghat = (double *)malloc(sizeof(double) * D);
    double *xhat = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(static)
    for (long t = 0; t < T; t++) {
      const double *x = O + t * D, *u = U + t * D, *dy = dY + t * D;
      int g = (norm == NORM_GLN) ? group[t] : 0;
      const double *gm = gamma ? gamma + (long)g * D : NULL;
      const double *bt = beta ? beta + (long)g * D : NULL;
      if (norm == NORM_NONE) {
        for (int c = 0; c < D; c++) {
          dU[t * D + c] = x[c] * dy[c];
          dO[t * D + c] = dy[c] * u[c];
        }
        continue;
      }
      double m1 = 0.0, m2 = 0.0;
      for (int c = 0; c < D; c++) {
        xhat[c] = (x[c] - mean[t]) * rstd[t];
        double nval = xhat[c] * (gm ? gm[c] : 1.0) + (bt ? bt[c] : 0.0);
        dU[t * D + c] = nval * dy[c];
        double dn = dy[c] * u[c];
        if (gamma) pg[((long)tid * G + g) * D + c] += dn * xhat[c];
        if (beta) pb[((long)tid * G + g) * D + c] += dn;
        ghat[c] = dn * (gm ? gm[c] : 1.0);
        m1 += ghat[c];
        m2 += ghat[c] * xhat[c];
      }
      m1 /= D;
      m2 /= D;
      for (int c = 0; c < D; c++) dO[t * D + c] = rstd[t] * (ghat[c] - m1 - xhat[c] * m2);
    }
    free(ghat);
    free(xhat);
  }

  /* Attention backward, per (sequence, head); each owns its rows of dQ/dK/dV:
   *   dA_ij = <dO_i, v_j>, dS_ij = dA_ij * SiLU'(s_ij) / n_max over visible pairs,
   *   dV_j += a_ij dO_i, dQ_i += dS_ij k_j, dK_j += dS_ij q_i,
   *   drab_p[idx] += dS_ij, drab_t[bucket] += dS_ij. */
  memset(dQ, 0, sizeof(double) * T * D);
  memset(dK, 0, sizeof(double) * T * D);
  memset(dV, 0, sizeof(double) * T * D);
#pragma omp parallel
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
#pragma omp for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)B * H; bh++) {
      int b = (int)(bh / H), h = (int)(bh % H);
      long base = offsets[b];
      frame_t f;
      f.L = offsets[b + 1] - offsets[b];
      f.P = prefix_len ? prefix_len[b] : 0;
      f.C = cand_len ? cand_len[b] : 0;
      f.d = d;
      f.q = Q + (base * H + h) * d; f.q_stride = D;
      f.k = K + (base * H + h) * d; f.k_stride = D;
      f.v = V + (base * H + h) * d; f.v_stride = D;
      f.ts = ts ? ts + base : NULL;
      f.rab_p = rab_p; f.n_pos = n_pos;
      f.rab_t = rab_t; f.n_tb = n_tb;
      f.inv_nmax = 1.0 / n_max;
      f.time_filter = time_filter;
      for (int i = 0; i < f.L; i++) {
        const double *doi = dO + (base + i) * D + (long)h * d;
        const double *qi = f.q + (long)i * D;
        double *dqi = dQ + (base + i) * D + (long)h * d;
        for (int j = 0; j < f.L; j++) {
          if (!visible_t(i, j, f.L, f.P, f.C, f.ts, f.time_filter)) continue;
          int pidx, tidx;
          double s = logit(&f, i, j, &pidx, &tidx);
          double sig = 1.0 / (1.0 + exp(-s));
          double a = s * sig * f.inv_nmax;
          const double *kj = f.k + (long)j * D, *vj = f.v + (long)j * D;
          double da = 0.0;
          for (int c = 0; c < d; c++) da += doi[c] * vj[c];
          double ds = da * sig * (1.0 + s * (1.0 - sig)) * f.inv_nmax;
          double *dkj = dK + (base + j) * D + (long)h * d;
          double *dvj = dV + (base + j) * D + (long)h * d;
          for (int c = 0; c < d; c++) {
            dvj[c] += a * doi[c];
            dqi[c] += ds * kj[c];
            dkj[c] += ds * qi[c];
          }
          if (pidx >= 0) {
            pp[(long)tid * n_pos + pidx] += ds;
            ppa[(long)tid * n_pos + pidx] += fabs(ds);
          }
          if (tidx >= 0) {
            pt[(long)tid * n_tb + tidx] += ds;
            pta[(long)tid * n_tb + tidx] += fabs(ds);
          }
        }
      }
    }
  }
  if (drab_p) {
    for (int p = 0; p < n_pos; p++) {
      double s = 0.0;
      for (int t = 0; t < nth; t++) s += pp[(long)t * n_pos + p];
      drab_p[p] = s;
    }
  }
  if (drab_t) {
    for (int p = 0; p < n_tb; p++) {
      double s = 0.0;
      for (int t = 0; t < nth; t++) s += pt[(long)t * n_tb + p];
      drab_t[p] = s;
    }
  }
  if (drab_p_abs) {
    for (int p = 0; p < n_pos; p++) {
      double s = 0.0;
      for (int t = 0; t < nth; t++) s += ppa[(long)t * n_pos + p];
      drab_p_abs[p] = s;
    }
  }
  if (drab_t_abs) {
    for (int p = 0; p < n_tb; p++) {
      double s = 0.0;
      for (int t = 0; t < nth; t++) s += pta[(long)t * n_tb + p];
      drab_t_abs[p] = s;
    }
  }
  if (dgamma && gamma) {
    for (long e = 0; e < (long)G * D; e++) {
      double s = 0.0;
      for (int t = 0; t < nth; t++) s += pg[(long)t * G * D + e];
      dgamma[e] = s;
    }
  }
  if (dbeta && beta) {
    for (long e = 0; e < (long)G * D; e++) {
      double s = 0.0;
      for (int t = 0; t < nth; t++) s += pb[(long)t * G * D + e];
      dbeta[e] = s;
    }
  }
  free(O); free(Yt); free(mean); free(rstd); free(dO);
  free(pg); free(pb); free(pp); free(pt); free(ppa); free(pta);
  return 0;
}

/*
 * M-FALCON scoring with cached history K/V. For user b the frame is
 * [history (n_b tokens) | candidates (m_b tokens)] with no prefix and a
 * candidate tail of m_b, i.e. candidates see the whole history and
 * themselves. Only candidate rows are produced. The history rows' K/V come
 * from the cache; the candidates' own Q/K/V/U from Qc/Kc/Vc/Uc. Layouts as in
 * oracle_fwd, with token counts hist_offsets[B] and cand_offsets[B].
 */
int oracle_mfalcon(int B, int H, int d, const int32_t *hist_offsets,
                   const int32_t *cand_offsets, const double *Kcache, const double *Vcache,
                   const int64_t *hist_ts, const double *Qc, const double *Kc, const double *Vc,
                   const double *Uc, const int64_t *cand_ts, const double *rab_p, int n_pos,
                   const double *rab_t, int n_tb, double n_max, int norm, double eps,
                   const uint8_t *cand_group, int n_groups, const double *gamma,
                   const double *beta, double *Yc, double *Oc, double *mean, double *rstd,
                   int time_filter, int nthreads) {
  if (B < 0 || H <= 0 || d <= 0 || !hist_offsets || !cand_offsets) return 1;
  if (hist_offsets[0] != 0 || cand_offsets[0] != 0) return 2;
  for (int b = 0; b < B; b++)
    if (hist_offsets[b + 1] < hist_offsets[b] || cand_offsets[b + 1] < cand_offsets[b]) return 3;
  if (n_max <= 0) return 5;
  if (norm == NORM_GLN && (!cand_group || n_groups <= 0)) return 6;
  const int D = H * d;
  const long Tc = cand_offsets[B];
  if (norm == NORM_GLN)
    for (long t = 0; t < Tc; t++)
      if (cand_group[t] >= n_groups) return 8;
  const int use_ts = hist_ts && cand_ts;
  if (time_filter && !use_ts) return 9;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < (long)B * H; bh++) {
    int b = (int)(bh / H), h = (int)(bh % H);
    int n = hist_offsets[b + 1] - hist_offsets[b];
    int m = cand_offsets[b + 1] - cand_offsets[b];
    long hb = hist_offsets[b], cb = cand_offsets[b];
    int L = n + m;
    /* Assemble the frame of this (user, head) as plain [L, d] arrays. */
    double *fq = (double *)calloc((size_t)L * d + 1, sizeof(double));
    double *fk = (double *)calloc((size_t)L * d + 1, sizeof(double));
    double *fv = (double *)calloc((size_t)L * d + 1, sizeof(double));
    int64_t *ft = (int64_t *)calloc((size_t)L + 1, sizeof(int64_t));
    for (int j = 0; j < n; j++) {
      memcpy(fk + (long)j * d, Kcache + ((hb + j) * H + h) * d, sizeof(double) * d);
      memcpy(fv + (long)j * d, Vcache + ((hb + j) * H + h) * d, sizeof(double) * d);
      if (use_ts) ft[j] = hist_ts[hb + j];
    }
    for (int c = 0; c < m; c++) {
      memcpy(fq + (long)(n + c) * d, Qc + ((cb + c) * H + h) * d, sizeof(double) * d);
      memcpy(fk + (long)(n + c) * d, Kc + ((cb + c) * H + h) * d, sizeof(double) * d);
      memcpy(fv + (long)(n + c) * d, Vc + ((cb + c) * H + h) * d, sizeof(double) * d);
      if (use_ts) ft[n + c] = cand_ts[cb + c];
    }
    frame_t f;
    f.L = L; f.P = 0; f.C = m; f.d = d;
    f.q = fq; f.q_stride = d;
    f.k = fk; f.k_stride = d;
    f.v = fv; f.v_stride = d;
    f.ts = use_ts ? ft : NULL;
    f.rab_p = rab_p; f.n_pos = n_pos;
    f.rab_t = rab_t; f.n_tb = n_tb;
    f.inv_nmax = 1.0 / n_max;
    f.time_filter = time_filter;
    for (int c = 0; c < m; c++) attend_row(&f, n + c, Oc + (cb + c) * D + (long)h * d);
    free(fq); free(fk); free(fv); free(ft);
  }
#pragma omp parallel for schedule(static)
  for (long t = 0; t < Tc; t++) {
    int g = (norm == NORM_GLN) ? cand_group[t] : 0;
    norm_token(norm, D, Oc + t * D, Uc + t * D, eps, gamma ? gamma + (long)g * D : NULL,
               beta ? beta + (long)g * D : NULL, Yc + t * D, mean + t, rstd + t);
  }
  return 0;
}

/*
 * Tile classification by brute force over every pair. A query tile covers
 * rows [r0, r0+nrows) of a frame of length L (prefix P, candidate tail C);
 * key tile kt covers keys [kt*BN, kt*BN+BN). The pairs that tiles carry are
 * the visible pairs except a candidate's pair with itself (that term is added
 * per row, outside the tiles). A key tile is present when it holds at least
 * one such pair and FULL when every (row, key) pair of it, keys beyond L
 * included, is such a pair. Writes kind[kt] = 0 absent, 1 partial, 2 full
 * for kt in [0, nkt) and returns the number of present tiles.
 */
int oracle_classify_tiles(int L, int P, int C, int r0, int nrows, int BN, int nkt, int8_t *kind) {
  return oracle_classify_tiles_tf(L, P, C, r0, nrows, BN, nkt, 0, kind);
}

/* The same when MTGR's timestamp filter is on. The schedule is built from
 * the segment structure alone, so a (candidate row, causal key) pair counts
 * as possibly visible: it makes its tile present, and never full. */
int oracle_classify_tiles_tf(int L, int P, int C, int r0, int nrows, int BN, int nkt,
                             int time_filter, int8_t *kind) {
  int E = L - C, present = 0;
  for (int kt = 0; kt < nkt; kt++) {
    long carried = 0, sure = 0, total = 0;
    for (int i = r0; i < r0 + nrows; i++) {
      for (int j = kt * BN; j < kt * BN + BN; j++) {
        total++;
        int cand_self = (i >= E && j == i);
        if (!oracle_visible(i, j, L, P, C) || cand_self) continue;
        carried++;
        if (!(time_filter && i >= E && j >= P && j < E)) sure++;
      }
    }
    kind[kt] = carried == 0 ? 0 : (sure == total ? 2 : 1);
    if (carried) present++;
  }
  return present;
}
