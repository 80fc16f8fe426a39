/*
 * Driver for a sanitizer build of oracle.c (test infrastructure only): runs
 * oracle_fwd, oracle_bwd, oracle_mfalcon, the tile classifier and the time
 * bucket on small seeded problems (empty and one-token sequences, prefixes,
 * candidate tails, Group LayerNorm, both rab tables, the timestamp filter and
 * a row selection), so that AddressSanitizer and UndefinedBehaviorSanitizer
 * see every loop bound and index of the oracle. Exit status 0 when every call
 * succeeds; the sanitizers abort on the first finding.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_time_bucket(int64_t dt, int n_tb);
int oracle_classify_tiles_tf(int L, int P, int C, int r0, int nrows, int BN, int nkt, int time_filter,
                             int8_t *kind);
int oracle_fwd(int B, int H, int d, const int32_t *offsets, const int32_t *prefix_len,
               const int32_t *cand_len, const double *Q, const double *K, const double *V,
               const double *U, const int64_t *ts, const double *rab_p, int n_pos,
               const double *rab_t, int n_tb, double n_max, int norm, double eps,
               const uint8_t *group, int n_groups, const double *gamma, const double *beta,
               const uint8_t *row_sel, double *Y, double *O, double *mean, double *rstd,
               int time_filter, int nthreads);
int oracle_bwd(int B, int H, int d, const int32_t *offsets, const int32_t *prefix_len,
               const int32_t *cand_len, const double *Q, const double *K, const double *V,
               const double *U, const int64_t *ts, const double *rab_p, int n_pos,
               const double *rab_t, int n_tb, double n_max, int norm, double eps,
               const uint8_t *group, int n_groups, const double *gamma, const double *beta,
               const double *dY, double *dQ, double *dK, double *dV, double *dU,
               double *drab_p, double *drab_t, double *dgamma, double *dbeta,
               double *drab_p_abs, double *drab_t_abs, int time_filter, int nthreads);
int oracle_mfalcon(int B, int H, int d, const int32_t *hist_offsets,
                   const int32_t *cand_offsets, const double *Kcache, const double *Vcache,
                   const int64_t *hist_ts, const double *Qc, const double *Kc, const double *Vc,
                   const double *Uc, const int64_t *cand_ts, const double *rab_p, int n_pos,
                   const double *rab_t, int n_tb, double n_max, int norm, double eps,
                   const uint8_t *cand_group, int n_groups, const double *gamma,
                   const double *beta, double *Yc, double *Oc, double *mean, double *rstd,
                   int time_filter, int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uni(void) { /* xorshift64*, uniform in [-0.5, 0.5) */
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0 - 0.5;
}
static double *vec(long n) {
  double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; i++) p[i] = uni();
  return p;
}

static int run_case(int B, const int *lens, const int *pre, const int *cand, int H, int d, int n_pos, int n_tb,
                    int norm, int G, int tf, int use_sel) {
  int32_t *off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B + 1)), *P = NULL, *C = NULL;
  off[0] = 0;
  for (int b = 0; b < B; b++) off[b + 1] = off[b] + lens[b];
  if (pre) { P = (int32_t *)malloc(sizeof(int32_t) * (size_t)B); for (int b = 0; b < B; b++) P[b] = pre[b]; }
  if (cand) { C = (int32_t *)malloc(sizeof(int32_t) * (size_t)B); for (int b = 0; b < B; b++) C[b] = cand[b]; }
  const long T = off[B], D = (long)H * d;
  double *Q = vec(T * D), *K = vec(T * D), *V = vec(T * D), *U = vec(T * D), *dY = vec(T * D);
  int64_t *ts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
  for (int b = 0; b < B; b++) {
    int64_t t = 1700000000 + b * 1000;
    for (int i = off[b]; i < off[b + 1]; i++) { t += (int64_t)((uni() + 0.5) * 7000.0); ts[i] = t; }
  }
  double *rp = n_pos ? vec(n_pos) : NULL, *rt = n_tb ? vec(n_tb) : NULL;
  uint8_t *grp = NULL, *sel = NULL;
  if (norm == 2) { grp = (uint8_t *)malloc((size_t)(T > 0 ? T : 1)); for (long t = 0; t < T; t++) grp[t] = (uint8_t)(t % G); }
  if (use_sel) { sel = (uint8_t *)malloc((size_t)(T > 0 ? T : 1)); for (long t = 0; t < T; t++) sel[t] = (uint8_t)(t % 3 == 0); }
  double *gam = norm ? vec((long)G * D) : NULL, *bet = norm ? vec((long)G * D) : NULL;
  double *Y = vec(T * D), *O = vec(T * D), *mu = vec(T), *rs = vec(T);
  double *dQ = vec(T * D), *dK = vec(T * D), *dV = vec(T * D), *dU = vec(T * D);
  double *drp = vec(n_pos), *drt = vec(n_tb), *dg = vec((long)G * D), *db = vec((long)G * D);
  double *drpa = vec(n_pos), *drta = vec(n_tb);
  int rc = oracle_fwd(B, H, d, off, P, C, Q, K, V, U, ts, rp, n_pos, rt, n_tb, 8.0, norm, 1e-5, grp, G, gam, bet,
                      sel, Y, O, mu, rs, tf, 1);
  if (!rc)
    rc = oracle_bwd(B, H, d, off, P, C, Q, K, V, U, ts, rp, n_pos, rt, n_tb, 8.0, norm, 1e-5, grp, G, gam, bet, dY,
                    dQ, dK, dV, dU, drp, drt, norm ? dg : NULL, norm ? db : NULL, drpa, drta, tf, 1);
  for (int b = 0; b < B && !rc; b++) {
    const int L = lens[b], BN = 16, nkt = (L + BN - 1) / BN;
    int8_t *kind = (int8_t *)malloc((size_t)(nkt > 0 ? nkt : 1));
    for (int r0 = 0; r0 < L; r0 += 16)
      oracle_classify_tiles_tf(L, P ? P[b] : 0, C ? C[b] : 0, r0, L - r0 < 16 ? L - r0 : 16, BN, nkt, tf, kind);
    free(kind);
  }
  free(off); free(P); free(C); free(Q); free(K); free(V); free(U); free(dY); free(ts); free(rp); free(rt);
  free(grp); free(sel); free(gam); free(bet); free(Y); free(O); free(mu); free(rs); free(dQ); free(dK); free(dV);
  free(dU); free(drp); free(drt); free(dg); free(db); free(drpa); free(drta);
  return rc;
}

static int run_mfalcon(int B, const int *nh, const int *mc, int H, int d, int n_pos, int n_tb, int tf) {
  int32_t *ho = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B + 1)), *co = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B + 1));
  ho[0] = co[0] = 0;
  for (int b = 0; b < B; b++) { ho[b + 1] = ho[b] + nh[b]; co[b + 1] = co[b] + mc[b]; }
  const long Th = ho[B], Tc = co[B], D = (long)H * d;
  double *Kc_ = vec(Th * D), *Vc_ = vec(Th * D), *Q = vec(Tc * D), *K = vec(Tc * D), *V = vec(Tc * D), *U = vec(Tc * D);
  int64_t *hts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Th > 0 ? Th : 1));
  int64_t *cts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Tc > 0 ? Tc : 1));
  for (long i = 0; i < Th; i++) hts[i] = 1700000000 + i * 100;
  for (long i = 0; i < Tc; i++) cts[i] = 1700000000 + (i * 37) % (Th > 0 ? Th * 100 : 1);
  double *rp = n_pos ? vec(n_pos) : NULL, *rt = n_tb ? vec(n_tb) : NULL;
  double *Y = vec(Tc * D), *O = vec(Tc * D), *mu = vec(Tc), *rs = vec(Tc);
  int rc = oracle_mfalcon(B, H, d, ho, co, Kc_, Vc_, hts, Q, K, V, U, cts, rp, n_pos, rt, n_tb, 16.0, 1, 1e-5, NULL,
                          1, NULL, NULL, Y, O, mu, rs, tf, 1);
  free(ho); free(co); free(Kc_); free(Vc_); free(Q); free(K); free(V); free(U); free(hts); free(cts); free(rp);
  free(rt); free(Y); free(O); free(mu); free(rs);
  return rc;
}

int main(void) {
  int rc = 0;
  for (int64_t dt = -70000; dt <= 70000; dt += 977) rc |= oracle_time_bucket(dt, 17) < 0;
  rc |= oracle_time_bucket(INT64_MIN + 1, 40) != 39;
  {
    const int lens[] = {0, 1, 37, 64, 90};
    rc |= run_case(5, lens, NULL, NULL, 2, 16, 40, 12, 1, 1, 0, 0);
  }
  {
    const int lens[] = {50, 3, 70, 0};
    const int pre[] = {20, 1, 10, 0}, cand[] = {10, 1, 30, 0};
    rc |= run_case(4, lens, pre, cand, 3, 8, 64, 20, 2, 3, 0, 0);
    rc |= run_case(4, lens, pre, cand, 1, 32, 8, 4, 2, 2, 1, 1);
    rc |= run_case(4, lens, pre, cand, 2, 8, 0, 0, 0, 1, 0, 1);
  }
  {
    const int nh[] = {0, 40, 17}, mc[] = {5, 0, 23};
    rc |= run_mfalcon(3, nh, mc, 2, 16, 50, 10, 0);
    rc |= run_mfalcon(3, nh, mc, 1, 8, 0, 0, 1);
  }
  printf("oracle sanitizer driver: %s\n", rc ? "FAILED" : "ok");
  return rc != 0;
}
