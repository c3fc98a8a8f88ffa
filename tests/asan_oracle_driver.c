/* Host-side memory and undefined-behaviour check of the oracle (test
 * infrastructure): every buffer is malloc'ed at its exact size, so an access
 * past any extent is reported by AddressSanitizer; UndefinedBehaviorSanitizer
 * watches the index arithmetic.  Runs the SSD forward / backward and the shell
 * oracles over shapes that cover ragged checkpoint segments, one step, several
 * threads, optional pointers left null, and an empty batch.  Exit status 0 and
 * finite outputs on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssd_oracle_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double *,
                   const double *, const double *, const double *, const double *, const double *,
                   const double *, double *, double *, double *, int);
int ssd_oracle_bwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double *,
                   const double *, const double *, const double *, const double *, const double *,
                   const double *, const double *, const double *, double *, double *, double *,
                   double *, double *, double *, double *, int);
int conv_oracle_fwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                    const double *, double *, double *);
int conv_oracle_bwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                    const double *, const double *, double *, double *, double *);
int rmsnorm_oracle_fwd(int64_t, int64_t, double, const double *, const double *, const double *,
                       double *, double *);
int rmsnorm_oracle_bwd(int64_t, int64_t, const double *, const double *, const double *,
                       const double *, const double *, double *, double *, double *);

static uint64_t state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *buf(int64_t n, double scale, double offset) {
  double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = offset + scale * urand();
  return p;
}
static int finite_all(const double *p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run_ssd(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q,
                   int with_h0, int with_dfinal, int threads) {
  const int64_t nx = b * T * H * P, nb = b * T * G * N, nt = b * T * H, ns = b * H * P * N;
  const int64_t nc = Q > 0 ? T / Q : 0;
  double *x = buf(nx, 1, 0), *B = buf(nb, 1, 0), *C = buf(nb, 1, 0), *dt = buf(nt, 0.05, 0.1);
  double *A_log = buf(H, 1, 1.5), *D = buf(H, 1, 0), *dy = buf(nx, 1, 0);
  double *h0 = with_h0 ? buf(ns, 0.1, 0) : NULL, *dfin = with_dfinal ? buf(ns, 1, 0) : NULL;
  double *y = buf(nx, 0, 0), *fin = buf(ns, 0, 0), *cs = Q > 0 ? buf(b * nc * H * P * N, 0, 0) : NULL;
  double *dx = buf(nx, 0, 0), *ddt = buf(nt, 0, 0), *dA = buf(H, 0, 0), *dB = buf(nb, 0, 0);
  double *dC = buf(nb, 0, 0), *dD = buf(H, 0, 0), *dh0 = buf(ns, 0, 0);
  int rc = ssd_oracle_fwd(b, T, H, P, N, G, Q, x, dt, A_log, B, C, D, h0, y, fin, cs, threads);
  if (rc == 0)
    rc = ssd_oracle_bwd(b, T, H, P, N, G, x, dt, A_log, B, C, D, h0, dy, dfin, dx, ddt, dA, dB, dC,
                        dD, dh0, threads);
  int ok = rc == 0 && finite_all(y, nx) && finite_all(fin, ns) && finite_all(dx, nx) &&
           finite_all(ddt, nt) && finite_all(dB, nb) && finite_all(dC, nb) && finite_all(dh0, ns) &&
           finite_all(dA, H) && finite_all(dD, H);
  double *ps[] = {x, B, C, dt, A_log, D, dy, h0, dfin, y, fin, cs, dx, ddt, dA, dB, dC, dD, dh0};
  for (size_t i = 0; i < sizeof(ps) / sizeof(ps[0]); ++i) free(ps[i]);
  if (!ok) fprintf(stderr, "ssd case b=%ld T=%ld H=%ld P=%ld N=%ld G=%ld Q=%ld failed (rc %d)\n", (long)b,
                   (long)T, (long)H, (long)P, (long)N, (long)G, (long)Q, rc);
  return ok;
}

static int run_shell(int64_t b, int64_t T, int64_t Cd, int64_t K) {
  const int64_t n = b * T * Cd;
  double *xbc = buf(n, 1, 0), *w = buf(Cd * K, 0.5, 0), *bias = buf(Cd, 0.1, 0), *pre = buf(n, 0, 0);
  double *act = buf(n, 0, 0), *g = buf(n, 1, 0), *dxbc = buf(n, 0, 0), *dw = buf(Cd * K, 0, 0);
  double *db = buf(Cd, 0, 0);
  int rc = conv_oracle_fwd(b, T, Cd, K, xbc, w, bias, pre, act);
  if (rc == 0) rc = conv_oracle_bwd(b, T, Cd, K, xbc, w, bias, g, dxbc, dw, db);
  const int64_t rows = b * T;
  double *z = buf(n, 1, 0), *nw = buf(Cd, 0.1, 1), *out = buf(n, 0, 0), *inv = buf(rows, 0, 0);
  double *dy = buf(n, 0, 0), *dz = buf(n, 0, 0), *dnw = buf(Cd, 0, 0);
  if (rc == 0) rc = rmsnorm_oracle_fwd(rows, Cd, 1e-5, xbc, z, nw, out, inv);
  if (rc == 0) rc = rmsnorm_oracle_bwd(rows, Cd, xbc, z, nw, inv, g, dy, dz, dnw);
  int ok = rc == 0 && finite_all(act, n) && finite_all(dxbc, n) && finite_all(dw, Cd * K) &&
           finite_all(out, n) && finite_all(dy, n) && finite_all(dz, n) && finite_all(dnw, Cd);
  double *ps[] = {xbc, w, bias, pre, act, g, dxbc, dw, db, z, nw, out, inv, dy, dz, dnw};
  for (size_t i = 0; i < sizeof(ps) / sizeof(ps[0]); ++i) free(ps[i]);
  if (!ok) fprintf(stderr, "shell case b=%ld T=%ld C=%ld K=%ld failed (rc %d)\n", (long)b, (long)T,
                   (long)Cd, (long)K, rc);
  return ok;
}

int main(void) {
  int ok = 1;
  ok &= run_ssd(1, 64, 2, 8, 4, 1, 16, 0, 0, 1);     /* the tiny workload's shape */
  ok &= run_ssd(2, 150, 4, 3, 5, 2, 50, 1, 1, 3);    /* ragged checkpoint segments, groups */
  ok &= run_ssd(1, 1, 3, 2, 2, 3, 1, 1, 0, 2);       /* one step */
  ok &= run_ssd(2, 131, 6, 4, 3, 2, 0, 0, 1, 4);     /* no chunk states, T past two checkpoints */
  ok &= run_ssd(0, 16, 2, 2, 2, 1, 16, 1, 1, 2);     /* empty batch */
  ok &= run_shell(2, 37, 12, 4);
  ok &= run_shell(1, 2, 5, 3);                       /* fewer steps than taps */
  ok &= run_shell(1, 9, 7, 1);
  if (!ok) return 1;
  puts("oracle sanitizer run ok");
  return 0;
}
