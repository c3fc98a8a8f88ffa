/*
 * Oracle for the Mamba-2 SSD core and its block shell.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the CPU-baseline
 * leg of the benchmark call this code; the product path never does.  It shares
 * no code, header or constant with the HIP library.
 *
 * Plain, slow and sequential in time, in double precision.  Each function
 * follows a passage of the burn_dragon_kernel 0.5.0 page
 * "src/sequence/mamba2/backward.rs":
 *
 *   ssd_oracle_fwd       the recurrence of ssd_forward_state_history_reference,
 *                        with the readout y = C . h_t + D x_t of the tensorized
 *                        block backward (the "y_grouped" expression).
 *   ssd_oracle_bwd       the reverse-time loop of ssd_backward_reference, plus
 *                        the gradient of the initial state (the carry left after
 *                        the step t = 0; the page computes it but does not return
 *                        it), and optionally a gradient of the final state, which
 *                        is the carry before the first reverse step (the page's
 *                        loop starts from a zero carry).
 *   conv_oracle_fwd/bwd  depthwise_conv_preact_with_history, silu, and the
 *                        tap loop of the block backward's conv/SiLU fallback.
 *   rmsnorm_oracle_fwd/bwd  rmsnorm_gated_forward_from_inv_rms (with inv_rms
 *                        computed as in the block backward) and
 *                        rmsnorm_gated_backward_from_inv_rms.
 *
 * Parallelism: independent (batch, head) units on POSIX threads; every
 * reduction across units (the per-group sums of dB/dC over heads, dA_log and
 * dD over the batch) runs afterwards in one fixed order, so results do not
 * depend on the thread count.
 *
 * Layouts (row-major): x, y, dy, dx [b,T,H,P]; dt, ddt [b,T,H];
 * B, C, dB, dC [b,T,G,N]; A_log, D, dA_log, dD [H]; h0, final, dh0 [b,H,P,N];
 * chunk_states [b,nc,H,P,N] = the state entering each chunk of length `chunk`.
 * Head h reads group h / (H/G).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t b, T, H, P, N, G;
} dims_t;

/* ---------------------------------------------------------------- threads */

typedef void (*unit_fn)(void *ctx, int64_t unit);

typedef struct {
  unit_fn fn;
  void *ctx;
  int64_t nunits;
  int64_t next; /* shared counter */
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    int64_t u = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
    if (u >= p->nunits) break;
    p->fn(p->ctx, u);
  }
  return NULL;
}

static void run_units(unit_fn fn, void *ctx, int64_t nunits, int nthreads) {
  pool_t p = {fn, ctx, nunits, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nunits) nthreads = (int)(nunits > 0 ? nunits : 1);
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[started], NULL, pool_worker, &p) == 0) ++started;
  }
  pool_worker(&p);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------ SSD forward */

typedef struct {
  dims_t d;
  int64_t chunk;
  const double *x, *dt, *A_log, *B, *C, *D, *h0;
  double *y, *final_state, *chunk_states;
} fwd_ctx;

/* One (batch, head) unit of the recurrence
 *   h_t = exp(dt_t * A) h_{t-1} + dt_t x_t (outer) B_t,   A = -exp(A_log)
 *   y_t = h_t . C_t + D x_t
 * with h_{-1} = h0 (zeros when absent).  The readout uses the updated state. */
static void fwd_unit(void *vctx, int64_t unit) {
  fwd_ctx *c = (fwd_ctx *)vctx;
  const dims_t d = c->d;
  const int64_t bi = unit / d.H, h = unit % d.H;
  const int64_t g = h / (d.H / d.G);
  const int64_t PN = d.P * d.N;
  const double A = -exp(c->A_log[h]);
  const double Dh = c->D[h];
  double *st = (double *)malloc(sizeof(double) * PN);
  if (c->h0)
    memcpy(st, c->h0 + (bi * d.H + h) * PN, sizeof(double) * PN);
  else
    memset(st, 0, sizeof(double) * PN);
  const int64_t nc = c->chunk > 0 ? d.T / c->chunk : 0;
  for (int64_t t = 0; t < d.T; ++t) {
    if (c->chunk_states && c->chunk > 0 && t % c->chunk == 0 && t / c->chunk < nc) {
      memcpy(c->chunk_states + ((bi * nc + t / c->chunk) * d.H + h) * PN, st, sizeof(double) * PN);
    }
    const double dtv = c->dt[(bi * d.T + t) * d.H + h];
    const double decay = exp(dtv * A);
    const double *xt = c->x + ((bi * d.T + t) * d.H + h) * d.P;
    const double *Bt = c->B + ((bi * d.T + t) * d.G + g) * d.N;
    const double *Ct = c->C + ((bi * d.T + t) * d.G + g) * d.N;
    double *yt = c->y ? c->y + ((bi * d.T + t) * d.H + h) * d.P : NULL;
    for (int64_t p = 0; p < d.P; ++p) {
      const double u = dtv * xt[p];
      double *row = st + p * d.N;
      double acc = 0.0;
      for (int64_t n = 0; n < d.N; ++n) {
        row[n] = decay * row[n] + u * Bt[n];
        acc += row[n] * Ct[n];
      }
      if (yt) yt[p] = acc + Dh * xt[p];
    }
  }
  if (c->final_state) memcpy(c->final_state + (bi * d.H + h) * PN, st, sizeof(double) * PN);
  free(st);
}

int ssd_oracle_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                   int64_t ngroups, int64_t chunk, const double *x, const double *dt,
                   const double *A_log, const double *B, const double *C, const double *D,
                   const double *h0, double *y, double *final_state, double *chunk_states,
                   int nthreads) {
  if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
    return -1;
  if (nheads % ngroups) return -2;
  if (chunk_states && (chunk <= 0 || seqlen % chunk)) return -2;
  fwd_ctx c = {{batch, seqlen, nheads, headdim, dstate, ngroups}, chunk, x, dt, A_log, B, C, D, h0,
               y, final_state, chunk_states};
  run_units(fwd_unit, &c, batch * nheads, nthreads);
  return 0;
}

/* ----------------------------------------------------------- SSD backward */

typedef struct {
  dims_t d;
  const double *x, *dt, *A_log, *B, *C, *D, *h0, *dy, *dfinal;
  double *dx, *ddt, *dh0;
  double *dB_head, *dC_head; /* per-head partials [b,T,H,N] */
  double *ga_unit, *dD_unit; /* per-unit partials [b*H] */
} bwd_ctx;

#define SEG 64 /* states are checkpointed every SEG steps and recomputed */

/* One (batch, head) unit of the reverse-time loop.  Per step t, going
 * backwards, with G_t = dy_t (outer) C_t + carry:
 *   dC_t   += sum_p dy_t[p] h_t[p,:]                  (summed over heads later)
 *   gdA     = <G_t, h_{t-1}>
 *   dB_t   += dt_t x_t^T G_t                          (summed over heads later)
 *   dx_t    = D dy_t + dt_t G_t B_t
 *   ddt_t   = <G_t, x_t (outer) B_t> + gdA exp(dt_t A) A
 *   ga     += gdA exp(dt_t A) dt_t
 *   carry   = G_t exp(dt_t A)
 * and afterwards dA_log = A * sum ga (over batch and time), dh0 = carry.
 * The forward states are recomputed segment by segment from checkpoints; the
 * recomputation is the same sequential loop, so h_t is bit-identical. */
static void bwd_unit(void *vctx, int64_t unit) {
  bwd_ctx *c = (bwd_ctx *)vctx;
  const dims_t d = c->d;
  const int64_t bi = unit / d.H, h = unit % d.H;
  const int64_t g = h / (d.H / d.G);
  const int64_t PN = d.P * d.N;
  const double A = -exp(c->A_log[h]);
  const double Dh = c->D[h];
  const int64_t nseg = (d.T + SEG - 1) / SEG;
  double *ckpt = (double *)malloc(sizeof(double) * PN * (nseg > 0 ? nseg : 1));
  double *seg = (double *)malloc(sizeof(double) * PN * SEG);
  double *carry = (double *)calloc((size_t)PN, sizeof(double));
  double *Gs = (double *)malloc(sizeof(double) * PN);
  /* the gradient of the final state enters the reverse loop as its carry
   * (zero when the loss does not involve the final state) */
  if (c->dfinal) memcpy(carry, c->dfinal + (bi * d.H + h) * PN, sizeof(double) * PN);
  double *st = (double *)malloc(sizeof(double) * PN);
  double ga = 0.0, dDacc = 0.0;

  /* forward pass, keeping the state that enters every segment */
  if (c->h0)
    memcpy(st, c->h0 + (bi * d.H + h) * PN, sizeof(double) * PN);
  else
    memset(st, 0, sizeof(double) * PN);
  for (int64_t t = 0; t < d.T; ++t) {
    if (t % SEG == 0) memcpy(ckpt + (t / SEG) * PN, st, sizeof(double) * PN);
    const double dtv = c->dt[(bi * d.T + t) * d.H + h];
    const double decay = exp(dtv * A);
    const double *xt = c->x + ((bi * d.T + t) * d.H + h) * d.P;
    const double *Bt = c->B + ((bi * d.T + t) * d.G + g) * d.N;
    for (int64_t p = 0; p < d.P; ++p) {
      const double u = dtv * xt[p];
      for (int64_t n = 0; n < d.N; ++n) st[p * d.N + n] = decay * st[p * d.N + n] + u * Bt[n];
    }
  }

  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t t0 = s * SEG;
    const int64_t t1 = (t0 + SEG < d.T) ? t0 + SEG : d.T;
    /* recompute h_t for t in [t0, t1) */
    memcpy(st, ckpt + s * PN, sizeof(double) * PN);
    for (int64_t t = t0; t < t1; ++t) {
      const double dtv = c->dt[(bi * d.T + t) * d.H + h];
      const double decay = exp(dtv * A);
      const double *xt = c->x + ((bi * d.T + t) * d.H + h) * d.P;
      const double *Bt = c->B + ((bi * d.T + t) * d.G + g) * d.N;
      for (int64_t p = 0; p < d.P; ++p) {
        const double u = dtv * xt[p];
        for (int64_t n = 0; n < d.N; ++n) st[p * d.N + n] = decay * st[p * d.N + n] + u * Bt[n];
      }
      memcpy(seg + (t - t0) * PN, st, sizeof(double) * PN);
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const double *ht = seg + (t - t0) * PN;
      const double *hprev = (t == t0) ? ckpt + s * PN : seg + (t - 1 - t0) * PN;
      const double dtv = c->dt[(bi * d.T + t) * d.H + h];
      const double decay = exp(dtv * A);
      const double *xt = c->x + ((bi * d.T + t) * d.H + h) * d.P;
      const double *dyt = c->dy + ((bi * d.T + t) * d.H + h) * d.P;
      const double *Bt = c->B + ((bi * d.T + t) * d.G + g) * d.N;
      const double *Ct = c->C + ((bi * d.T + t) * d.G + g) * d.N;
      double *dxt = c->dx + ((bi * d.T + t) * d.H + h) * d.P;
      double *dBt = c->dB_head + ((bi * d.T + t) * d.H + h) * d.N;
      double *dCt = c->dC_head + ((bi * d.T + t) * d.H + h) * d.N;

      for (int64_t n = 0; n < d.N; ++n) { dBt[n] = 0.0; dCt[n] = 0.0; }
      double gdA = 0.0, gdrive = 0.0;
      for (int64_t p = 0; p < d.P; ++p) {
        double xb = 0.0;
        for (int64_t n = 0; n < d.N; ++n) {
          const double gsv = dyt[p] * Ct[n] + carry[p * d.N + n];
          Gs[p * d.N + n] = gsv;
          dCt[n] += dyt[p] * ht[p * d.N + n];
          gdA += gsv * hprev[p * d.N + n];
          gdrive += gsv * xt[p] * Bt[n];
          dBt[n] += dtv * xt[p] * gsv;
          xb += gsv * Bt[n];
        }
        dxt[p] = Dh * dyt[p] + dtv * xb;
        dDacc += dyt[p] * xt[p];
      }
      c->ddt[(bi * d.T + t) * d.H + h] = gdrive + gdA * decay * A;
      ga += gdA * decay * dtv;
      for (int64_t i = 0; i < PN; ++i) carry[i] = Gs[i] * decay;
    }
  }
  if (c->dh0) memcpy(c->dh0 + (bi * d.H + h) * PN, carry, sizeof(double) * PN);
  c->ga_unit[unit] = ga;
  c->dD_unit[unit] = dDacc;
  free(ckpt);
  free(seg);
  free(carry);
  free(Gs);
  free(st);
}

int ssd_oracle_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                   int64_t ngroups, const double *x, const double *dt, const double *A_log,
                   const double *B, const double *C, const double *D, const double *h0,
                   const double *dy, const double *dfinal, double *dx, double *ddt, double *dA_log,
                   double *dB, double *dC, double *dD, double *dh0, int nthreads) {
  if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
    return -1;
  if (nheads % ngroups) return -2;
  const int64_t b = batch, T = seqlen, H = nheads, N = dstate, G = ngroups, hpg = H / G;
  const int64_t nunit = b * H;
  double *dB_head = (double *)malloc(sizeof(double) * (size_t)(b * T * H * N + 1));
  double *dC_head = (double *)malloc(sizeof(double) * (size_t)(b * T * H * N + 1));
  double *ga_unit = (double *)calloc((size_t)(nunit + 1), sizeof(double));
  double *dD_unit = (double *)calloc((size_t)(nunit + 1), sizeof(double));
  if (!dB_head || !dC_head || !ga_unit || !dD_unit) {
    free(dB_head); free(dC_head); free(ga_unit); free(dD_unit);
    return -3;
  }
  bwd_ctx c = {{b, T, H, headdim, N, G}, x, dt, A_log, B, C, D, h0, dy, dfinal, dx, ddt, dh0,
               dB_head, dC_head, ga_unit, dD_unit};
  run_units(bwd_unit, &c, nunit, nthreads);

  /* group sums over heads, ascending head order */
  for (int64_t bt = 0; bt < b * T; ++bt)
    for (int64_t g = 0; g < G; ++g)
      for (int64_t n = 0; n < N; ++n) {
        double sb = 0.0, sc = 0.0;
        for (int64_t j = 0; j < hpg; ++j) {
          sb += dB_head[(bt * H + g * hpg + j) * N + n];
          sc += dC_head[(bt * H + g * hpg + j) * N + n];
        }
        dB[(bt * G + g) * N + n] = sb;
        dC[(bt * G + g) * N + n] = sc;
      }
  /* parameter gradients, ascending batch order */
  for (int64_t h = 0; h < H; ++h) {
    double ga = 0.0, sd = 0.0;
    for (int64_t bi = 0; bi < b; ++bi) {
      ga += ga_unit[bi * H + h];
      sd += dD_unit[bi * H + h];
    }
    dA_log[h] = -exp(A_log[h]) * ga;
    dD[h] = sd;
  }
  free(dB_head);
  free(dC_head);
  free(ga_unit);
  free(dD_unit);
  return 0;
}

/* ------------------------------------------------- conv1d + SiLU (shell) */

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Causal depthwise conv with a zero initial state, then SiLU.
 * xbc, act: [b,T,Cd]; w: [Cd,K]; bias: [Cd] (nullable); preact (nullable).
 * Tap k = K-1 multiplies the current step:
 *   preact[t,c] = bias[c] + sum_k w[c,k] * xbc[t-(K-1)+k, c]   (zero before t=0)
 *   act = preact * sigmoid(preact)                                          */
int conv_oracle_fwd(int64_t batch, int64_t seqlen, int64_t channels, int64_t d_conv,
                    const double *xbc, const double *w, const double *bias, double *preact,
                    double *act) {
  if (batch < 0 || seqlen < 0 || channels <= 0 || d_conv <= 0) return -1;
  for (int64_t bi = 0; bi < batch; ++bi)
    for (int64_t t = 0; t < seqlen; ++t)
      for (int64_t ch = 0; ch < channels; ++ch) {
        double acc = bias ? bias[ch] : 0.0;
        for (int64_t k = 0; k < d_conv; ++k) {
          const int64_t src = t - (d_conv - 1) + k;
          if (src >= 0) acc += w[ch * d_conv + k] * xbc[(bi * seqlen + src) * channels + ch];
        }
        const int64_t o = (bi * seqlen + t) * channels + ch;
        if (preact) preact[o] = acc;
        if (act) act[o] = acc * sigmoid(acc);
      }
  return 0;
}

/* Backward of the above.  gact: gradient of act [b,T,Cd].
 *   gp = gact * s (1 + p (1 - s)),  s = sigmoid(p)
 *   dbias[c]  = sum_{b,t} gp[t,c]
 *   dw[c,k]   = sum_{b,t} gp[t,c] * xbc[t-(K-1)+k, c]
 *   dxbc[u,c] = sum_k gp[u+(K-1)-k, c] * w[c,k]                             */
int conv_oracle_bwd(int64_t batch, int64_t seqlen, int64_t channels, int64_t d_conv,
                    const double *xbc, const double *w, const double *bias, const double *gact,
                    double *dxbc, double *dw, double *dbias) {
  if (batch < 0 || seqlen < 0 || channels <= 0 || d_conv <= 0) return -1;
  const int64_t n = batch * seqlen * channels;
  double *gp = (double *)malloc(sizeof(double) * (size_t)(n + 1));
  if (!gp) return -3;
  for (int64_t bi = 0; bi < batch; ++bi)
    for (int64_t t = 0; t < seqlen; ++t)
      for (int64_t ch = 0; ch < channels; ++ch) {
        double p = bias ? bias[ch] : 0.0;
        for (int64_t k = 0; k < d_conv; ++k) {
          const int64_t src = t - (d_conv - 1) + k;
          if (src >= 0) p += w[ch * d_conv + k] * xbc[(bi * seqlen + src) * channels + ch];
        }
        const double s = sigmoid(p);
        const int64_t o = (bi * seqlen + t) * channels + ch;
        gp[o] = gact[o] * s * (1.0 + p * (1.0 - s));
      }
  for (int64_t ch = 0; ch < channels; ++ch) {
    double sb = 0.0;
    for (int64_t bi = 0; bi < batch; ++bi)
      for (int64_t t = 0; t < seqlen; ++t) sb += gp[(bi * seqlen + t) * channels + ch];
    dbias[ch] = sb;
    for (int64_t k = 0; k < d_conv; ++k) {
      double sw = 0.0;
      for (int64_t bi = 0; bi < batch; ++bi)
        for (int64_t t = 0; t < seqlen; ++t) {
          const int64_t src = t - (d_conv - 1) + k;
          if (src >= 0)
            sw += gp[(bi * seqlen + t) * channels + ch] * xbc[(bi * seqlen + src) * channels + ch];
        }
      dw[ch * d_conv + k] = sw;
    }
  }
  for (int64_t bi = 0; bi < batch; ++bi)
    for (int64_t u = 0; u < seqlen; ++u)
      for (int64_t ch = 0; ch < channels; ++ch) {
        double acc = 0.0;
        for (int64_t k = 0; k < d_conv; ++k) {
          const int64_t t = u + (d_conv - 1) - k;
          if (t < seqlen) acc += gp[(bi * seqlen + t) * channels + ch] * w[ch * d_conv + k];
        }
        dxbc[(bi * seqlen + u) * channels + ch] = acc;
      }
  free(gp);
  return 0;
}

/* ---------------------------------------------- RMSNorm-gated (shell) */

/* rows = b*T rows of width D.
 *   inv_rms = 1 / sqrt(mean(y^2) + eps)
 *   out     = y * inv_rms * w * silu(z)                                    */
int rmsnorm_oracle_fwd(int64_t rows, int64_t width, double eps, const double *y, const double *z,
                       const double *w, double *out, double *inv_rms) {
  if (rows < 0 || width <= 0) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const double *yr = y + r * width;
    double ss = 0.0;
    for (int64_t i = 0; i < width; ++i) ss += yr[i] * yr[i];
    const double inv = 1.0 / sqrt(ss / (double)width + eps);
    if (inv_rms) inv_rms[r] = inv;
    if (out)
      for (int64_t i = 0; i < width; ++i) {
        const double zv = z[r * width + i];
        out[r * width + i] = yr[i] * inv * w[i] * (zv * sigmoid(zv));
      }
  }
  return 0;
}

/* Backward with inv_rms taken as given (it still depends on y, and that
 * dependence is in the dy formula):
 *   gw    = g * silu(z)                      (grad of y*inv*w)
 *   dw    = sum_rows gw * y * inv
 *   gn    = gw * w
 *   dy    = gn * inv - y * (sum_i gn*y) * inv^3 / width
 *   dz    = g * (y*inv*w) * s (1 + z (1 - s)),  s = sigmoid(z)              */
int rmsnorm_oracle_bwd(int64_t rows, int64_t width, const double *y, const double *z,
                       const double *w, const double *inv_rms, const double *g, double *dy,
                       double *dz, double *dw) {
  if (rows < 0 || width <= 0) return -1;
  for (int64_t i = 0; i < width; ++i) dw[i] = 0.0;
  for (int64_t r = 0; r < rows; ++r) {
    const double inv = inv_rms[r];
    const double *yr = y + r * width, *zr = z + r * width, *gr = g + r * width;
    double dot = 0.0;
    for (int64_t i = 0; i < width; ++i) {
      const double gate = zr[i] * sigmoid(zr[i]);
      dot += gr[i] * gate * w[i] * yr[i];
    }
    for (int64_t i = 0; i < width; ++i) {
      const double s = sigmoid(zr[i]);
      const double gate = zr[i] * s;
      const double normalized = yr[i] * inv;
      const double gw = gr[i] * gate;
      dw[i] += gw * normalized;
      dy[r * width + i] = gw * w[i] * inv - yr[i] * dot * inv * inv * inv / (double)width;
      dz[r * width + i] = gr[i] * normalized * w[i] * s * (1.0 + zr[i] * (1.0 - s));
    }
  }
  return 0;
}
