/*
 * gdnref.c -- plain fp64 CPU oracle for the Gated DeltaNet forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or helper with the GPU library: it is written from the pages'
 * definitions, slowly and obviously, token by token, in double precision.
 *
 * Sources (the pages are named by title and section):
 *  - "Source notes" (NextTransformer methods page), section "Linear
 *    attention", rows deltanet / kda / gdn: the gated delta-rule state update
 *    with a scalar per-head decay applied before the delta update (gdn), a
 *    per-key-channel decay applied before the delta update (kda), the read
 *    y = q^T S after the write (deltanet), causal conv + SiLU and
 *    L2-normalised q/k (deltanet, kda).
 *  - same page, section "Backend and numerical limits": query scale is 1; an
 *    FP64 recurrent scan is the correctness reference.
 *  - "Frontier model atlas", entries 03 and 08 (Gated DeltaNet): four-token
 *    causal convolution in front of the state update; 16 key heads shared by
 *    48 value heads.
 *
 * Orientation.  The pages write the state as a K x V matrix S with read
 * y = q^T S.  Here the state of one (batch, value head) is its transpose,
 * a dv x dk matrix (row i = value channel, column j = key channel), so that
 * the read is o_t = S_t q_t.  Both orientations give the same numbers.
 *
 * Readings where the pages leave a step open (all are listed in the design
 * notes of the repository):
 *  - decay first, then the prediction uses the decayed state:
 *        S <- alpha_t S          (kda: S <- S diag(alpha_t))
 *        p  = S k_t
 *        S <- S + beta_t (v_t - p) k_t^T
 *        o_t = S q_t             (read after the write, scale 1)
 *  - alpha_t = exp(g_t) with g_t the natural-log decay handed in;
 *  - value head h reads key/query head h / (Hv / Hk) (consecutive grouping);
 *  - conv: depthwise, 4 taps, no bias, zero history before t = 0, tap 3
 *    multiplies the current token; SiLU after the conv; q and k are then
 *    divided by sqrt(sum z^2 + eps) per (token, head).
 *
 * Inputs are float arrays whose values are the exact stored values (bf16 and
 * fp16 widen to float exactly); every operation is carried out in double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Recurrence                                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
  int B, T, Hk, Hv, dk, dv, per_channel_gate, no_delta;
  const float *q, *k, *v, *g, *beta, *S0;
  const double *S0d; /* used instead of S0 when set */
  int nsel;
  const int *sel_b, *sel_h;
  double *o, *S_T;
  int next; /* next chain index to take (guarded by mu) */
  pthread_mutex_t mu;
} rec_job;

/* One (batch b, value head h) chain over all T tokens. */
static void rec_chain(const rec_job *J, int n, double *S) {
  const int b = J->sel_b[n], h = J->sel_h[n];
  const int dk = J->dk, dv = J->dv, T = J->T;
  const int kh = h / (J->Hv / J->Hk); /* key/query head read by value head h */
  double *o = J->o + (size_t)n * T * dv;
  int i, j, t;

  if (J->S0d) {
    memcpy(S, J->S0d + ((size_t)b * J->Hv + h) * dv * dk, sizeof(double) * dv * dk);
  } else if (J->S0) {
    const float *s0 = J->S0 + ((size_t)b * J->Hv + h) * dv * dk;
    for (i = 0; i < dv * dk; ++i) S[i] = (double)s0[i];
  } else {
    memset(S, 0, sizeof(double) * dv * dk);
  }

  for (t = 0; t < T; ++t) {
    const size_t bt = (size_t)b * T + t;
    const float *qt = J->q + (bt * J->Hk + kh) * dk;
    const float *kt = J->k + (bt * J->Hk + kh) * dk;
    const float *vt = J->v + (bt * J->Hv + h) * dv;
    const double beta = (double)J->beta[bt * J->Hv + h];

    /* decay before the delta update */
    if (J->per_channel_gate) {
      const float *gt = J->g + (bt * J->Hv + h) * dk;
      for (j = 0; j < dk; ++j) {
        const double a = exp((double)gt[j]);
        for (i = 0; i < dv; ++i) S[(size_t)i * dk + j] *= a;
      }
    } else {
      const double a = exp((double)J->g[bt * J->Hv + h]);
      for (i = 0; i < dv * dk; ++i) S[i] *= a;
    }

    /* delta update: S <- S + beta (v - S k) k^T; without the delta
       correction ("SinkProbe" page, hybrid_nodelta; "Source notes", gla
       row): S <- S + beta v k^T */
    for (i = 0; i < dv; ++i) {
      double *row = S + (size_t)i * dk;
      double p = 0.0;
      if (!J->no_delta)
        for (j = 0; j < dk; ++j) p += row[j] * (double)kt[j];
      const double u = beta * ((double)vt[i] - p);
      for (j = 0; j < dk; ++j) row[j] += u * (double)kt[j];
    }

    /* read after the write, scale 1 */
    for (i = 0; i < dv; ++i) {
      const double *row = S + (size_t)i * dk;
      double acc = 0.0;
      for (j = 0; j < dk; ++j) acc += row[j] * (double)qt[j];
      o[(size_t)t * dv + i] = acc;
    }
  }
  memcpy(J->S_T + (size_t)n * dv * dk, S, sizeof(double) * dv * dk);
}

static void *rec_worker(void *arg) {
  rec_job *J = (rec_job *)arg;
  double *S = (double *)malloc(sizeof(double) * (size_t)J->dv * J->dk);
  if (!S) return NULL;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int n = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (n >= J->nsel) break;
    rec_chain(J, n, S);
  }
  free(S);
  return NULL;
}

/*
 * gdnref_recurrent: token-by-token recurrence for the selected chains.
 *
 *   q, k  [B,T,Hk,dk]   v [B,T,Hv,dv]
 *   g     [B,T,Hv] (bit 0 of gate_flags clear) or [B,T,Hv,dk] (set), natural log;
 *         bit 1 of gate_flags set: the update without the delta correction
 *   beta  [B,T,Hv]
 *   S0    [B,Hv,dv,dk] or NULL (zeros); float, or double when s0_double
 *   sel_b, sel_h [nsel]: the (batch, value head) chains to run
 *   o     [nsel,T,dv] (double, out)     S_T [nsel,dv,dk] (double, out)
 *
 * A decode step is this function with T = 1.  Returns 0, or -1 on a bad
 * argument.
 */
int gdnref_recurrent(int B, int T, int Hk, int Hv, int dk, int dv,
                     int gate_flags, const float *q, const float *k,
                     const float *v, const float *g, const float *beta,
                     const void *S0, int s0_double, int nsel, const int *sel_b,
                     const int *sel_h, double *o, double *S_T, int nthreads) {
  int n, t;
  if (B <= 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return -1;
  if (Hv % Hk != 0 || nsel < 0 || !q || !k || !v || !g || !beta || !o || !S_T)
    return -1;
  for (n = 0; n < nsel; ++n)
    if (sel_b[n] < 0 || sel_b[n] >= B || sel_h[n] < 0 || sel_h[n] >= Hv)
      return -1;
  rec_job J;
  J.B = B; J.T = T; J.Hk = Hk; J.Hv = Hv; J.dk = dk; J.dv = dv;
  J.per_channel_gate = gate_flags & 1;
  J.no_delta = (gate_flags >> 1) & 1;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
  J.S0 = s0_double ? NULL : (const float *)S0;
  J.S0d = s0_double ? (const double *)S0 : NULL;
  J.nsel = nsel; J.sel_b = sel_b; J.sel_h = sel_h; J.o = o; J.S_T = S_T;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nsel) nthreads = nsel > 0 ? nsel : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  int started = 0;
  for (t = 0; th && t + 1 < nthreads; ++t)
    if (pthread_create(&th[started], NULL, rec_worker, &J) == 0) ++started;
  rec_worker(&J); /* the calling thread works too */
  for (t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Prologue: 4-tap causal depthwise conv, SiLU, optional L2 normalisation   */
/* ------------------------------------------------------------------------ */

/*
 * gdnref_conv_silu: x [B,T,H,d] -> y [B,T,H,d] (double).
 *   w [H*d][4] (tap 3 multiplies token t, tap 0 multiplies token t-3; zero
 *   history before t = 0);  y = z * sigmoid(z) with z the conv output;
 *   if l2norm, every (b,t,h) row of y is divided by sqrt(sum y^2 + eps).
 */
int gdnref_conv_silu(int B, int T, int H, int d, const float *x,
                     const float *w, int l2norm, double eps, double *y) {
  int b, t, h, c, j;
  if (B <= 0 || T < 0 || H <= 0 || d <= 0 || !x || !w || !y) return -1;
  for (b = 0; b < B; ++b)
    for (t = 0; t < T; ++t)
      for (h = 0; h < H; ++h) {
        double *yr = y + (((size_t)b * T + t) * H + h) * d;
        for (c = 0; c < d; ++c) {
          const int ch = h * d + c;
          double z = 0.0;
          for (j = 0; j < 4; ++j) {
            const int ts = t - 3 + j;
            if (ts < 0) continue;
            z += (double)w[(size_t)ch * 4 + j] *
                 (double)x[(((size_t)b * T + ts) * H + h) * d + c];
          }
          yr[c] = z / (1.0 + exp(-z));
        }
        if (l2norm) {
          double ss = 0.0;
          for (c = 0; c < d; ++c) ss += yr[c] * yr[c];
          const double inv = 1.0 / sqrt(ss + eps);
          for (c = 0; c < d; ++c) yr[c] *= inv;
        }
      }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Gated output norm after the state read                                   */
/* ------------------------------------------------------------------------ */

/*
 * gdnref_output_gate: o [rows][d] (double), z [rows][d], gain [d] -> y [rows][d].
 *   "Source notes", section "Linear attention", row gdn: the read-out of the
 *   state is RMS-normalised, multiplied by a learned gain and by a SiLU gate.
 *   "Adopt vs. port", entry burn-rmsnorm: the RMS norm divides a vector by the
 *   square root of the mean of its squares plus eps, then multiplies it by the
 *   gain, element by element.
 * One row per (batch, token, value head), normalised over its d channels; one
 * gain vector for every row; the SiLU gate is z sigmoid(z):
 *     y_c = o_c / sqrt((1/d) sum_c' o_c'^2 + eps) * gain_c * z_c / (1 + e^{-z_c})
 */
int gdnref_output_gate(long rows, int d, const double *o, const float *z,
                       const float *gain, double eps, double *y) {
  long r;
  int c;
  if (rows < 0 || d <= 0 || eps < 0.0 || !o || !z || !gain || !y) return -1;
  for (r = 0; r < rows; ++r) {
    const double *orow = o + (size_t)r * d;
    const float *zrow = z + (size_t)r * d;
    double *yrow = y + (size_t)r * d;
    double ss = 0.0;
    for (c = 0; c < d; ++c) ss += orow[c] * orow[c];
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (c = 0; c < d; ++c) {
      const double zc = (double)zrow[c];
      yrow[c] = orow[c] * inv * (double)gain[c] * (zc / (1.0 + exp(-zc)));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of the recurrence (first-order, with the state history)         */
/* ------------------------------------------------------------------------ */

/*
 * gdnref_backward: the gradients of L = sum_t <dO_t, o_t> + <dS_T, S_T> with
 * respect to every input of gdnref_recurrent, by reverse-mode
 * differentiation of its steps with the state before every token kept (the
 * first-order backward with one complete state history that "Source notes",
 * section "Linear attention", row kda, describes).  Per token t, with
 * D = alpha S_{t-1} (per-key-channel gate: S_{t-1} diag(alpha)), a = D k,
 * u = beta (v - a), S_t = D + u k^T, o_t = S_t q, and G the gradient of L
 * with respect to S_t, in reverse token order:
 *   G += dO_t q^T;   dq_t = S_t^T dO_t
 *   du = G k;   dv_t = beta du;   dbeta_t = du . (v - a)
 *   dk_t = G^T u - beta D^T du
 *   dD = G - beta du k^T
 *   dg_t = <dD, D>  (per-key-channel gate: column sums of dD o D)
 *   G <- alpha dD  (per-key-channel gate: dD diag(alpha)), the gradient for S_{t-1}
 * and dS0 = G after token 0.  dq and dk of a key head add up over its value
 * heads.  Without the delta correction (bit 1 of gate_flags, as for
 * gdnref_recurrent) a = 0: u = beta v, so the terms in beta du drop out of dk
 * and dD, and dbeta_t = du . v.
 * Inputs as for gdnref_recurrent (S0 double or NULL); dO [B,T,Hv,dv],
 * dST [B,Hv,dv,dk] or NULL; outputs double: dq, dk [B,T,Hk,dk], dv
 * [B,T,Hv,dv], dg like g, dbeta [B,T,Hv], dS0 [B,Hv,dv,dk].
 */
int gdnref_backward(int B, int T, int Hk, int Hv, int dk, int dv, int gate_flags,
                    const float *q, const float *k, const float *v, const float *g,
                    const float *beta, const double *S0, const double *dO, const double *dST,
                    double *dq, double *dkk, double *dvv, double *dg, double *dbeta,
                    double *dS0) {
  int b, h, t, i, j;
  const int per_channel_gate = gate_flags & 1, no_delta = (gate_flags >> 1) & 1;
  if (B <= 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0) return -1;
  if (!q || !k || !v || !g || !beta || !dO || !dq || !dkk || !dvv || !dg || !dbeta || !dS0) return -1;
  const size_t ss = (size_t)dv * dk;
  double *hist = (double *)malloc(sizeof(double) * ss * ((size_t)T + 1));
  double *G = (double *)malloc(sizeof(double) * ss);
  double *D = (double *)malloc(sizeof(double) * ss);
  double *St = (double *)malloc(sizeof(double) * ss);
  double *u = (double *)malloc(sizeof(double) * dv);
  double *a = (double *)malloc(sizeof(double) * dv);
  double *du = (double *)malloc(sizeof(double) * dv);
  double *al = (double *)malloc(sizeof(double) * dk);
  if (!hist || !G || !D || !St || !u || !a || !du || !al) {
    free(hist); free(G); free(D); free(St); free(u); free(a); free(du); free(al);
    return -2;
  }
  memset(dq, 0, sizeof(double) * (size_t)B * T * Hk * dk);
  memset(dkk, 0, sizeof(double) * (size_t)B * T * Hk * dk);
  for (b = 0; b < B; ++b)
    for (h = 0; h < Hv; ++h) {
      const int kh = h / (Hv / Hk);
      /* forward: hist[t] = the state before token t */
      if (S0) memcpy(hist, S0 + ((size_t)b * Hv + h) * ss, sizeof(double) * ss);
      else memset(hist, 0, sizeof(double) * ss);
      for (t = 0; t < T; ++t) {
        const size_t bt = (size_t)b * T + t;
        const float *kt = k + (bt * Hk + kh) * dk;
        const float *vt = v + (bt * Hv + h) * dv;
        const double bet = (double)beta[bt * Hv + h];
        const double *P = hist + (size_t)t * ss;
        double *N = hist + (size_t)(t + 1) * ss;
        for (j = 0; j < dk; ++j)
          al[j] = exp((double)(per_channel_gate ? g[(bt * Hv + h) * dk + j] : g[bt * Hv + h]));
        for (i = 0; i < dv; ++i) {
          double p = 0.0;
          if (!no_delta)
            for (j = 0; j < dk; ++j) p += P[(size_t)i * dk + j] * al[j] * (double)kt[j];
          const double uu = bet * ((double)vt[i] - p);
          for (j = 0; j < dk; ++j) N[(size_t)i * dk + j] = P[(size_t)i * dk + j] * al[j] + uu * (double)kt[j];
        }
      }
      /* backward */
      if (dST) memcpy(G, dST + ((size_t)b * Hv + h) * ss, sizeof(double) * ss);
      else memset(G, 0, sizeof(double) * ss);
      for (t = T - 1; t >= 0; --t) {
        const size_t bt = (size_t)b * T + t;
        const float *qt = q + (bt * Hk + kh) * dk;
        const float *kt = k + (bt * Hk + kh) * dk;
        const float *vt = v + (bt * Hv + h) * dv;
        const double *dOt = dO + (bt * Hv + h) * dv;
        const double bet = (double)beta[bt * Hv + h];
        const double *P = hist + (size_t)t * ss;
        for (j = 0; j < dk; ++j)
          al[j] = exp((double)(per_channel_gate ? g[(bt * Hv + h) * dk + j] : g[bt * Hv + h]));
        for (i = 0; i < dv; ++i) {
          double p = 0.0;
          for (j = 0; j < dk; ++j) {
            D[(size_t)i * dk + j] = P[(size_t)i * dk + j] * al[j];
            p += D[(size_t)i * dk + j] * (double)kt[j];
          }
          a[i] = no_delta ? 0.0 : p;
          u[i] = bet * ((double)vt[i] - a[i]);
          for (j = 0; j < dk; ++j) St[(size_t)i * dk + j] = D[(size_t)i * dk + j] + u[i] * (double)kt[j];
        }
        /* o_t = S_t q */
        for (i = 0; i < dv; ++i)
          for (j = 0; j < dk; ++j) G[(size_t)i * dk + j] += dOt[i] * (double)qt[j];
        double *dqt = dq + (bt * Hk + kh) * dk, *dkt = dkk + (bt * Hk + kh) * dk;
        for (j = 0; j < dk; ++j) {
          double s = 0.0;
          for (i = 0; i < dv; ++i) s += St[(size_t)i * dk + j] * dOt[i];
          dqt[j] += s;
        }
        /* S_t = D + u k^T, u = beta (v - D k) */
        double db = 0.0;
        for (i = 0; i < dv; ++i) {
          double s = 0.0;
          for (j = 0; j < dk; ++j) s += G[(size_t)i * dk + j] * (double)kt[j];
          du[i] = s;
          dvv[(bt * Hv + h) * dv + i] = bet * s;
          db += s * ((double)vt[i] - a[i]);
        }
        dbeta[bt * Hv + h] = db;
        for (j = 0; j < dk; ++j) {
          double s = 0.0;
          for (i = 0; i < dv; ++i)
            s += G[(size_t)i * dk + j] * u[i] - (no_delta ? 0.0 : bet * du[i] * D[(size_t)i * dk + j]);
          dkt[j] += s;
        }
        /* dD, the decay's gradient, then the gradient for S_{t-1} */
        double dgh = 0.0;
        for (j = 0; j < dk; ++j) {
          double colsum = 0.0;
          for (i = 0; i < dv; ++i) {
            const double dd = G[(size_t)i * dk + j] - (no_delta ? 0.0 : bet * du[i] * (double)kt[j]);
            colsum += dd * D[(size_t)i * dk + j];
            G[(size_t)i * dk + j] = dd * al[j];
          }
          if (per_channel_gate) dg[(bt * Hv + h) * dk + j] = colsum;
          else dgh += colsum;
        }
        if (!per_channel_gate) dg[bt * Hv + h] = dgh;
      }
      memcpy(dS0 + ((size_t)b * Hv + h) * ss, G, sizeof(double) * ss);
    }
  free(hist); free(G); free(D); free(St); free(u); free(a); free(du); free(al);
  return 0;
}
