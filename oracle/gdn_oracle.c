/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; it exists so that tests, the smoke check and the benchmark's
 * CPU-baseline leg can compare the HIP kernels against an obviously correct
 * definition.  It shares no code, header or constant with the HIP library.
 *
 * What it computes.  The pages ("Qwen's FlashQLA targets the expensive bit of
 * long-context AI", section "What happened"; "FlashQLA resource", section 2
 * "What It Actually Is") name the operator -- the forward and backward pass of
 * Gated DeltaNet (GDN) chunked prefill -- but print no formula.  The oracle
 * therefore runs the published gated delta rule itself, token by token:
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * with S a dv x dk matrix.  The state is imported/exported as h = S^T
 * ([dk][dv], row-major), the layout the chunked form keeps on the GPU.
 * "FlashQLA resource", section 3, says the chunked reformulation loses no
 * numerical precision, so this plain recurrence *is* the reference result.
 *
 * Layout (token-major, one packed stream):
 *   q, k  [Ttot][H][Dk], v, o [Ttot][H][Dv], g, beta [Ttot][H]
 *   sequence n occupies tokens cu[n] .. cu[n+1]-1; the state restarts at every
 *   sequence start from h0[n] (or zero when h0 == NULL).
 *   h0, hT, dhT, dh0  [N][H][Dk][Dv]
 *
 * Backward: reverse-mode differentiation of the recurrence above (BPTT).  The
 * states of one sequence are checkpointed every CKPT tokens and recomputed one
 * block at a time.  With dS = dL/dS_t, S' = S_{t-1}, a = exp(g_t):
 *   dq_t  = scale * S_t^T do_t            (after dS += scale * do_t q_t^T)
 *   dv_t  = beta * dS k
 *   dbeta = (dS k) . (v - a S' k)
 *   dk_t  = beta * dS^T v - a beta (dS^T S' + S'^T dS) k
 *   dg_t  = a * <dS, S' (I - beta k k^T)>
 *   dS_{t-1} = a * dS (I - beta k k^T)
 * and dh0 = (dS at the sequence start)^T.
 *
 * Parallelism: OpenMP over (sequence, head) pairs, nothing else.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

static size_t tok3(int64_t t, int h, int H, int D) { return ((size_t)t * H + h) * D; }

/* S (dv x dk) <- exp(g) * S * (I - beta k k^T) + beta v k^T ; p = S_old k is scratch (dv). */
static void step(double *S, int Dk, int Dv, const double *k, const double *v,
                 double g, double beta, double *p) {
  double a = exp(g);
  for (int i = 0; i < Dv; ++i) {
    double s = 0.0;
    for (int j = 0; j < Dk; ++j) s += S[i * Dk + j] * k[j];
    p[i] = s;
  }
  for (int i = 0; i < Dv; ++i)
    for (int j = 0; j < Dk; ++j)
      S[i * Dk + j] = a * (S[i * Dk + j] - beta * p[i] * k[j]) + beta * v[i] * k[j];
}

static void load_state(double *S, const double *h, int Dk, int Dv) {
  /* S[i][j] = h[j][i] */
  for (int i = 0; i < Dv; ++i)
    for (int j = 0; j < Dk; ++j) S[i * Dk + j] = h ? h[(size_t)j * Dv + i] : 0.0;
}

static void store_state(double *h, const double *S, int Dk, int Dv) {
  for (int i = 0; i < Dv; ++i)
    for (int j = 0; j < Dk; ++j) h[(size_t)j * Dv + i] = S[i * Dk + j];
}

int gdn_oracle_fwd(int N, const int64_t *cu, int H, int Dk, int Dv,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *h0,
                   double scale, double *o, double *hT) {
  int ok = 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int nh = 0; nh < N * H; ++nh) {
    int n = nh / H, h = nh % H;
    double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
    double *p = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!S || !p) { ok = 0; free(S); free(p); continue; }
    load_state(S, h0 ? h0 + (size_t)nh * Dk * Dv : NULL, Dk, Dv);
    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      const double *kt = k + tok3(t, h, H, Dk), *qt = q + tok3(t, h, H, Dk);
      const double *vt = v + tok3(t, h, H, Dv);
      size_t s1 = (size_t)t * H + h;
      step(S, Dk, Dv, kt, vt, g[s1], beta[s1], p);
      double *ot = o + tok3(t, h, H, Dv);
      for (int i = 0; i < Dv; ++i) {
        double s = 0.0;
        for (int j = 0; j < Dk; ++j) s += S[i * Dk + j] * qt[j];
        ot[i] = scale * s;
      }
    }
    if (hT) store_state(hT + (size_t)nh * Dk * Dv, S, Dk, Dv);
    free(S);
    free(p);
  }
  return ok ? 0 : 1;
}

int gdn_oracle_bwd(int N, const int64_t *cu, int H, int Dk, int Dv,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *h0,
                   double scale, const double *dout, const double *dhT,
                   double *dq, double *dk, double *dv, double *dg,
                   double *dbeta, double *dh0) {
  int ok = 1;
  size_t SS = (size_t)Dk * Dv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int nh = 0; nh < N * H; ++nh) {
    int n = nh / H, h = nh % H;
    int64_t t0 = cu[n], L = cu[n + 1] - cu[n];
    int64_t nblk = (L + CKPT - 1) / CKPT;
    /* ck[b] = state before token t0 + b*CKPT; blk[i] = state after token i of a block */
    double *ck = (double *)malloc(sizeof(double) * SS * (size_t)(nblk + 1));
    double *blk = (double *)malloc(sizeof(double) * SS * (CKPT + 1));
    double *dS = (double *)malloc(sizeof(double) * SS);
    double *p = (double *)malloc(sizeof(double) * (size_t)(Dv > Dk ? Dv : Dk) * 4);
    if (!ck || !blk || !dS || !p) { ok = 0; free(ck); free(blk); free(dS); free(p); continue; }
    double *Sk = p, *dSk = p + Dv, *dSTv = p + 2 * Dv; /* Dv, Dv, Dk */
    double *tmp = p + 2 * Dv + Dk;                       /* Dk */

    load_state(ck, h0 ? h0 + (size_t)nh * SS : NULL, Dk, Dv);
    for (int64_t b = 0; b < nblk; ++b) {
      memcpy(ck + (size_t)(b + 1) * SS, ck + (size_t)b * SS, sizeof(double) * SS);
      int64_t e = (b + 1) * CKPT < L ? (b + 1) * CKPT : L;
      for (int64_t t = t0 + b * CKPT; t < t0 + e; ++t) {
        size_t s1 = (size_t)t * H + h;
        step(ck + (size_t)(b + 1) * SS, Dk, Dv, k + tok3(t, h, H, Dk),
             v + tok3(t, h, H, Dv), g[s1], beta[s1], Sk);
      }
    }
    if (dhT) load_state(dS, dhT + (size_t)nh * SS, Dk, Dv);
    else memset(dS, 0, sizeof(double) * SS);

    for (int64_t b = nblk - 1; b >= 0; --b) {
      int64_t tb = t0 + b * CKPT;
      int64_t e = (b + 1) * CKPT < L ? (b + 1) * CKPT : L;
      int nb = (int)(e - b * CKPT);
      memcpy(blk, ck + (size_t)b * SS, sizeof(double) * SS);
      for (int i = 0; i < nb; ++i) {
        memcpy(blk + (size_t)(i + 1) * SS, blk + (size_t)i * SS, sizeof(double) * SS);
        size_t s1 = (size_t)(tb + i) * H + h;
        step(blk + (size_t)(i + 1) * SS, Dk, Dv, k + tok3(tb + i, h, H, Dk),
             v + tok3(tb + i, h, H, Dv), g[s1], beta[s1], Sk);
      }
      for (int i = nb - 1; i >= 0; --i) {
        int64_t t = tb + i;
        size_t s1 = (size_t)t * H + h;
        const double *St = blk + (size_t)(i + 1) * SS, *Sp = blk + (size_t)i * SS;
        const double *qt = q + tok3(t, h, H, Dk), *kt = k + tok3(t, h, H, Dk);
        const double *vt = v + tok3(t, h, H, Dv), *dot = dout + tok3(t, h, H, Dv);
        double a = exp(g[s1]), bt = beta[s1];
        /* output term */
        for (int r = 0; r < Dv; ++r)
          for (int c = 0; c < Dk; ++c) dS[r * Dk + c] += scale * dot[r] * qt[c];
        double *dqt = dq + tok3(t, h, H, Dk);
        for (int c = 0; c < Dk; ++c) {
          double s = 0.0;
          for (int r = 0; r < Dv; ++r) s += St[r * Dk + c] * dot[r];
          dqt[c] = scale * s;
        }
        /* Sk = S' k, dSk = dS k, dSTv = dS^T v */
        for (int r = 0; r < Dv; ++r) {
          double s1v = 0.0, s2 = 0.0;
          for (int c = 0; c < Dk; ++c) { s1v += Sp[r * Dk + c] * kt[c]; s2 += dS[r * Dk + c] * kt[c]; }
          Sk[r] = s1v;
          dSk[r] = s2;
        }
        for (int c = 0; c < Dk; ++c) {
          double s = 0.0;
          for (int r = 0; r < Dv; ++r) s += dS[r * Dk + c] * vt[r];
          dSTv[c] = s;
        }
        double *dvt = dv + tok3(t, h, H, Dv);
        double db = 0.0;
        for (int r = 0; r < Dv; ++r) {
          dvt[r] = bt * dSk[r];
          db += dSk[r] * (vt[r] - a * Sk[r]);
        }
        dbeta[s1] = db;
        /* (dS^T S' + S'^T dS) k = dS^T (S' k) + S'^T (dS k) */
        double *dkt = dk + tok3(t, h, H, Dk);
        for (int c = 0; c < Dk; ++c) {
          double s = 0.0;
          for (int r = 0; r < Dv; ++r) s += dS[r * Dk + c] * Sk[r] + Sp[r * Dk + c] * dSk[r];
          tmp[c] = s;
          dkt[c] = bt * dSTv[c] - a * bt * s;
        }
        /* dg = a <dS, S'(I - b k k^T)> = a (<dS, S'> - b (dS k).(S' k)) */
        double inner = 0.0, cross = 0.0;
        for (size_t e2 = 0; e2 < SS; ++e2) inner += dS[e2] * Sp[e2];
        for (int r = 0; r < Dv; ++r) cross += dSk[r] * Sk[r];
        dg[s1] = a * (inner - bt * cross);
        /* dS <- a dS (I - b k k^T) */
        for (int r = 0; r < Dv; ++r)
          for (int c = 0; c < Dk; ++c) dS[r * Dk + c] = a * (dS[r * Dk + c] - bt * dSk[r] * kt[c]);
      }
    }
    if (dh0) store_state(dh0 + (size_t)nh * SS, dS, Dk, Dv);
    free(ck);
    free(blk);
    free(dS);
    free(p);
  }
  return ok ? 0 : 1;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of OpenMP threads the oracle's parallel loops will use. */
int gdn_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
