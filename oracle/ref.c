/*
 * Float64 CPU oracle loops -- TEST INFRASTRUCTURE ONLY.
 *
 * The same definitions as oracle/scan.py, oracle/attn.py, oracle/gla.py and
 * oracle/sscan.py, written as plain
 * sequential loops in C so that full-size samples and the CPU baseline run in
 * seconds.  OpenMP spreads independent units (channels, heads) over the host
 * cores; each unit runs strictly in time order.  Nothing in the GPU library
 * includes or links this file, and this file includes nothing of it.
 *
 * Inputs are the exact device inputs: fp32 values and bf16 bit patterns, upcast
 * to double before any arithmetic.  All arithmetic and all outputs are double.
 *
 * Citations (page title, then section):
 *   ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
 *   LA2 = "Lightning Attention-2: A Free Lunch for Handling Unlimited Sequence
 *         Lengths in Large Language Models" (paper-graph-ui summary)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Diagonal recurrence, forward.  ZTF "The scan for one number of state":
 * h_t = a_t h_{t-1} + b_t from h_0 (zero when h0 is NULL).
 * a, b: [B, T, D] fp32; h0: [B, D] fp32 or NULL.
 * Computes the block of channels b in [b0, b1), d in [d0, d1):
 * h: [b1-b0, T, d1-d0] double, hT: [b1-b0, d1-d0] double.
 */
void oracle_scan_fwd(const float *a, const float *b, const float *h0, double *h,
                     double *hT, int64_t B, int64_t T, int64_t D, int64_t b0,
                     int64_t b1, int64_t d0, int64_t d1) {
  int64_t nb = b1 - b0, nd = d1 - d0;
  (void)B;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t ib = 0; ib < nb; ++ib) {
    for (int64_t id = 0; id < nd; ++id) {
      int64_t bb = b0 + ib, dd = d0 + id;
      double s = h0 ? (double)h0[bb * D + dd] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        int64_t src = (bb * T + t) * D + dd;
        s = (double)a[src] * s + (double)b[src];
        h[(ib * T + t) * nd + id] = s;
      }
      hT[ib * nd + id] = s;
    }
  }
}

/*
 * Diagonal recurrence, backward.  ZTF "The backward pass is a scan in
 * reverse": hbar_T = g_T + dh_T, hbar_t = g_t + a_{t+1} hbar_{t+1};
 * db_t = hbar_t, da_t = hbar_t h_{t-1} (h_0 at t = 1), dh0 = a_1 hbar_1.
 * a, h (forward output), dh: [B, T, D] fp32; h0, dhT: [B, D] fp32 or NULL.
 * Outputs for the channel block: da, db [nb, T, nd], dh0 [nb, nd], double.
 */
void oracle_scan_bwd(const float *a, const float *h, const float *h0,
                     const float *dh, const float *dhT, double *da, double *db,
                     double *dh0, int64_t B, int64_t T, int64_t D, int64_t b0,
                     int64_t b1, int64_t d0, int64_t d1) {
  int64_t nb = b1 - b0, nd = d1 - d0;
  (void)B;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t ib = 0; ib < nb; ++ib) {
    for (int64_t id = 0; id < nd; ++id) {
      int64_t bb = b0 + ib, dd = d0 + id;
      double hbar = dhT ? (double)dhT[bb * D + dd] : 0.0;
      for (int64_t t = T - 1; t >= 0; --t) {
        int64_t src = (bb * T + t) * D + dd;
        if (t < T - 1) hbar *= (double)a[src + D];
        hbar += (double)dh[src];
        double hprev = t > 0 ? (double)h[src - D] : (h0 ? (double)h0[bb * D + dd] : 0.0);
        db[(ib * T + t) * nd + id] = hbar;
        da[(ib * T + t) * nd + id] = hbar * hprev;
      }
      dh0[ib * nd + id] = T > 0 ? (double)a[(bb * T) * D + dd] * hbar : hbar;
    }
  }
}

/*
 * Matrix-state recurrence, forward, for a list of heads.  ZTF "The chunkwise
 * algorithm" (the recurrence it is derived for) and "Scans over vector and
 * matrix states": S_t = a_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, a_t =
 * exp(l_t).
 * q, k: [B, H, T, DK] bf16 bits; v: [B, H, T, DV] bf16 bits; l: [B, H, T]
 * fp32; S0: [B, H, DK, DV] fp32 or NULL.  heads: flat indices b*H + h.
 * Outputs: o [nheads, T, DV], ST [nheads, DK, DV], double.
 */
void oracle_la_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const float *l, const float *S0, double *o, double *ST,
                   int64_t T, int64_t DK, int64_t DV, const int64_t *heads,
                   int64_t nheads) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nheads; ++i) {
    int64_t hd = heads[i];
    const uint16_t *qh = q + hd * T * DK, *kh = k + hd * T * DK, *vh = v + hd * T * DV;
    const float *lh = l + hd * T;
    double *S = (double *)malloc(sizeof(double) * DK * DV);
    double *kt = (double *)malloc(sizeof(double) * (DK + DV + DK));
    double *vt = kt + DK, *qt = vt + DV;
    for (int64_t e = 0; e < DK * DV; ++e) S[e] = S0 ? (double)S0[hd * DK * DV + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      double at = exp((double)lh[t]);
      for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
      for (int64_t x = 0; x < DK; ++x) qt[x] = bf16_to_double(qh[t * DK + x]);
      for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
      for (int64_t x = 0; x < DK; ++x)
        for (int64_t y = 0; y < DV; ++y) S[x * DV + y] = at * S[x * DV + y] + kt[x] * vt[y];
      double *ot = o + (i * T + t) * DV;
      for (int64_t y = 0; y < DV; ++y) ot[y] = 0.0;
      for (int64_t x = 0; x < DK; ++x)
        for (int64_t y = 0; y < DV; ++y) ot[y] += S[x * DV + y] * qt[x];
    }
    memcpy(ST + i * DK * DV, S, sizeof(double) * DK * DV);
    free(kt);
    free(S);
  }
}

/*
 * Matrix-state recurrence, backward, for a list of heads.  ZTF "The backward
 * pass of linear attention": Sbar_T = q_T dO_T^T + dS_T,
 * Sbar_t = q_t dO_t^T + a_{t+1} Sbar_{t+1}; dq_t = S_t dO_t,
 * dk_t = Sbar_t v_t, dv_t = Sbar_t^T k_t, dl_t = a_t <Sbar_t, S_{t-1}>,
 * dS0 = a_1 Sbar_1.  The states S_{t-1}, S_t are recomputed in the reverse
 * sweep from checkpoints stored every CK steps of a first forward loop
 * (ZTF "The backward pass is a scan in reverse": chunked kernels store only
 * boundary states and recompute the rest; here it only bounds memory).
 * dO: [B, H, T, DV] bf16 bits; dST: [B, H, DK, DV] fp32 or NULL.
 * Outputs: dq, dk [nheads, T, DK]; dv [nheads, T, DV]; dl [nheads, T];
 * dS0 [nheads, DK, DV]; double.
 */
void oracle_la_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const float *l, const float *S0, const uint16_t *dO,
                   const float *dST, double *dq, double *dk, double *dv,
                   double *dl, double *dS0, int64_t T, int64_t DK, int64_t DV,
                   const int64_t *heads, int64_t nheads) {
  const int64_t CK = 64;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nheads; ++i) {
    int64_t hd = heads[i];
    const uint16_t *qh = q + hd * T * DK, *kh = k + hd * T * DK, *vh = v + hd * T * DV;
    const uint16_t *doh = dO + hd * T * DV;
    const float *lh = l + hd * T;
    int64_t SZ = DK * DV;
    int64_t ncp = T / CK + 1;
    /* checkpoints: cp[c] = S_{c*CK} */
    double *cp = (double *)malloc(sizeof(double) * SZ * ncp);
    /* states of one block: blk[j] = S_{t0 + j}, j = 0..CK */
    double *blk = (double *)malloc(sizeof(double) * SZ * (CK + 1));
    double *Sb = (double *)malloc(sizeof(double) * SZ);
    double *tmp = (double *)malloc(sizeof(double) * (2 * DK + 2 * DV));
    double *kt = tmp, *qt = tmp + DK, *vt = tmp + 2 * DK, *dot = tmp + 2 * DK + DV;
    double *S = blk; /* scratch for the first forward loop */
    for (int64_t e = 0; e < SZ; ++e) S[e] = S0 ? (double)S0[hd * SZ + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      if (t % CK == 0) memcpy(cp + (t / CK) * SZ, S, sizeof(double) * SZ);
      double at = exp((double)lh[t]);
      for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
      for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
      for (int64_t x = 0; x < DK; ++x)
        for (int64_t y = 0; y < DV; ++y) S[x * DV + y] = at * S[x * DV + y] + kt[x] * vt[y];
    }
    for (int64_t e = 0; e < SZ; ++e) Sb[e] = dST ? (double)dST[hd * SZ + e] : 0.0;
    int64_t nblk = (T + CK - 1) / CK;
    for (int64_t c = nblk - 1; c >= 0; --c) {
      int64_t t0 = c * CK, n = (T - t0 < CK) ? T - t0 : CK;
      memcpy(blk, cp + c * SZ, sizeof(double) * SZ);
      for (int64_t j = 0; j < n; ++j) {
        int64_t t = t0 + j;
        double at = exp((double)lh[t]);
        for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
        for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
        const double *Sp = blk + j * SZ;
        double *Sn = blk + (j + 1) * SZ;
        for (int64_t x = 0; x < DK; ++x)
          for (int64_t y = 0; y < DV; ++y) Sn[x * DV + y] = at * Sp[x * DV + y] + kt[x] * vt[y];
      }
      for (int64_t j = n - 1; j >= 0; --j) {
        int64_t t = t0 + j;
        if (t < T - 1) {
          double an = exp((double)lh[t + 1]);
          for (int64_t e = 0; e < SZ; ++e) Sb[e] *= an;
        }
        for (int64_t x = 0; x < DK; ++x) qt[x] = bf16_to_double(qh[t * DK + x]);
        for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
        for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
        for (int64_t y = 0; y < DV; ++y) dot[y] = bf16_to_double(doh[t * DV + y]);
        for (int64_t x = 0; x < DK; ++x)
          for (int64_t y = 0; y < DV; ++y) Sb[x * DV + y] += qt[x] * dot[y];
        const double *Sprev = blk + j * SZ, *Scur = blk + (j + 1) * SZ;
        double *gq = dq + (i * T + t) * DK, *gk = dk + (i * T + t) * DK;
        double *gv = dv + (i * T + t) * DV;
        for (int64_t x = 0; x < DK; ++x) {
          double sq = 0.0, sk = 0.0;
          for (int64_t y = 0; y < DV; ++y) {
            sq += Scur[x * DV + y] * dot[y];
            sk += Sb[x * DV + y] * vt[y];
          }
          gq[x] = sq;
          gk[x] = sk;
        }
        for (int64_t y = 0; y < DV; ++y) gv[y] = 0.0;
        for (int64_t x = 0; x < DK; ++x)
          for (int64_t y = 0; y < DV; ++y) gv[y] += Sb[x * DV + y] * kt[x];
        double inner = 0.0;
        for (int64_t e = 0; e < SZ; ++e) inner += Sb[e] * Sprev[e];
        dl[i * T + t] = exp((double)lh[t]) * inner;
      }
    }
    double a1 = T > 0 ? exp((double)lh[0]) : 1.0;
    for (int64_t e = 0; e < SZ; ++e) dS0[i * SZ + e] = a1 * Sb[e];
    free(tmp);
    free(Sb);
    free(blk);
    free(cp);
  }
}

/*
 * Matrix-state recurrence with one decay per key dimension (gated linear
 * attention), forward, for a list of heads.  ZTF "Scans over vector and
 * matrix states" (the diagonal transition) and "The chunkwise algorithm" (the
 * GLA form S_t = G_t (.) S_{t-1} + k_t^T v_t): row x of the state decays by
 * a_t[x] = exp(l_t[x]), then o_t = S_t^T q_t.
 * l: [B, H, T, DK] fp32.  Other arguments as oracle_la_fwd.
 */
void oracle_gla_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *l, const float *S0, double *o, double *ST,
                    int64_t T, int64_t DK, int64_t DV, const int64_t *heads,
                    int64_t nheads) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nheads; ++i) {
    int64_t hd = heads[i];
    const uint16_t *qh = q + hd * T * DK, *kh = k + hd * T * DK, *vh = v + hd * T * DV;
    const float *lh = l + hd * T * DK;
    double *S = (double *)malloc(sizeof(double) * DK * DV);
    double *kt = (double *)malloc(sizeof(double) * (DK + DV + DK + DK));
    double *vt = kt + DK, *qt = vt + DV, *at = qt + DK;
    for (int64_t e = 0; e < DK * DV; ++e) S[e] = S0 ? (double)S0[hd * DK * DV + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t x = 0; x < DK; ++x) at[x] = exp((double)lh[t * DK + x]);
      for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
      for (int64_t x = 0; x < DK; ++x) qt[x] = bf16_to_double(qh[t * DK + x]);
      for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
      for (int64_t x = 0; x < DK; ++x)
        for (int64_t y = 0; y < DV; ++y) S[x * DV + y] = at[x] * S[x * DV + y] + kt[x] * vt[y];
      double *ot = o + (i * T + t) * DV;
      for (int64_t y = 0; y < DV; ++y) ot[y] = 0.0;
      for (int64_t x = 0; x < DK; ++x)
        for (int64_t y = 0; y < DV; ++y) ot[y] += S[x * DV + y] * qt[x];
    }
    memcpy(ST + i * DK * DV, S, sizeof(double) * DK * DV);
    free(kt);
    free(S);
  }
}

/*
 * The same recurrence, backward (ZTF "The backward pass of linear attention"
 * with the diagonal decay): Sbar_T = q_T dO_T^T + dS_T,
 * Sbar_t = q_t dO_t^T + diag(a_{t+1}) Sbar_{t+1}; dq_t = S_t dO_t,
 * dk_t = Sbar_t v_t, dv_t = Sbar_t^T k_t,
 * dl_t[x] = a_t[x] <Sbar_t[x, :], S_{t-1}[x, :]>, dS0 = diag(a_1) Sbar_1.
 * States are recomputed from checkpoints every CK steps, as in oracle_la_bwd.
 * Outputs: dq, dk, dl [nheads, T, DK]; dv [nheads, T, DV]; dS0 [nheads, DK, DV].
 */
void oracle_gla_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *l, const float *S0, const uint16_t *dO,
                    const float *dST, double *dq, double *dk, double *dv,
                    double *dl, double *dS0, int64_t T, int64_t DK, int64_t DV,
                    const int64_t *heads, int64_t nheads) {
  const int64_t CK = 64;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nheads; ++i) {
    int64_t hd = heads[i];
    const uint16_t *qh = q + hd * T * DK, *kh = k + hd * T * DK, *vh = v + hd * T * DV;
    const uint16_t *doh = dO + hd * T * DV;
    const float *lh = l + hd * T * DK;
    int64_t SZ = DK * DV;
    int64_t ncp = T / CK + 1;
    double *cp = (double *)malloc(sizeof(double) * SZ * ncp);
    double *blk = (double *)malloc(sizeof(double) * SZ * (CK + 1));
    double *Sb = (double *)malloc(sizeof(double) * SZ);
    double *tmp = (double *)malloc(sizeof(double) * (3 * DK + 2 * DV));
    double *kt = tmp, *qt = tmp + DK, *at = tmp + 2 * DK, *vt = tmp + 3 * DK,
           *dot = tmp + 3 * DK + DV;
    double *S = blk;
    for (int64_t e = 0; e < SZ; ++e) S[e] = S0 ? (double)S0[hd * SZ + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      if (t % CK == 0) memcpy(cp + (t / CK) * SZ, S, sizeof(double) * SZ);
      for (int64_t x = 0; x < DK; ++x) at[x] = exp((double)lh[t * DK + x]);
      for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
      for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
      for (int64_t x = 0; x < DK; ++x)
        for (int64_t y = 0; y < DV; ++y) S[x * DV + y] = at[x] * S[x * DV + y] + kt[x] * vt[y];
    }
    for (int64_t e = 0; e < SZ; ++e) Sb[e] = dST ? (double)dST[hd * SZ + e] : 0.0;
    int64_t nblk = (T + CK - 1) / CK;
    for (int64_t c = nblk - 1; c >= 0; --c) {
      int64_t t0 = c * CK, n = (T - t0 < CK) ? T - t0 : CK;
      memcpy(blk, cp + c * SZ, sizeof(double) * SZ);
      for (int64_t j = 0; j < n; ++j) {
        int64_t t = t0 + j;
        for (int64_t x = 0; x < DK; ++x) at[x] = exp((double)lh[t * DK + x]);
        for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
        for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
        const double *Sp = blk + j * SZ;
        double *Sn = blk + (j + 1) * SZ;
        for (int64_t x = 0; x < DK; ++x)
          for (int64_t y = 0; y < DV; ++y)
            Sn[x * DV + y] = at[x] * Sp[x * DV + y] + kt[x] * vt[y];
      }
      for (int64_t j = n - 1; j >= 0; --j) {
        int64_t t = t0 + j;
        if (t < T - 1) {
          for (int64_t x = 0; x < DK; ++x) {
            double an = exp((double)lh[(t + 1) * DK + x]);
            for (int64_t y = 0; y < DV; ++y) Sb[x * DV + y] *= an;
          }
        }
        for (int64_t x = 0; x < DK; ++x) qt[x] = bf16_to_double(qh[t * DK + x]);
        for (int64_t x = 0; x < DK; ++x) kt[x] = bf16_to_double(kh[t * DK + x]);
        for (int64_t y = 0; y < DV; ++y) vt[y] = bf16_to_double(vh[t * DV + y]);
        for (int64_t y = 0; y < DV; ++y) dot[y] = bf16_to_double(doh[t * DV + y]);
        for (int64_t x = 0; x < DK; ++x)
          for (int64_t y = 0; y < DV; ++y) Sb[x * DV + y] += qt[x] * dot[y];
        const double *Sprev = blk + j * SZ, *Scur = blk + (j + 1) * SZ;
        double *gq = dq + (i * T + t) * DK, *gk = dk + (i * T + t) * DK;
        double *gv = dv + (i * T + t) * DV, *gl = dl + (i * T + t) * DK;
        for (int64_t x = 0; x < DK; ++x) {
          double sq = 0.0, sk = 0.0, sl = 0.0;
          for (int64_t y = 0; y < DV; ++y) {
            sq += Scur[x * DV + y] * dot[y];
            sk += Sb[x * DV + y] * vt[y];
            sl += Sb[x * DV + y] * Sprev[x * DV + y];
          }
          gq[x] = sq;
          gk[x] = sk;
          gl[x] = exp((double)lh[t * DK + x]) * sl;
        }
        for (int64_t y = 0; y < DV; ++y) gv[y] = 0.0;
        for (int64_t x = 0; x < DK; ++x)
          for (int64_t y = 0; y < DV; ++y) gv[y] += Sb[x * DV + y] * kt[x];
      }
    }
    for (int64_t x = 0; x < DK; ++x) {
      double a1 = T > 0 ? exp((double)lh[x]) : 1.0;
      for (int64_t y = 0; y < DV; ++y) dS0[i * SZ + x * DV + y] = a1 * Sb[x * DV + y];
    }
    free(tmp);
    free(Sb);
    free(blk);
    free(cp);
  }
}

/* ------------------------------------------------------------------------
 * Selective scan with N state entries per channel (Mamba-1's recurrence):
 *   a_t[d,n] = exp(delta_t[d] A[d,n]),  b_t[d,n] = delta_t[d] B_t[n] x_t[d],
 *   h_t = a_t h_{t-1} + b_t,  y_t[d] = sum_n C_t[n] h_t[d,n]
 * (ZTF "Scans over vector and matrix states"; "What limits a recurrent
 * layer" for the decay exp(delta A)).  Layouts: x, delta, dy [Bt, T, D];
 * A [D, N]; B, C [Bt, T, N]; h0, dhT [Bt, D, N].  chans lists the (batch,
 * channel) units to run, as b * D + d; per-unit outputs are indexed by the
 * position in that list.
 * ------------------------------------------------------------------------ */

void oracle_sscan_fwd(const float *x, const float *delta, const float *A, const float *Bm,
                      const float *Cm, const float *h0, int64_t Bt, int64_t T, int64_t D,
                      int64_t N, const int64_t *chans, int64_t nch, double *y, double *hT) {
  (void)Bt;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t b = chans[c] / D, d = chans[c] % D;
    double *h = (double *)malloc(sizeof(double) * (size_t)N);
    for (int64_t n = 0; n < N; ++n) h[n] = h0 ? (double)h0[(b * D + d) * N + n] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double dl = delta[(b * T + t) * D + d], xv = x[(b * T + t) * D + d];
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double a = exp(dl * (double)A[d * N + n]);
        h[n] = a * h[n] + dl * (double)Bm[(b * T + t) * N + n] * xv;
        acc += (double)Cm[(b * T + t) * N + n] * h[n];
      }
      y[c * T + t] = acc;
    }
    for (int64_t n = 0; n < N; ++n) hT[c * N + n] = h[n];
    free(h);
  }
}

/* Backward: the reverse-time adjoint per entry, hbar_t = C_t dy_t + a_{t+1}
 * hbar_{t+1} (+ dhT at the end), dL/da_t = hbar_t h_{t-1}, dL/db_t = hbar_t,
 * dh0 = a_1 hbar_1 (ZTF "The backward pass is a scan in reverse"), then the
 * chain rule through a = exp(delta A) and b = delta B x.  Per unit: dx,
 * ddelta [nch, T], dA [nch, N] (this unit's sum over t), dh0 [nch, N].  dB and
 * dC [Bt, T, N] receive the sums over the listed units (they are zeroed
 * here first). */
void oracle_sscan_bwd(const float *x, const float *delta, const float *A, const float *Bm,
                      const float *Cm, const float *h0, const float *dy, const float *dhT,
                      int64_t Bt, int64_t T, int64_t D, int64_t N, const int64_t *chans,
                      int64_t nch, double *dx, double *ddelta, double *dA, double *dB,
                      double *dC, double *dh0) {
  const size_t nbtn = (size_t)(Bt * T * N);
  memset(dB, 0, sizeof(double) * nbtn);
  memset(dC, 0, sizeof(double) * nbtn);
#pragma omp parallel
  {
    double *pB = (double *)calloc(nbtn, sizeof(double));
    double *pC = (double *)calloc(nbtn, sizeof(double));
    double *hs = (double *)malloc(sizeof(double) * (size_t)((T + 1) * N));
    double *hbar = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < nch; ++c) {
      const int64_t b = chans[c] / D, d = chans[c] % D;
      /* hs[t] = h_{t-1} for t = 0..T (hs[0] = h0, hs[T] = h_T) */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? (double)h0[(b * D + d) * N + n] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const double dl = delta[(b * T + t) * D + d], xv = x[(b * T + t) * D + d];
        for (int64_t n = 0; n < N; ++n) {
          const double a = exp(dl * (double)A[d * N + n]);
          hs[(t + 1) * N + n] = a * hs[t * N + n] + dl * (double)Bm[(b * T + t) * N + n] * xv;
        }
      }
      for (int64_t n = 0; n < N; ++n) {
        hbar[n] = dhT ? (double)dhT[(b * D + d) * N + n] : 0.0;
        dA[c * N + n] = 0.0;
      }
      for (int64_t t = T - 1; t >= 0; --t) {
        const double dl = delta[(b * T + t) * D + d], xv = x[(b * T + t) * D + d];
        const double g = dy[(b * T + t) * D + d];
        const double dl_next = t + 1 < T ? delta[(b * T + t + 1) * D + d] : 0.0;
        double dd = 0.0, sb = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double An = A[d * N + n];
          if (t + 1 < T) hbar[n] *= exp(dl_next * An);
          hbar[n] += (double)Cm[(b * T + t) * N + n] * g;
          const double a = exp(dl * An);
          const double da = hbar[n] * hs[t * N + n];
          dd += da * a * An;
          dA[c * N + n] += da * a * dl;
          sb += hbar[n] * (double)Bm[(b * T + t) * N + n];
          pB[(b * T + t) * N + n] += hbar[n] * dl * xv;
          pC[(b * T + t) * N + n] += g * hs[(t + 1) * N + n];
        }
        ddelta[c * T + t] = dd + sb * xv;
        dx[c * T + t] = dl * sb;
      }
      for (int64_t n = 0; n < N; ++n) {
        const double a1 = T > 0 ? exp((double)delta[(b * T) * D + d] * (double)A[d * N + n]) : 1.0;
        dh0[c * N + n] = a1 * hbar[n];
      }
    }
#pragma omp critical
    {
      for (size_t i = 0; i < nbtn; ++i) {
        dB[i] += pB[i];
        dC[i] += pC[i];
      }
    }
    free(pB);
    free(pC);
    free(hs);
    free(hbar);
  }
}
