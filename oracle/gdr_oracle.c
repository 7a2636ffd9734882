/*
 * gdr_oracle.c -- plain fp64 CPU oracle of the channel-wise gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP implementation, and the HIP
 * implementation never calls it.
 *
 * What it computes (one independent stream = one (batch, head) pair, run
 * token by token in double precision on the exact stored input values):
 *
 *   pre-pass   (Kimi3 = GPT2 x 22580 blog, hubwiz translation, section 3
 *               "DeltaNet", forward(): SiLU then L2-normalise q and k;
 *               Muir reading notes (arXiv:2611.08376), section 2.1: q and k
 *               per head SiLU + l2, v left as is)
 *       qh = SiLU(q_t) / max(|SiLU(q_t)|, 1e-12)
 *       kn = SiLU(k_t) / max(|SiLU(k_t)|, 1e-12)
 *     the 1e-12 floor is the default epsilon of the F.normalize call the
 *     blog's forward() prints.  normalize_qk = 0 skips both.
 *
 *   read-out gain (Muir notes, section 2.1, the Muir read-out): the query
 *     only is scaled by a static per-channel profile gamma and a dynamic
 *     2*sigmoid(z_t) in (0, 2):
 *       qt = scale * gamma (.) 2 sigma(z_t) (.) qh
 *
 *   GDN-2 update (Muir notes, section 2.1): with row vectors k, q in R^dk,
 *     v in R^dv and the state S in R^{dk x dv} (rows = key channels),
 *       S_hat = Diag(alpha_t) S_{t-1}        alpha_t = exp(log_alpha_t)
 *       k_hat = b_t (.) kn ,  v_hat = w_t (.) v_t
 *       u     = v_hat - k_hat S_hat          (old value read at the erase key)
 *       S_t   = S_hat + kn^T u
 *       o_t   = qt S_t                        (read after the write)
 *     The display equation of the update is missing from the notes; this is
 *     the reading under which the notes' chunk system (section 2.4,
 *     T Z = [V_hat, K_hat decayed], T = I + L_strict) holds exactly, and it
 *     is the blog's DeltaNet step (v_old = k S; u = beta (v - v_old);
 *     S += k^T u) with the erase key b (.) k and the write value w (.) v.
 *     With b = w = beta it is Kimi Delta Attention; with a scalar alpha it is
 *     Gated DeltaNet; with alpha = 1 as well it is DeltaNet; with b = 0 it is
 *     gated linear attention.
 *
 * Parity pins (tests/test_oracle_pins.py): every reduction above against an
 * independent formula, brute-force products of the explicit transition
 * matrices, a dense solve of the whole-sequence triangular system, exact
 * recall, alpha -> 0 clearing, linearity, split/resume and the write/erase
 * sensitivity identity.  The backward (gdr_oracle_backward, reverse mode of
 * the same token loop) is pinned by central differences of the forward for
 * every input and gate mode, by split/resume across its checkpoints, and by
 * the closed form of linear attention.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* x * sigmoid(x), written as x / (1 + e^-x). */
static double silu(double x) { return x / (1.0 + exp(-x)); }

/* 2 * sigmoid(x). */
static double two_sigmoid(double x) { return 2.0 / (1.0 + exp(-x)); }

/* out = SiLU(x) / max(|SiLU(x)|_2, 1e-12), or a plain copy. */
static void silu_l2(const double *x, int d, int normalize, double *out) {
  int j;
  double ss = 0.0, nrm;
  if (!normalize) {
    for (j = 0; j < d; ++j) out[j] = x[j];
    return;
  }
  for (j = 0; j < d; ++j) {
    out[j] = silu(x[j]);
    ss += out[j] * out[j];
  }
  nrm = sqrt(ss);
  if (nrm < 1e-12) nrm = 1e-12;
  for (j = 0; j < d; ++j) out[j] /= nrm;
}

/*
 * Pre-pass of one token, exposed for the pre-pass pins.
 *   q, k, z: [dk]; gamma: [dk] or NULL (= 1); z may be NULL (2 sigma = 1).
 *   qt_out, k_out: [dk].
 */
void gdr_oracle_prepass(int dk, const double *q, const double *k,
                        const double *gamma, const double *z, double scale,
                        int normalize_qk, double *qt_out, double *k_out) {
  int j;
  silu_l2(q, dk, normalize_qk, qt_out);
  silu_l2(k, dk, normalize_qk, k_out);
  for (j = 0; j < dk; ++j) {
    double g = gamma ? gamma[j] : 1.0;
    double dyn = z ? two_sigmoid(z[j]) : 1.0;
    qt_out[j] = scale * g * dyn * qt_out[j];
  }
}

/*
 * The recurrence over n_streams independent streams of T tokens.
 *   q, k, log_alpha, b, z : [n_streams, T, dk]   (z may be NULL)
 *   v, w                  : [n_streams, T, dv]
 *   gamma                 : [n_streams, dk] or NULL
 *   S0                    : [n_streams, dk, dv] or NULL (zero state)
 *   o                     : [n_streams, T, dv]  (written)
 *   S_T                   : [n_streams, dk, dv] or NULL (written; may alias S0)
 * Returns 0, or -1 when scratch memory cannot be allocated.
 */
int gdr_oracle_forward(long n_streams, long T, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *b,
                       const double *w, const double *gamma, const double *z,
                       double scale, int normalize_qk, const double *S0,
                       double *o, double *S_T, int n_threads) {
  long n;
  int failed = 0;
  if (n_threads < 1) n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(|| : failed)
  for (n = 0; n < n_streams; ++n) {
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *qt = (double *)malloc(sizeof(double) * dk);
    double *kn = (double *)malloc(sizeof(double) * dk);
    double *kh = (double *)malloc(sizeof(double) * dk);
    double *vh = (double *)malloc(sizeof(double) * dv);
    double *u = (double *)malloc(sizeof(double) * dv);
    long t;
    int i, j;
    if (!S || !qt || !kn || !kh || !vh || !u) {
      failed = 1;
    } else {
      if (S0)
        memcpy(S, S0 + (size_t)n * dk * dv, sizeof(double) * (size_t)dk * dv);
      else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
      for (t = 0; t < T; ++t) {
        size_t rk = ((size_t)n * T + t) * dk; /* row of a [n,T,dk] tensor */
        size_t rv = ((size_t)n * T + t) * dv; /* row of a [n,T,dv] tensor */
        gdr_oracle_prepass(dk, q + rk, k + rk, gamma ? gamma + (size_t)n * dk : NULL,
                           z ? z + rk : NULL, scale, normalize_qk, qt, kn);
        for (i = 0; i < dk; ++i) kh[i] = b[rk + i] * kn[i];
        for (j = 0; j < dv; ++j) vh[j] = w[rv + j] * v[rv + j];
        /* S_hat = Diag(alpha) S : row i decays by alpha_i */
        for (i = 0; i < dk; ++i) {
          double a = exp(log_alpha[rk + i]);
          for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
        }
        /* u = v_hat - k_hat S_hat */
        for (j = 0; j < dv; ++j) {
          double r = 0.0;
          for (i = 0; i < dk; ++i) r += kh[i] * S[(size_t)i * dv + j];
          u[j] = vh[j] - r;
        }
        /* S = S_hat + kn^T u */
        for (i = 0; i < dk; ++i)
          for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kn[i] * u[j];
        /* o_t = qt S */
        for (j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + j];
          o[rv + j] = acc;
        }
      }
      if (S_T)
        memcpy(S_T + (size_t)n * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    }
    free(S);
    free(qt);
    free(kn);
    free(kh);
    free(vh);
    free(u);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * Backward pass: reverse-mode derivatives of the recurrence above, token by
 * token in fp64, for the loss  <dO, o> + <dS_T, S_T>  (the gradients a caller
 * gets when dO and dS_T are the upstream gradients of o and S_T).
 *
 * Reverse of one token (dS = gradient of S_t, read after the write):
 *   dS    += qt^T dO_t                 dqt  = S_t dO_t^T
 *   du     = kn dS                     dkn  = dS u^T
 *   dShat  = dS - k_hat^T du           dkh  = -S_hat du^T      dvh = du
 *   dalpha_i = sum_j dShat_ij S_{t-1,ij}
 *   dS_{t-1} = Diag(alpha) dShat
 * then the elementwise chains: dlog_alpha = dalpha * alpha, db = dkh * kn,
 * dkn += dkh * b, dw = dvh * v, dv = dvh * w, the read-out gain
 * (d 2 sigma(z) / dz = 2 sigma (1 - sigma)), and SiLU + l2 normalisation
 * (d(s / |s|) = (ds - y (y . ds)) / |s|; below the 1e-12 floor, ds / 1e-12).
 * The states S_{t-1} are recomputed from checkpoints every 64 tokens.
 * ------------------------------------------------------------------------ */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* dy -> dx through y = SiLU(x) / max(|SiLU(x)|, 1e-12) (or y = x). */
static void silu_l2_bwd(const double *x, int d, int normalize, const double *dy, double *dx) {
  int j;
  double ss = 0.0, nrm, dot = 0.0;
  if (!normalize) {
    for (j = 0; j < d; ++j) dx[j] = dy[j];
    return;
  }
  for (j = 0; j < d; ++j) {
    double sj = silu(x[j]);
    ss += sj * sj;
  }
  nrm = sqrt(ss);
  if (nrm > 1e-12) {
    for (j = 0; j < d; ++j) dot += (silu(x[j]) / nrm) * dy[j];
    for (j = 0; j < d; ++j) dx[j] = (dy[j] - (silu(x[j]) / nrm) * dot) / nrm;
  } else {
    for (j = 0; j < d; ++j) dx[j] = dy[j] / 1e-12;
  }
  for (j = 0; j < d; ++j) {
    double sg = sigmoid(x[j]);
    dx[j] *= sg * (1.0 + x[j] * (1.0 - sg));  /* SiLU'(x) */
  }
}

#define GDR_ORACLE_CKPT 64

/*
 * Arguments as gdr_oracle_forward, plus
 *   dO   [n_streams, T, dv]; dS_T [n_streams, dk, dv] or NULL (= 0)
 * and the gradients (all written; each may be NULL if not wanted):
 *   dq, dk_, dlog_alpha, db, dz : [n_streams, T, dk]
 *   dv_, dw                     : [n_streams, T, dv]
 *   dgamma                      : [n_streams, dk]   (summed over the stream's tokens)
 *   dS0                         : [n_streams, dk, dv]
 * Returns 0, or -1 when scratch memory cannot be allocated.
 */
int gdr_oracle_backward(long n_streams, long T, int dk, int dv,
                        const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *b,
                        const double *w, const double *gamma, const double *z,
                        double scale, int normalize_qk, const double *S0,
                        const double *dO, const double *dS_T,
                        double *dq, double *dk_, double *dv_, double *dlog_alpha,
                        double *db, double *dw, double *dgamma, double *dz,
                        double *dS0, int n_threads) {
  long n;
  int failed = 0;
  const size_t DD = (size_t)dk * dv;
  const long nck = (T + GDR_ORACLE_CKPT - 1) / GDR_ORACLE_CKPT;
  if (n_threads < 1) n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(|| : failed)
  for (n = 0; n < n_streams; ++n) {
    /* checkpoints: state before token c * CKPT; seg: states before each token
       of one segment and after its last */
    double *ck = (double *)malloc(sizeof(double) * DD * (size_t)(nck > 0 ? nck : 1));
    double *seg = (double *)malloc(sizeof(double) * DD * (GDR_ORACLE_CKPT + 1));
    double *dS = (double *)malloc(sizeof(double) * DD);
    double *Sh = (double *)malloc(sizeof(double) * DD);
    double *vec = (double *)malloc(sizeof(double) * (size_t)(16 * dk + 8 * dv));
    double *gsum = (double *)calloc((size_t)dk, sizeof(double));
    long t, c;
    int i, j;
    if (!ck || !seg || !dS || !Sh || !vec || !gsum) {
      failed = 1;
    } else {
      double *qh = vec, *qt = vec + dk, *kn = vec + 2 * dk, *kh = vec + 3 * dk;
      double *gain = vec + 4 * dk, *al = vec + 5 * dk, *dqt = vec + 6 * dk;
      double *dkn = vec + 7 * dk, *dkh = vec + 8 * dk, *dal = vec + 9 * dk;
      double *dqh = vec + 10 * dk, *tmp = vec + 11 * dk;
      double *vh = vec + 16 * dk, *u = vh + dv, *du = vh + 2 * dv;
      const double *gam = gamma ? gamma + (size_t)n * dk : NULL;
      /* token t's pre-pass values (qh, qt, gain, kn, kh, vh, alpha) */
#define GDR_TOKEN(t_)                                                         \
  do {                                                                        \
    size_t rk_ = ((size_t)n * T + (t_)) * dk, rv_ = ((size_t)n * T + (t_)) * dv; \
    silu_l2(q + rk_, dk, normalize_qk, qh);                                   \
    silu_l2(k + rk_, dk, normalize_qk, kn);                                   \
    for (i = 0; i < dk; ++i) {                                                \
      gain[i] = scale * (gam ? gam[i] : 1.0) * (z ? two_sigmoid(z[rk_ + i]) : 1.0); \
      qt[i] = gain[i] * qh[i];                                                \
      kh[i] = b[rk_ + i] * kn[i];                                             \
      al[i] = exp(log_alpha[rk_ + i]);                                        \
    }                                                                         \
    for (j = 0; j < dv; ++j) vh[j] = w[rv_ + j] * v[rv_ + j];                 \
  } while (0)
      /* one forward token step: Snew from Sold (both [dk, dv]) */
#define GDR_STEP(Sold, Snew)                                                  \
  do {                                                                        \
    for (i = 0; i < dk; ++i)                                                  \
      for (j = 0; j < dv; ++j) Sh[(size_t)i * dv + j] = al[i] * (Sold)[(size_t)i * dv + j]; \
    for (j = 0; j < dv; ++j) {                                                \
      double r_ = 0.0;                                                        \
      for (i = 0; i < dk; ++i) r_ += kh[i] * Sh[(size_t)i * dv + j];          \
      u[j] = vh[j] - r_;                                                      \
    }                                                                         \
    for (i = 0; i < dk; ++i)                                                  \
      for (j = 0; j < dv; ++j) (Snew)[(size_t)i * dv + j] = Sh[(size_t)i * dv + j] + kn[i] * u[j]; \
  } while (0)
      /* forward: checkpoints */
      if (S0)
        memcpy(seg, S0 + (size_t)n * DD, sizeof(double) * DD);
      else
        memset(seg, 0, sizeof(double) * DD);
      for (t = 0; t < T; ++t) {
        if (t % GDR_ORACLE_CKPT == 0) memcpy(ck + (size_t)(t / GDR_ORACLE_CKPT) * DD, seg, sizeof(double) * DD);
        GDR_TOKEN(t);
        GDR_STEP(seg, seg + DD);
        memcpy(seg, seg + DD, sizeof(double) * DD);
      }
      /* backward */
      if (dS_T)
        memcpy(dS, dS_T + (size_t)n * DD, sizeof(double) * DD);
      else
        memset(dS, 0, sizeof(double) * DD);
      for (c = nck - 1; c >= 0; --c) {
        long t0 = c * GDR_ORACLE_CKPT, t1 = t0 + GDR_ORACLE_CKPT < T ? t0 + GDR_ORACLE_CKPT : T;
        memcpy(seg, ck + (size_t)c * DD, sizeof(double) * DD);
        for (t = t0; t < t1; ++t) {
          GDR_TOKEN(t);
          GDR_STEP(seg + (size_t)(t - t0) * DD, seg + (size_t)(t - t0 + 1) * DD);
        }
        for (t = t1 - 1; t >= t0; --t) {
          const double *Sp = seg + (size_t)(t - t0) * DD;    /* S_{t-1} */
          const double *St = Sp + DD;                        /* S_t */
          size_t rk = ((size_t)n * T + t) * dk, rv = ((size_t)n * T + t) * dv;
          GDR_TOKEN(t);
          for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) Sh[(size_t)i * dv + j] = al[i] * Sp[(size_t)i * dv + j];
          for (j = 0; j < dv; ++j) { /* u */
            double r = 0.0;
            for (i = 0; i < dk; ++i) r += kh[i] * Sh[(size_t)i * dv + j];
            u[j] = vh[j] - r;
          }
          /* o_t = qt S_t */
          for (i = 0; i < dk; ++i) {
            double a = 0.0;
            for (j = 0; j < dv; ++j) a += St[(size_t)i * dv + j] * dO[rv + j];
            dqt[i] = a;
            for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += qt[i] * dO[rv + j];
          }
          /* S_t = S_hat + kn^T u */
          for (j = 0; j < dv; ++j) {
            double a = 0.0;
            for (i = 0; i < dk; ++i) a += kn[i] * dS[(size_t)i * dv + j];
            du[j] = a;
          }
          for (i = 0; i < dk; ++i) {
            double a = 0.0;
            for (j = 0; j < dv; ++j) a += dS[(size_t)i * dv + j] * u[j];
            dkn[i] = a;
          }
          /* u = v_hat - k_hat S_hat */
          for (i = 0; i < dk; ++i) {
            double a = 0.0;
            for (j = 0; j < dv; ++j) {
              a += Sh[(size_t)i * dv + j] * du[j];
              dS[(size_t)i * dv + j] -= kh[i] * du[j]; /* now dS_hat */
            }
            dkh[i] = -a;
          }
          /* S_hat = Diag(alpha) S_{t-1} */
          for (i = 0; i < dk; ++i) {
            double a = 0.0;
            for (j = 0; j < dv; ++j) {
              a += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
              dS[(size_t)i * dv + j] *= al[i];
            }
            dal[i] = a;
          }
          /* elementwise chains */
          for (i = 0; i < dk; ++i) {
            if (dlog_alpha) dlog_alpha[rk + i] = dal[i] * al[i];
            if (db) db[rk + i] = dkh[i] * kn[i];
            dkn[i] += dkh[i] * b[rk + i];
            dqh[i] = dqt[i] * gain[i];
            gsum[i] += dqt[i] * qh[i] * scale * (z ? two_sigmoid(z[rk + i]) : 1.0);
            if (dz) {
              double sg = sigmoid(z ? z[rk + i] : 0.0);
              dz[rk + i] = z ? dqt[i] * qh[i] * scale * (gam ? gam[i] : 1.0) * 2.0 * sg * (1.0 - sg) : 0.0;
            }
          }
          for (j = 0; j < dv; ++j) {
            if (dw) dw[rv + j] = du[j] * v[rv + j];
            if (dv_) dv_[rv + j] = du[j] * w[rv + j];
          }
          if (dq) {
            silu_l2_bwd(q + rk, dk, normalize_qk, dqh, tmp);
            for (i = 0; i < dk; ++i) dq[rk + i] = tmp[i];
          }
          if (dk_) {
            silu_l2_bwd(k + rk, dk, normalize_qk, dkn, tmp);
            for (i = 0; i < dk; ++i) dk_[rk + i] = tmp[i];
          }
        }
      }
      if (dS0) memcpy(dS0 + (size_t)n * DD, dS, sizeof(double) * DD);
      if (dgamma) memcpy(dgamma + (size_t)n * dk, gsum, sizeof(double) * dk);
#undef GDR_TOKEN
#undef GDR_STEP
    }
    free(ck);
    free(seg);
    free(dS);
    free(Sh);
    free(vec);
    free(gsum);
  }
  return failed ? -1 : 0;
}

/* Number of threads an OpenMP region would use by default (1 without OpenMP). */
int gdr_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
