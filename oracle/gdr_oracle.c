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
 * sensitivity identity.
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

/* Number of threads an OpenMP region would use by default (1 without OpenMP). */
int gdr_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
