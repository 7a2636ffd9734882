// gdr_chunk.hip -- chunkwise forward of the channel-wise gated delta rule.
//
// Chunk algebra (Muir reading notes, arXiv:2611.08376, section 2.4
// "Boundary-Pivoted Chunkwise Kernel"; the blog "Kimi3 = GPT2 x 22580",
// section 4 "DeltaNet", chunk_delta_rule_forward, for the UT/WY form).
// Within a chunk of C tokens with incoming state S (rows t, 0-based):
//   Lambda_t = sum_{r<=t} log alpha_r (fp32, per key channel)
//   pi_ts    = exp(Lambda_t - Lambda_s)                         (s <= t)
//   L[t,s]   = sum_c k_hat_t,c pi_ts,c kn_s,c   (s < t)          decayed Gram
//   A[t,s]   = sum_c qt_t,c    pi_ts,c kn_s,c   (s <= t)         read-out scores
//   (I + L) Z = R,  R = [V_hat | K_hat e^Lambda],  Z = [U_bar | Y]
//   O   = (Qt e^Lambda - A Y) S + A U_bar      =: Q' S + O_bar
//   S' = (Diag(e^Lambda_C) - K'^T Y) S + K'^T U_bar =: M S + N,  K' = kn e^{Lambda_C - Lambda}
// Kernel 1 ("intra", fully parallel over chunks) reduces every chunk to its
// affine map (Q', O_bar, M, N); kernel 2 ("scan") carries S in fp32 through
// the chunks of one stream, split over value-column slices, and writes o.
//
// Decay factors never divide by a decay prefix: every exponent is <= 0.  The
// chunk is cut into 16-token blocks; for a pair of blocks (i > j) the pivot is
// the last token of block i-1, p: pi_ts = exp(Lambda_t - Lambda_p) *
// exp(Lambda_p - Lambda_s), both factors in (0, 1] (the notes' boundary
// pivot).  Diagonal blocks use the block's own pivot; their column factor is
// exp(range) at most, range = the block's largest per-channel decay, and a
// block whose range exceeds kMaxDiagRange falls back to exact pairwise
// exponentials.  No C x C x dk tensor is formed.
//
// Matrix products run on bf16 MFMA (16x16x32) with every fp32 operand split
// into NS bf16 planes (NS = 2 for bf16 inputs, 3 for fp32 inputs) and fp32
// accumulation; the triangular inverse uses 16x16x16 MFMA the same way.
//
// Workspace per (stream, chunk) -- layouts are the scan kernel's operand
// fragments, so that it loads them as 16-byte vectors:
//   Qp : NS planes x [C/16][D/32][64 lanes][8] bf16   A-fragments of Q'
//   Mm : NS planes x [D/16][D/32][64][8]   bf16        A-fragments of M
//   Ob : [C/16][D/16][64][4] fp32                      accumulator tiles of O_bar
//   Nn : [D/16][D/16][64][4] fp32                      accumulator tiles of N
// The contraction index of Q' and M (a state row) is in tile-pair order, the
// order in which the scan kernel's accumulator tiles of S hold it.
#include <mutex>

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

constexpr float kMaxDiagRange = 40.0f;



__device__ __forceinline__ int tidx(int i, int j) { return i * (i + 1) / 2 + j; }

template <int NS>
__device__ __forceinline__ f32x4 mfma16_split(const float a[4], const float b[4], f32x4 c) {
  s16x4 ap[NS], bp[NS];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t ha[NS], hb[NS];
    split<NS>(a[e], ha);
    split<NS>(b[e], hb);
#pragma unroll
    for (int p = 0; p < NS; ++p) { ap[p][e] = (short)ha[p]; bp[p][e] = (short)hb[p]; }
  }
#pragma unroll
  for (int s = NS - 1; s >= 0; --s)
#pragma unroll
    for (int pa = 0; pa <= s; ++pa)
      c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ap[pa], bp[s - pa], c, 0, 0, 0);
  return c;
}

// Store NS planes of 4 fp32 values as 4 consecutive bf16 per plane.
template <int NS>
__device__ __forceinline__ void store4_planes(uint16_t *base, size_t plane_stride, const float x[4]) {
  uint16_t h[4][NS];
#pragma unroll
  for (int r = 0; r < 4; ++r) split<NS>(x[r], h[r]);
#pragma unroll
  for (int p = 0; p < NS; ++p) {
    uint2 u;
    u.x = (uint32_t)h[0][p] | ((uint32_t)h[1][p] << 16);
    u.y = (uint32_t)h[2][p] | ((uint32_t)h[3][p] << 16);
    *reinterpret_cast<uint2 *>(base + p * plane_stride) = u;
  }
}

template <int NS>
__device__ __forceinline__ void store8_planes(uint16_t *base, size_t plane_stride, const float x[8]) {
  bf16x8 f[NS];
  split8<NS>(x, f);
#pragma unroll
  for (int p = 0; p < NS; ++p) *reinterpret_cast<bf16x8 *>(base + p * plane_stride) = f[p];
}

template <int NS>
__device__ __forceinline__ void load_frag(const uint16_t *base, size_t plane_stride, bf16x8 f[NS]) {
#pragma unroll
  for (int p = 0; p < NS; ++p) f[p] = *reinterpret_cast<const bf16x8 *>(base + p * plane_stride);
}

template <int C, int D, int NS>
struct IntraLds {
  static constexpr int NB = C / 16, NKC = C / 32;
  static constexpr int LAM_LD = D + 4;     // padded rows: conflict-free 16-byte reads
  static constexpr int TILE_LD = 20;
  static constexpr int TILE_SZ = 16 * TILE_LD;
  static constexpr int NTILES = NB * (NB + 1) / 2;
  static constexpr int FRAG = 64 * 8;      // bf16 per fragment plane
  static constexpr int STAGE = NKC * 2 * NS * FRAG;
  static constexpr size_t bytes = sizeof(float) * ((size_t)C * LAM_LD + 2 * C + NTILES * TILE_SZ) +
                                  sizeof(uint16_t) * 2 * STAGE + sizeof(int) * NB;
};

// ============================================================================
// Kernel 1: one workgroup (8 waves) per (stream, chunk).
// ============================================================================
template <int C, int D, int NS, bool BF>
__global__ void __launch_bounds__(512) chunk_intra_kernel(ChunkArgs a) {
  using Lds = IntraLds<C, D, NS>;
  constexpr int NB = C / 16, NKC = C / 32, NKD = D / 32, NMT = D / 16;
  constexpr int LAM_LD = Lds::LAM_LD, TILE_LD = Lds::TILE_LD, TILE_SZ = Lds::TILE_SZ;
  constexpr int FRAG = Lds::FRAG;
  static_assert(NB <= 8 && NMT <= 8, "one wave per block row and per channel tile");

  extern __shared__ __align__(16) unsigned char smem[];
  float *lam = reinterpret_cast<float *>(smem);
  float *inq = lam + C * LAM_LD;
  float *ink = inq + C;
  float *Lt = ink + C;
  uint16_t *rst = reinterpret_cast<uint16_t *>(Lt + Lds::NTILES * TILE_SZ);
  uint16_t *zst = rst + Lds::STAGE;
  int *dflag = reinterpret_cast<int *>(zst + Lds::STAGE);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int NC = a.T / C;
  const size_t ch = blockIdx.x;
  const size_t bh = ch / NC;
  const int h = (int)(bh % a.H);
  const size_t row0 = bh * (size_t)a.T + (size_t)(ch % NC) * C;  // first token row
  const bool norm = a.normalize_qk != 0;

  // -------------------------------------------------- A1: inverse norms
  for (int t = wave; t < C; t += 8) {
    float sq = 0.f, sk = 0.f;
    for (int c = lane; c < D; c += 64) {
      float qv = ld1<BF>(a.q, (row0 + t) * D + c), kv = ld1<BF>(a.k, (row0 + t) * D + c);
      if (norm) { qv = silu(qv); kv = silu(kv); }
      sq += qv * qv;
      sk += kv * kv;
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    if (lane == 0) {
      inq[t] = norm ? 1.f / fmaxf(sqrtf(sq), 1e-12f) : 1.f;
      ink[t] = norm ? 1.f / fmaxf(sqrtf(sk), 1e-12f) : 1.f;
    }
  }
  // -------------------------------------------------- A2: Lambda (prefix over tokens)
  {
    constexpr int P = 512 / D, TP = C / P;
    const int c = tid % D, part = tid / D;
    float *tot = Lt;  // scratch, Lt is not live yet
    float run = 0.f;
    for (int u = 0; u < TP; ++u) {
      const int t = part * TP + u;
      run += log_alpha_at(a.log_alpha, a.alpha_mode, row0 + t, c, D);
      lam[t * LAM_LD + c] = run;
    }
    tot[part * D + c] = run;
    __syncthreads();
    float off = 0.f;
    for (int p2 = 0; p2 < part; ++p2) off += tot[p2 * D + c];
    if (part)
      for (int u = 0; u < TP; ++u) lam[(part * TP + u) * LAM_LD + c] += off;
  }
  __syncthreads();
  // diagonal-block decay ranges
  if (wave < NB) {
    const int i = wave;
    float m = 0.f;
    for (int c = lane; c < D; c += 64) {
      const float ref = i ? lam[(16 * i - 1) * LAM_LD + c] : 0.f;
      m = fmaxf(m, ref - lam[(16 * i + 15) * LAM_LD + c]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) dflag[i] = m > kMaxDiagRange;
  }
  __syncthreads();

  // per-channel gain pieces: qt_c = scale * gamma_c * 2 sigma(z_c) * q_c * inq
  auto qtilde = [&](size_t row, int t, int c, float qraw, float zraw) {
    float qn = (norm ? silu(qraw) : qraw) * inq[t];
    float gm = a.gamma ? a.gamma[(size_t)h * D + c] : 1.f;
    float dy = a.z ? two_sigmoid(zraw) : 1.f;
    return a.scale * gm * dy * qn;
  };

  // -------------------------------------------------- B: L and A tiles
  // Wave i owns token block i.  Products are computed transposed
  // (rows = s, cols = t) so that the accumulator lane <-> t.
  bf16x8 afr[NKC][NS];  // A-fragments of A (row block i), tile-pair order over s
#pragma unroll
  for (int ks = 0; ks < NKC; ++ks)
#pragma unroll
    for (int p = 0; p < NS; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) afr[ks][p][e] = (__bf16)0.f;

  if (wave < NB) {
    const int i = wave;
    const int t = 16 * i + l16;
    const size_t rowt = row0 + t;
    const float *lref = lam + (16 * i - 1) * LAM_LD;  // valid for i > 0
    bf16x8 qr[NKD][NS], kr[NKD][NS];                 // Qt R_i and K_hat R_i, lane <-> t
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      const int c0 = 32 * ks + 8 * g;
      float qv[8], kv[8], zv[8], xq[8], xk[8];
      ld8<BF>(a.q, rowt * D + c0, qv);
      ld8<BF>(a.k, rowt * D + c0, kv);
      if (a.z) ld8<BF>(a.z, rowt * D + c0, zv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        const float f = __expf(lam[t * LAM_LD + c] - (i ? lref[c] : 0.f));
        const float kn = (norm ? silu(kv[e]) : kv[e]) * ink[t];
        const float bb = gate_at<BF>(a.b, a.b_mode, rowt, c, D);
        xq[e] = qtilde(rowt, t, c, qv[e], a.z ? zv[e] : 0.f) * f;
        xk[e] = bb * kn * f;
      }
      split8<NS>(xq, qr[ks]);
      split8<NS>(xk, kr[ks]);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j > i) continue;
      const int s = 16 * j + l16;
      const size_t rows = row0 + s;
      f32x4 accL = zero4(), accA = zero4();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const int c0 = 32 * ks + 8 * g;
        float kv[8], x[8];
        ld8<BF>(a.k, rows * D + c0, kv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + e;
          const float kn = (norm ? silu(kv[e]) : kv[e]) * ink[s];
          x[e] = kn * __expf((i ? lref[c] : 0.f) - lam[s * LAM_LD + c]);
        }
        bf16x8 kc[NS];
        split8<NS>(x, kc);
        accL = mfma32_split<NS>(kc, kr[ks], accL);
        accA = mfma32_split<NS>(kc, qr[ks], accA);
      }
      // lane (col t, group g) holds rows s = 16j + 4g + r
      if (j == i) {
        if (dflag[i]) {
          // exact pairwise exponentials for a block whose decay range is too wide
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s2 = 16 * j + 4 * g + r;
            float lsum = 0.f, asum = 0.f;
            if (s2 <= t) {
              const size_t r2 = row0 + s2;
              for (int c = 0; c < D; ++c) {
                const float pi = __expf(lam[t * LAM_LD + c] - lam[s2 * LAM_LD + c]);
                const float kns = (norm ? silu(ld1<BF>(a.k, r2 * D + c)) : ld1<BF>(a.k, r2 * D + c)) * ink[s2];
                const float knt = (norm ? silu(ld1<BF>(a.k, rowt * D + c)) : ld1<BF>(a.k, rowt * D + c)) * ink[t];
                const float bb = gate_at<BF>(a.b, a.b_mode, rowt, c, D);
                const float qt = qtilde(rowt, t, c, ld1<BF>(a.q, rowt * D + c),
                                        a.z ? ld1<BF>(a.z, rowt * D + c) : 0.f);
                lsum += bb * knt * pi * kns;
                asum += qt * pi * kns;
              }
            }
            accL[r] = lsum;
            accA[r] = asum;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s2 = 16 * j + 4 * g + r;
          if (s2 >= t) accL[r] = 0.f;
          if (s2 > t) accA[r] = 0.f;
        }
      }
      // L[t][s] -> LDS tile (i, j), row t, columns 4g..4g+3
      *reinterpret_cast<float4 *>(Lt + tidx(i, j) * TILE_SZ + l16 * TILE_LD + 4 * g) =
          make_float4(accL[0], accL[1], accL[2], accL[3]);
      // A -> fragment ks = j/2, elements 4*(j%2) + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint16_t hp[NS];
        split<NS>(accA[r], hp);
#pragma unroll
        for (int p = 0; p < NS; ++p) afr[j / 2][p][4 * (j % 2) + r] = __builtin_bit_cast(__bf16, hp[p]);
      }
    }
  }
  __syncthreads();

  // -------------------------------------------------- C1: leaf inverses
  if (wave < NB && lane < 16) {
    float *Tii = Lt + tidx(wave, wave) * TILE_SZ;
    const int cc = lane;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = (t == cc) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < t; ++s)
        if (s >= cc) acc -= Tii[t * TILE_LD + s] * x[s];
      x[t] = (t < cc) ? 0.f : acc;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 16; ++t) Tii[t * TILE_LD + cc] = x[t];
  }
  __syncthreads();

  // -------------------------------------------------- C2: blocked forward substitution
  // X[i][q] = -X[i][i] sum_{j=q}^{i-1} L[i][j] X[j][q]; wave q owns column block q.
  for (int i = 1; i < NB; ++i) {
    const int qb = wave;
    f32x4 res = zero4();
    if (qb < i) {
      f32x4 W = zero4();
      for (int j = qb; j < i; ++j) {
        const float *Lij = Lt + tidx(i, j) * TILE_SZ;
        const float *Xjq = Lt + tidx(j, qb) * TILE_SZ;
        float av[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          av[e] = Lij[l16 * TILE_LD + 4 * g + e];
          bv[e] = Xjq[(4 * g + e) * TILE_LD + l16];
        }
        W = mfma16_split<NS>(av, bv, W);
      }
      const float *Xii = Lt + tidx(i, i) * TILE_SZ;
      float av[4], bv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = Xii[l16 * TILE_LD + 4 * g + e];
        bv[e] = W[e];
      }
      res = mfma16_split<NS>(av, bv, zero4());
    }
    __syncthreads();
    if (qb < i) {
      float *Xiq = Lt + tidx(i, qb) * TILE_SZ;
#pragma unroll
      for (int r = 0; r < 4; ++r) Xiq[(4 * g + r) * TILE_LD + l16] = -res[r];
    }
    __syncthreads();
  }

  // -------------------------------------------------- D: Z = T^-1 R and the chunk map
  // T^-1 A-fragments for row block i (lane <-> t), tile-pair order over s.
  bf16x8 tif[NKC][NS];
  if (wave < NB) {
    const int i = wave;
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jb = 2 * ks + e / 4;
        const int sc = 4 * g + (e % 4);
        x[e] = (jb <= i) ? Lt[tidx(i, jb) * TILE_SZ + l16 * TILE_LD + sc] : 0.f;
      }
      split8<NS>(x, tif[ks]);
    }
  }
  // K'^T fragments for channel tile m (lane <-> c), tile-pair order over s.
  bf16x8 kpf[NKC][NS];
  float gdiag = 0.f;
  if (wave < NMT) {
    const int c = 16 * wave + l16;
    const float lamC = lam[(C - 1) * LAM_LD + c];
    gdiag = __expf(lamC);
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = 32 * ks + 16 * (e / 4) + 4 * g + (e % 4);
        const float kv = ld1<BF>(a.k, (row0 + s) * D + c);
        x[e] = (norm ? silu(kv) : kv) * ink[s] * __expf(lamC - lam[s * LAM_LD + c]);
      }
      split8<NS>(x, kpf[ks]);
    }
  }

  const size_t chq = ch * NS;
  uint16_t *Qp = a.Qp + chq * (size_t)C * D;
  uint16_t *Mm = a.Mm + chq * (size_t)D * D;
  float *Ob = a.Ob + ch * (size_t)C * D;
  float *Nn = a.Nn + ch * (size_t)D * D;

  for (int cp = 0; cp < 2 * D / 32; ++cp) {
    const bool vhalf = cp < D / 32;
    // D1: stage R[:, 32cp .. 32cp+32) as B-fragments (lane <-> column)
    for (int item = tid; item < (C / 4) * 32; item += 512) {
      const int jl = item % 32, s0 = 4 * (item / 32);
      const int jcol = 32 * cp + jl;
      float val[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = s0 + r;
        const size_t rs = row0 + s;
        if (vhalf) {
          val[r] = gate_at<BF>(a.w, a.w_mode, rs, jcol, D) * ld1<BF>(a.v, rs * D + jcol);
        } else {
          const int c = jcol - D;
          const float kv = ld1<BF>(a.k, rs * D + c);
          val[r] = gate_at<BF>(a.b, a.b_mode, rs, c, D) * (norm ? silu(kv) : kv) * ink[s] *
                   __expf(lam[s * LAM_LD + c]);
        }
      }
      const int ks = s0 / 32, w32 = s0 % 32;
      const int ehi = w32 / 16, gq = (w32 % 16) / 4;
      const int ln = (jl % 16) + 16 * gq;
      store4_planes<NS>(rst + ((ks * 2 + jl / 16) * NS) * FRAG + ln * 8 + 4 * ehi, FRAG, val);
    }
    __syncthreads();
    // D2: Z rows of block i (wave i), two column tiles
    if (wave < NB) {
      const int i = wave;
#pragma unroll
      for (int ctl = 0; ctl < 2; ++ctl) {
        f32x4 zacc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) {
          if (2 * ks > i) continue;
          bf16x8 rb[NS];
          load_frag<NS>(rst + ((ks * 2 + ctl) * NS) * FRAG + lane * 8, FRAG, rb);
          zacc = mfma32_split<NS>(tif[ks], rb, zacc);
        }
        float zv[4] = {zacc[0], zacc[1], zacc[2], zacc[3]};
        store4_planes<NS>(zst + (((i / 2) * 2 + ctl) * NS) * FRAG + lane * 8 + 4 * (i % 2), FRAG, zv);
      }
    }
    __syncthreads();
    // D3: products with Z
    if (vhalf) {
      if (wave < NMT) {  // N = K'^T U_bar
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < NKC; ++ks) {
            bf16x8 zb[NS];
            load_frag<NS>(zst + ((ks * 2 + ctl) * NS) * FRAG + lane * 8, FRAG, zb);
            acc = mfma32_split<NS>(kpf[ks], zb, acc);
          }
          const int jt = 2 * cp + ctl;
          *reinterpret_cast<f32x4 *>(Nn + ((size_t)(wave * NMT + jt) * 64 + lane) * 4) = acc;
        }
      }
      if (wave < NB) {  // O_bar = A U_bar
        const int i = wave;
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < NKC; ++ks) {
            if (2 * ks > i) continue;
            bf16x8 zb[NS];
            load_frag<NS>(zst + ((ks * 2 + ctl) * NS) * FRAG + lane * 8, FRAG, zb);
            acc = mfma32_split<NS>(afr[ks], zb, acc);
          }
          const int jt = 2 * cp + ctl;
          *reinterpret_cast<f32x4 *>(Ob + ((size_t)(i * NMT + jt) * 64 + lane) * 4) = acc;
        }
      }
    } else {
      const int ksy = cp - D / 32;  // k-step of the state-row index covered by this pair
      if (wave < NMT) {             // M = Diag(e^Lambda_C) - K'^T Y, as (K'^T Y)^T = Y^T K'
        const int c = 16 * wave + l16;
        float mv[8];
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < NKC; ++ks) {
            bf16x8 zb[NS];
            load_frag<NS>(zst + ((ks * 2 + ctl) * NS) * FRAG + lane * 8, FRAG, zb);
            acc = mfma32_split<NS>(zb, kpf[ks], acc);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cpr = 32 * ksy + 16 * ctl + 4 * g + r;
            mv[4 * ctl + r] = (cpr == c ? gdiag : 0.f) - acc[r];
          }
        }
        store8_planes<NS>(Mm + ((size_t)(wave * NKD + ksy) * 64 + lane) * 8, (size_t)D * D, mv);
      }
      if (wave < NB) {  // Q' = Qt e^Lambda - A Y, as (A Y)^T = Y^T A^T
        const int i = wave;
        const int t = 16 * i + l16;
        const size_t rowt = row0 + t;
        float qv8[8];
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < NKC; ++ks) {
            if (2 * ks > i) continue;
            bf16x8 zb[NS];
            load_frag<NS>(zst + ((ks * 2 + ctl) * NS) * FRAG + lane * 8, FRAG, zb);
            acc = mfma32_split<NS>(zb, afr[ks], acc);
          }
          const int c0 = 32 * ksy + 16 * ctl + 4 * g;
          float qr4[4], zr4[4] = {0.f, 0.f, 0.f, 0.f};
          ld4<BF>(a.q, rowt * D + c0, qr4);
          if (a.z) ld4<BF>(a.z, rowt * D + c0, zr4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = c0 + r;
            const float qe = qtilde(rowt, t, c, qr4[r], zr4[r]) * __expf(lam[t * LAM_LD + c]);
            qv8[4 * ctl + r] = qe - acc[r];
          }
        }
        store8_planes<NS>(Qp + ((size_t)(i * NKD + ksy) * 64 + lane) * 8, (size_t)C * D, qv8);
      }
    }
    __syncthreads();
  }
}

// ============================================================================
// Kernel 2: one workgroup (4 waves) per (stream, 16-column value slice).
// The fp32 state slice lives in the accumulator tiles of the waves; its NS
// bf16 planes are shared through LDS as B-fragments every chunk.
// ============================================================================
template <int C, int D, int NS, bool OB16>
__global__ void __launch_bounds__(256) chunk_scan_kernel(ChunkArgs a) {
  constexpr int NRT = C / 16, NMT = D / 16, NKD = D / 32, NSL = D / 16;
  constexpr int RPW = (NRT + 3) / 4, MPW = (NMT + 3) / 4;
  constexpr int FRAG = 64 * 8;
  __shared__ __align__(16) uint16_t sfr[NKD * NS * FRAG];

  // all slices of one stream on the same XCD (workgroups go round-robin over 8)
  const int id = blockIdx.x;
  const int grp = id / (8 * NSL), rem = id % (8 * NSL);
  const int slice = rem / 8;
  const size_t bh = (size_t)grp * 8 + rem % 8;
  if (bh >= (size_t)a.B * a.H) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int NC = a.T / C;
  const int col = 16 * slice + l16;

  f32x4 S[MPW];
#pragma unroll
  for (int u = 0; u < MPW; ++u) {
    const int mt = wave + 4 * u;
    S[u] = zero4();
    if (mt < NMT && a.S0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[u][r] = a.S0[(bh * D + 16 * mt + 4 * g + r) * D + col];
    }
  }
  auto publish = [&]() {
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int mt = wave + 4 * u;
      if (mt < NMT) {
        float x[4] = {S[u][0], S[u][1], S[u][2], S[u][3]};
        store4_planes<NS>(sfr + ((mt / 2) * NS) * FRAG + lane * 8 + 4 * (mt % 2), FRAG, x);
      }
    }
  };
  publish();
  __syncthreads();

  for (int c = 0; c < NC; ++c) {
    const size_t ch = bh * NC + c;
    const uint16_t *Qp = a.Qp + ch * NS * (size_t)C * D;
    const uint16_t *Mm = a.Mm + ch * NS * (size_t)D * D;
    const float *Ob = a.Ob + ch * (size_t)C * D;
    const float *Nn = a.Nn + ch * (size_t)D * D;
    bf16x8 sf[NKD][NS];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) load_frag<NS>(sfr + (ks * NS) * FRAG + lane * 8, FRAG, sf[ks]);
    // outputs
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int rt = wave + 4 * u;
      if (rt < NRT) {
        f32x4 acc = *reinterpret_cast<const f32x4 *>(Ob + ((size_t)(rt * NMT + slice) * 64 + lane) * 4);
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) {
          bf16x8 qa[NS];
          load_frag<NS>(Qp + ((size_t)(rt * NKD + ks) * 64 + lane) * 8, (size_t)C * D, qa);
          acc = mfma32_split<NS>(qa, sf[ks], acc);
        }
        const size_t orow = bh * (size_t)a.T + (size_t)c * C + 16 * rt + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) st1<OB16>(a.o, (orow + r) * D + col, acc[r]);
      }
    }
    // next state
    f32x4 Sn[MPW];
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int mt = wave + 4 * u;
      Sn[u] = zero4();
      if (mt < NMT) {
        f32x4 acc = *reinterpret_cast<const f32x4 *>(Nn + ((size_t)(mt * NMT + slice) * 64 + lane) * 4);
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) {
          bf16x8 ma[NS];
          load_frag<NS>(Mm + ((size_t)(mt * NKD + ks) * 64 + lane) * 8, (size_t)D * D, ma);
          acc = mfma32_split<NS>(ma, sf[ks], acc);
        }
        Sn[u] = acc;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MPW; ++u) S[u] = Sn[u];
    publish();
    __syncthreads();
  }
  if (a.S_T) {
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int mt = wave + 4 * u;
      if (mt < NMT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) a.S_T[(bh * D + 16 * mt + 4 * g + r) * D + col] = S[u][r];
      }
    }
  }
}

// ============================================================================
// host side
// ============================================================================
size_t chunk_workspace_bytes(int B, int H, int T, int C, int D, int NS) {
  const size_t nch = (size_t)B * H * (T / C);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(nch * NS * (size_t)C * D * 2) + al(nch * NS * (size_t)D * D * 2) +
         al(nch * (size_t)C * D * 4) + al(nch * (size_t)D * D * 4);
}

bool chunk_intra_fits(int C, int D, int NS) {
  size_t b = 0;
#define GDR_FIT(CC, DD, NN) if (C == CC && D == DD && NS == NN) b = IntraLds<CC, DD, NN>::bytes;
  GDR_FIT(64, 64, 2) GDR_FIT(64, 64, 3) GDR_FIT(64, 128, 2) GDR_FIT(64, 128, 3)
  GDR_FIT(128, 64, 2) GDR_FIT(128, 64, 3) GDR_FIT(128, 128, 2) GDR_FIT(128, 128, 3)
#undef GDR_FIT
  return b > 0 && b <= 160 * 1024;
}

template <int C, int D, int NS, bool BF, bool OB16>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t st) {
  using Lds = IntraLds<C, D, NS>;
  static_assert(Lds::bytes <= 160 * 1024 || NS == 3, "intra-chunk LDS budget");
  if constexpr (Lds::bytes <= 160 * 1024) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [] {
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lds::bytes);
    });
    if (attr_err != hipSuccess) return attr_err;
    const size_t nbh = (size_t)a.B * a.H;
    const size_t nch = nbh * (size_t)(a.T / C);
    if (nch > 0) {
      hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF>), dim3((unsigned)nch), dim3(512), Lds::bytes, st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    constexpr int NSL = D / 16;
    const size_t nblk = ((nbh + 7) / 8) * 8 * NSL;
    hipLaunchKernelGGL((chunk_scan_kernel<C, D, NS, OB16>), dim3((unsigned)nblk), dim3(256), 0, st, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk(const gdr_desc &d, const ChunkArgs &a, hipStream_t st) {
  const bool ib = d.in_dtype == GDR_BF16, ob = d.out_dtype == GDR_BF16;
#define GDR_CH(CC, DD, IB, OBB)                                                            \
  if (d.chunk == CC && d.dk == DD && ib == IB && ob == OBB)                                \
    return launch_chunk_t<CC, DD, (IB ? 2 : 3), IB, OBB>(a, st);
  GDR_CH(64, 64, true, false) GDR_CH(64, 64, true, true) GDR_CH(64, 64, false, false)
  GDR_CH(64, 64, false, true) GDR_CH(64, 128, true, false) GDR_CH(64, 128, true, true)
  GDR_CH(64, 128, false, false) GDR_CH(64, 128, false, true) GDR_CH(128, 64, true, false)
  GDR_CH(128, 64, true, true) GDR_CH(128, 64, false, false) GDR_CH(128, 64, false, true)
  GDR_CH(128, 128, true, false) GDR_CH(128, 128, true, true)
#undef GDR_CH
  return hipErrorInvalidValue;
}

}  // namespace gdr
