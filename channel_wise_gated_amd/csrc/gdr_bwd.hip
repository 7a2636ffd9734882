// gdr_bwd.hip -- backward pass of the chunkwise forward: reverse-mode
// derivatives of the GDN-2 recurrence with the read-out gain (Muir reading
// notes, arXiv:2611.08376, section 2.1), through the chunk system of section
// 2.4.  For the loss <dO, o> + <dS_T, S_T> it returns the gradients of q, k,
// v, the gates, gamma, z and S0.
//
// Chunks of C = 64 tokens.  With the chunk-start state S0, the gradient X of
// the chunk-end state, a_t = e^{Lambda_t} (cumulative log-decay inside the
// chunk), K_a = K_hat (.) a, Q_a = Q_tilde (.) a, K' = K (.) a_C / a and the
// forward's T = I + L (L strictly lower), A (lower, diagonal included):
//   U     = T^-1 (V_hat - K_a S0)              (the per-token u of the recurrence)
//   dU~   = T^-T (A^T dO + K' X)
//   dA    = dO U^T  (s <= t),   dL = -dU~ U^T  (s < t)
//   dQ_a  = dO S0^T,  dK_a = -dU~ S0^T,  dK' = U X^T,  dV_hat = dU~
// and each decayed product L_ts = sum_i k_hat_ti k_si e^{Lambda_ti - Lambda_si}
// (A_ts likewise with q_tilde) is differentiated pair by pair.  The chunk-end
// gradients come from a chain over chunks, last to first:
//   X_{c-1} = M_c^T X_c + Q'_c^T dO_c
// with M and Q' from the forward's intra-chunk kernel; it runs in the forward
// chain kernel, with M^T and Q'^T dO in its M and N slots.
//
// Order of a call (gdr_chunk_bwd): the forward's intra-chunk kernel
// recomputes the chunk maps; the prep kernel forms M^T and Q'^T dO; the forward
// chain (chunk-start states) and the reverse chain (X) run side by side in one
// launch; then per chunk the pre-pass, the Gram kernel (A, T^-1), the dense
// products and the Gram backprop with the chains to the inputs; last dgamma.
// Everything is fp32 (products on the fp32 matrix cores, v_mfma_f32_16x16x4);
// the stages hand over through per-chunk scratch of the workspace.  Pair decays
// are split at per-block pivots, with a pair-by-pair path for steep blocks.
#include <stdint.h>

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

namespace {

constexpr int kBC = 64;  // chunk size of the backward

// Where a chunk slot's tokens are: the token row (of the [B,H,T] or packed
// [1,H,T] tensors) of its first token, how many of its 64 tokens are real and
// its head.  Uniform batches: slot = stream * NC + chunk.  Packed batches:
// slot = entry * H + head over the chunk list (entries past the end hold no
// tokens).
struct SlotTokens {
  size_t row;
  int valid, head;
};
__device__ __forceinline__ SlotTokens slot_tokens(const BwdArgs &a, size_t slot) {
  SlotTokens s;
  if (a.ctab) {
    const int4 e = a.ctab[slot / a.H];
    s.head = (int)(slot % a.H);
    s.valid = e.x < 0 ? 0 : e.w;
    s.row = (size_t)s.head * a.T + (e.x < 0 ? 0 : e.z);
  } else {
    const size_t bh = slot / a.NC;
    const int c = (int)(slot % a.NC);
    s.head = (int)(bh % a.H);
    s.valid = min(kBC, a.T - c * kBC);
    s.row = bh * a.T + (size_t)c * kBC;
  }
  return s;
}

// ---------------------------------------------------------------------------
// Prep: per chunk slot, M^T (plane by plane, in M's A-fragment layout) and
// G = Q'^T dO (in N's accumulator-tile layout) for the reverse chain.  Each M
// plane goes through LDS row-major (16-byte fragment reads and writes on both
// sides); G is computed on the fp32 matrix cores from Q' and dO in LDS, wave w
// owning G's row tiles w * NMT/4 to (w + 1) * NMT/4 - 1 (NMT = D / 16).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma4(float x, float y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0);
}

// four consecutive dO values (fp32 or bf16)
__device__ __forceinline__ f32x4 ld_do4(const void *p, size_t i, int bf) {
  if (bf) {
    const uint2 r = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
    return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                 __uint_as_float(r.y & 0xffff0000u)};
  }
  const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
  return f32x4{v.x, v.y, v.z, v.w};
}

template <int D, int NS>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdArgs a) {
  constexpr int C = kBC, NKD = D / 32, NMT = D / 16, MP = D + 8, SP = D + 4, RT = NMT / 4;
  static_assert(D * MP * 2 <= 2 * C * SP * 4, "an M plane fits in the Q' / dO space");
  // first one plane of M at a time, row-major (bf16); then Q' [t][i] and dO [t][j]
  __shared__ __align__(16) float lds[2 * C * SP];
  uint16_t *mp = reinterpret_cast<uint16_t *>(lds);
  float *qs = lds, *ds = lds + C * SP;
  const size_t slot = blockIdx.x;
  const SlotTokens st = slot_tokens(a, slot);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  // A-fragment entry (f, lane) of a D x D plane: 8 values of row 16 (f / NKD) + l16,
  // columns 32 (f % NKD) + 4 g + {0..3} and + 16
  const uint16_t *Ms = a.Mm + slot * NS * (size_t)D * D;
  uint16_t *Mt = a.Mt + slot * NS * (size_t)D * D;
#pragma unroll
  for (int p = 0; p < NS; ++p) {
    for (int idx = tid; idx < D * D / 8; idx += 256) {
      const int f = idx >> 6, ln = idx & 63, row = 16 * (f / NKD) + (ln & 15), col = 32 * (f % NKD) + 4 * (ln >> 4);
      const uint4 v = reinterpret_cast<const uint4 *>(Ms + (size_t)p * D * D)[idx];
      *reinterpret_cast<uint2 *>(mp + row * MP + col) = uint2{v.x, v.y};
      *reinterpret_cast<uint2 *>(mp + row * MP + col + 16) = uint2{v.z, v.w};
    }
    __syncthreads();
    for (int idx = tid; idx < D * D / 8; idx += 256) {
      // M^T[R][Cc] = M[Cc][R]: R = 16 (f / NKD) + l16, Cc over the entry's 8 columns
      const int f = idx >> 6, ln = idx & 63, R = 16 * (f / NKD) + (ln & 15), c0 = 32 * (f % NKD) + 4 * (ln >> 4);
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = mp[(c0 + 16 * (e >> 2) + (e & 3)) * MP + R];
      reinterpret_cast<uint4 *>(Mt + (size_t)p * D * D)[idx] =
          uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
    __syncthreads();
  }
  // Q' (planes summed in fp32) and dO into LDS
  const uint16_t *Qs = a.Qp + slot * NS * (size_t)C * D;
  for (int idx = tid; idx < C * D / 8; idx += 256) {
    const int f = idx >> 6, ln = idx & 63, t = 16 * (f / NKD) + (ln & 15), col = 32 * (f % NKD) + 4 * (ln >> 4);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const bf16x8 q8 = reinterpret_cast<const bf16x8 *>(Qs + (size_t)p * C * D)[idx];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += (float)q8[e];
    }
    *reinterpret_cast<float4 *>(qs + t * SP + col) = float4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<float4 *>(qs + t * SP + col + 16) = float4{v[4], v[5], v[6], v[7]};
  }
  for (int idx = tid; idx < C * D / 4; idx += 256) {
    const int t = idx / (D / 4), j4 = idx % (D / 4);
    *reinterpret_cast<f32x4 *>(ds + t * SP + 4 * j4) =
        t < st.valid ? ld_do4(a.dO, (st.row + t) * D + 4 * j4, a.do_bf16) : zero4();
  }
  __syncthreads();
  // G[i][j] = sum_t Q'[t][i] dO[t][j]: lane (l16, g) supplies k = t = 16 kb + 4 g + e
  f32x4 acc[RT][NMT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int jt = 0; jt < NMT; ++jt) acc[rt][jt] = zero4();
#pragma unroll
  for (int kb = 0; kb < C / 16; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * kb + 4 * g + e;
      float av[RT], bv[NMT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) av[rt] = qs[t * SP + 16 * (RT * w + rt) + l16];
#pragma unroll
      for (int jt = 0; jt < NMT; ++jt) bv[jt] = ds[t * SP + 16 * jt + l16];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jt = 0; jt < NMT; ++jt) acc[rt][jt] = mfma4(av[rt], bv[jt], acc[rt][jt]);
    }
  f32x4 *G = reinterpret_cast<f32x4 *>(a.Gn + slot * (size_t)D * D);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int jt = 0; jt < NMT; ++jt) G[((RT * w + rt) * NMT + jt) * 64 + lane] = acc[rt][jt];
}

// ---------------------------------------------------------------------------
// Pre-pass: per chunk slot, the forward's per-token vectors kn, k_hat,
// q_tilde, v_hat and the cumulative log-decay Lambda.  Wave w takes tokens
// 16w..16w+15, lane CPL = D / 64 consecutive channels; Lambda is summed along
// the wave's tokens in registers, then offset by the earlier waves' totals.
// Padding tokens past T are zero (identity steps).
// ---------------------------------------------------------------------------
template <bool BF, int N>
__device__ __forceinline__ void ldc(const void *p, size_t i, float (&o)[N]) {
  if constexpr (N == 2) {
    if constexpr (BF) {
      const uint32_t u = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(p) + i);
      o[0] = __uint_as_float(u << 16);
      o[1] = __uint_as_float(u & 0xffff0000u);
    } else {
      const float2 f = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(p) + i);
      o[0] = f.x;
      o[1] = f.y;
    }
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) o[u] = ld1<BF>(p, i + u);
  }
}

template <int N>
__device__ __forceinline__ void stc(float *p, const float (&x)[N]) {
  if constexpr (N == 2)
    *reinterpret_cast<float2 *>(p) = float2{x[0], x[1]};
  else
#pragma unroll
    for (int u = 0; u < N; ++u) p[u] = x[u];
}

template <int D, bool BF>
__global__ void __launch_bounds__(256) bwd_prepass_kernel(BwdArgs a) {
  constexpr int C = kBC, CPL = D / 64, TW = C / 4;
  __shared__ float tot[4][D];
  const size_t slot = blockIdx.x;
  const SlotTokens st = slot_tokens(a, slot);
  const int h = st.head;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ch0 = CPL * lane;
  const size_t base = slot * (size_t)C * D;
  float gam[CPL], run[CPL], lam[TW][CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    gam[u] = a.gamma ? a.gamma[(size_t)h * D + ch0 + u] : 1.f;
    run[u] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int t = TW * w + j;
    const bool ok = t < st.valid;  // uniform over the wave
    const size_t row = st.row + (ok ? t : 0);
    float qv[CPL], kv[CPL], vv[CPL], zv[CPL], bg[CPL], wg[CPL], la[CPL];
    float sq = 0.f, sk = 0.f;
    if (ok) {
      ldc<BF, CPL>(a.q, row * D + ch0, qv);
      ldc<BF, CPL>(a.k, row * D + ch0, kv);
      ldc<BF, CPL>(a.v, row * D + ch0, vv);
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        zv[u] = a.z ? ld1<BF>(a.z, row * D + ch0 + u) : 0.f;
        bg[u] = gate_at<BF>(a.b, a.b_mode, row, ch0 + u, D);
        wg[u] = gate_at<BF>(a.w, a.w_mode, row, ch0 + u, D);
        la[u] = log_alpha_at(a.log_alpha, a.alpha_mode, row, ch0 + u, D);
      }
    } else {
#pragma unroll
      for (int u = 0; u < CPL; ++u) qv[u] = kv[u] = vv[u] = zv[u] = bg[u] = wg[u] = la[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      if (a.normalize_qk) {
        qv[u] = silu(qv[u]);
        kv[u] = silu(kv[u]);
      }
      sq += qv[u] * qv[u];
      sk += kv[u] * kv[u];
    }
    float iq = 1.f, ik = 1.f;
    if (a.normalize_qk) {
      iq = 1.f / fmaxf(sqrtf(wave_sum(sq)), 1e-12f);
      ik = 1.f / fmaxf(sqrtf(wave_sum(sk)), 1e-12f);
    }
    float kn[CPL], kh[CPL], qt[CPL], vh[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const float dyn = (a.z && ok) ? 2.f / (1.f + expf(-zv[u])) : 1.f;
      kn[u] = kv[u] * ik;
      kh[u] = bg[u] * kn[u];
      qt[u] = ok ? a.scale * gam[u] * dyn * qv[u] * iq : 0.f;
      vh[u] = wg[u] * vv[u];
      run[u] += la[u];
      lam[j][u] = run[u];
    }
    const size_t o = base + (size_t)t * D + ch0;
    stc<CPL>(a.KN + o, kn);
    stc<CPL>(a.KH + o, kh);
    stc<CPL>(a.QT + o, qt);
    stc<CPL>(a.VH + o, vh);
  }
#pragma unroll
  for (int u = 0; u < CPL; ++u) tot[w][ch0 + u] = run[u];
  __syncthreads();
  float off[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    off[u] = 0.f;
    for (int w2 = 0; w2 < w; ++w2) off[u] += tot[w2][ch0 + u];
  }
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    float x[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) x[u] = lam[j][u] + off[u];
    stc<CPL>(a.LAM + base + (size_t)(TW * w + j) * D + ch0, x);
  }
}

// ---------------------------------------------------------------------------
// Gram: per chunk slot, A (s <= t) and L (s < t), A_ts = sum_i q_tilde_ti
// kn_si e^{Lambda_ti - Lambda_si} and L_ts likewise with k_hat, on the fp32
// matrix cores by 16 x 16 tiles: the pair decay is split at a per-channel pivot
// P, e^{Lambda_t - P} on the t side and e^{P - Lambda_s} on the s side.  For a
// tile below the diagonal P is Lambda at the s-block's last token, so both
// factors are <= 1 (a factor that underflows belongs to a product that does
// too).  For a diagonal tile P is Lambda at the block's first token: the s-side
// factor grows to e^{range} over the block; when the range exceeds 60 (far
// from fp32 overflow) the tile is recomputed pair by pair.  Then
// T^-1 = (I + L)^-1 column by column (forward substitution, four lanes a
// column).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

template <int D>
__global__ void __launch_bounds__(256) bwd_gram_kernel(BwdArgs a) {
  constexpr int C = kBC, NKB = D / 16, LP = C + 1;
  constexpr float kMaxRange = 60.f;
  static_assert(C == 64, "tile list for four 16-token blocks");
  __shared__ float L[C * LP], ti[C * LP];
  const size_t slot = blockIdx.x;
  const size_t base = slot * (size_t)C * D, cbase = slot * (size_t)C * C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  for (int e = tid; e < C * C; e += 256) {
    const int t = e / C, s2 = e % C;
    if ((s2 >> 4) > (t >> 4)) a.AM[cbase + e] = 0.f;  // tiles above the diagonal
  }
  // the ten tiles (tb, sb), sb <= tb: diagonal first, wave w takes w, w + 4, w + 8
  // nibble k of each word: tb and sb of tile k
  constexpr unsigned long long kTb = 0x3323213210ull, kSb = 0x0102103210ull;
  for (int k = w; k < 10; k += 4) {
    const int tb = (int)((kTb >> (4 * k)) & 15), sb = (int)((kSb >> (4 * k)) & 15);
    const bool diag = tb == sb;
    const int prow = diag ? 16 * sb : 16 * sb + 15;
    const size_t rt = base + (size_t)(16 * tb + l16) * D, rs = base + (size_t)(16 * sb + l16) * D,
                 rp = base + (size_t)prow * D;
    f32x4 accA = zero4(), accL = zero4();
    float emax = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int i0 = 16 * kb + 4 * g;
      const float4 qt = *reinterpret_cast<const float4 *>(a.QT + rt + i0);
      const float4 kh = *reinterpret_cast<const float4 *>(a.KH + rt + i0);
      const float4 lt = *reinterpret_cast<const float4 *>(a.LAM + rt + i0);
      const float4 kn = *reinterpret_cast<const float4 *>(a.KN + rs + i0);
      const float4 ls = *reinterpret_cast<const float4 *>(a.LAM + rs + i0);
      const float4 lp = *reinterpret_cast<const float4 *>(a.LAM + rp + i0);
      const float q4[4] = {qt.x, qt.y, qt.z, qt.w}, h4[4] = {kh.x, kh.y, kh.z, kh.w};
      const float t4[4] = {lt.x, lt.y, lt.z, lt.w}, n4[4] = {kn.x, kn.y, kn.z, kn.w};
      const float s4[4] = {ls.x, ls.y, ls.z, ls.w}, p4[4] = {lp.x, lp.y, lp.z, lp.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fa = __expf(t4[e] - p4[e]), xb = p4[e] - s4[e];
        emax = fmaxf(emax, xb);
        const float b = n4[e] * __expf(xb);
        accA = mfma4(q4[e] * fa, b, accA);
        accL = mfma4(h4[e] * fa, b, accL);
      }
    }
    if (diag && wave_max(emax) > kMaxRange) {
      // steep decay over the block: every pair of the lane's outputs exactly
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * g + r, s2 = 16 * sb + l16;
        float sa = 0.f, sl = 0.f;
        if (s2 <= t)
          for (int i = 0; i < D; ++i) {
            const float x = a.KN[base + (size_t)s2 * D + i] *
                            __expf(a.LAM[base + (size_t)t * D + i] - a.LAM[base + (size_t)s2 * D + i]);
            sa += a.QT[base + (size_t)t * D + i] * x;
            sl += a.KH[base + (size_t)t * D + i] * x;
          }
        accA[r] = sa;
        accL[r] = sl;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tb + 4 * g + r, s2 = 16 * sb + l16;
      a.AM[cbase + (size_t)t * C + s2] = (!diag || s2 <= t) ? accA[r] : 0.f;
      L[t * LP + s2] = (!diag || s2 < t) ? accL[r] : 0.f;
    }
  }
  __syncthreads();
  // T^-1 column s by four adjacent lanes (each summing every fourth r):
  // x_t = delta_ts - sum_{s <= r < t} L[t][r] x_r
  {
    const int s2 = tid >> 2, j = tid & 3;
    for (int t = 0; t < C; ++t) {
      float part = 0.f;
      if (t > s2)
        for (int r = s2 + j; r < t; r += 4) part += L[t * LP + r] * ti[r * LP + s2];
      part += __shfl_xor(part, 1, kWave);
      part += __shfl_xor(part, 2, kWave);
      if (j == 0) ti[t * LP + s2] = (t == s2 ? 1.f : 0.f) - part;
    }
  }
  __syncthreads();
  for (int e = tid; e < C * C; e += 256) a.TI[cbase + e] = ti[(e / C) * LP + e % C];
}

// ---------------------------------------------------------------------------
// Dense products: per chunk slot, the products of the chunk system's reverse, on the
// fp32 matrix cores (v_mfma_f32_16x16x4_f32):
//   R   = V_hat - K_a S0       U  = T^-1 R            dQ_a = dO S0^T
//   dA  = dO U^T (s <= t)      Z  = A^T dO + K' X     dK'  = U X^T
//   dU~ = T^-T Z               dL = -dU~ U^T (s < t)  dK_a = -dU~ S0^T
// Wave w owns token rows 16w..16w+15 of every C x D result; of the C x C
// results it owns the row tiles w (dA) and 3 - w (dL), so that the triangles
// give every wave the same number of tiles.  In a 16x16x4 MFMA, lane
// (l16, g) = (lane % 16, lane / 16) supplies A[l16][k] and B[k][l16] for one
// k and receives D[4g + r][l16], r = 0..3.  A k-block of 16 takes four MFMAs,
// lane group g supplying k = 16 kb + 4 g + e at step e, so every lane reads
// its A values (and, for products with a transposed B, its B values) as one
// float4.  LDS rows are padded by 4 floats: conflict-free for both access
// patterns.
// ---------------------------------------------------------------------------
// acc[ct] += A B over k-blocks kb0..kb1-1; B[k][col] row-major in LDS (stride sp)
template <int NK, int NT>
__device__ __forceinline__ void mm_nn(f32x4 (&acc)[NT], const f32x4 (&af)[NK], const float *B, int sp, int kb0,
                                      int kb1, int g, int l16) {
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    if (kb < kb0 || kb >= kb1) continue;  // wave-uniform
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float *brow = B + (16 * kb + 4 * g + e) * sp + l16;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) acc[ct] = mfma4(af[kb][e], brow[16 * ct], acc[ct]);
    }
  }
}

// acc[ct] += A Y^T for column tiles ct < ct1; Y[col][k] row-major in LDS
template <int NK, int NT>
__device__ __forceinline__ void mm_nt(f32x4 (&acc)[NT], const f32x4 (&af)[NK], const float *Y, int sp, int ct1,
                                      int g, int l16) {
#pragma unroll
  for (int kb = 0; kb < NK; ++kb)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      if (ct >= ct1) continue;  // wave-uniform
      const f32x4 b4 = *reinterpret_cast<const f32x4 *>(Y + (16 * ct + l16) * sp + 16 * kb + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ct] = mfma4(af[kb][e], b4[e], acc[ct]);
    }
}

template <int NT>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[NT]) {
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) acc[ct] = zero4();
}

template <int D, int NS>
__global__ void __launch_bounds__(256) bwd_mm_kernel(BwdArgs a) {
  constexpr int C = kBC, SP = D + 4, NKB = D / 16, NCT = D / 16, NTC = C / 16;
  constexpr int BBR = 2 * C > D ? 2 * C : D, NFR = (D / 32) * NS, FRAG = 512;
  static_assert(NTC == 4, "four waves, one 16-token row tile each");
  static_assert(4 % (D / 32) == 0, "a thread's plane entries share their rows");
  __shared__ __align__(16) float ss[D * SP];    // S0, then X, then dU~ (rows < C)
  __shared__ __align__(16) float bb[BBR * SP];  // rows < C: R, dO, Z; rows C..2C-1: U; last: S0
  __shared__ float xs[D];                       // row dots of X and S0
  float *bt = bb, *bu = bb + C * SP;
  const size_t slot = blockIdx.x;
  const SlotTokens st = slot_tokens(a, slot);
  const size_t base = slot * (size_t)C * D, cbase = slot * (size_t)C * C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int ar = 16 * w + l16;  // the A-operand row this lane supplies
  const uint16_t *S0p = a.Sc + slot * NS * (size_t)D * D, *Xp = a.Xc + slot * NS * (size_t)D * D;
  // A state from the chains' bf16 planes (summed in fp32) into padded LDS rows.
  // Entry (slice sl, k-step ks, lane) of a plane holds 8 values of column
  // 16 sl + l16, rows 32 ks + 16 (e / 4) + 4 g + e % 4; this thread's entries
  // are tid + 256 k (k < NE), all with the same ks.  Loads and LDS stores are
  // separate steps so that loads can be issued a phase ahead.
  constexpr int NE = D * D / 8 / 256;
  static_assert(NE * 256 * 8 == D * D, "plane entries per thread");
  const int ks = (tid >> 6) % (D / 32);
  auto load_planes = [&](const uint16_t *pl, bf16x8 (&r)[NE][NS]) {
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      const int sl = ((tid + 256 * k) >> 6) / (D / 32);
      const size_t off = (size_t)sl * NFR * FRAG + (size_t)(ks * NS) * FRAG + lane * 8;
#pragma unroll
      for (int p = 0; p < NS; ++p) r[k][p] = *reinterpret_cast<const bf16x8 *>(pl + off + p * FRAG);
    }
  };
  // with `dots`, also the row dots with the state in `o` (same layout) -> xs
  auto store_planes = [&](float *dst, const bf16x8 (&r)[NE][NS], const bf16x8 (&o)[NE][NS], bool dots) {
    float dot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      const int sl = ((tid + 256 * k) >> 6) / (D / 32), col = 16 * sl + l16;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = 0.f, u = 0.f;
#pragma unroll
        for (int p = 0; p < NS; ++p) {
          v += (float)r[k][p][e];
          if (dots) u += (float)o[k][p][e];
        }
        dst[(32 * ks + 16 * (e >> 2) + 4 * g + (e & 3)) * SP + col] = v;
        if (dots) dot[e] += v * u;
      }
    }
    if (dots) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float d = dot[e];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) d += __shfl_xor(d, off, kWave);
        if (l16 == 0) atomicAdd(&xs[32 * ks + 16 * (e >> 2) + 4 * g + (e & 3)], d);
      }
    }
  };
  // C x D result rows 16 rt + 4 g + r, columns 16 ct + l16
  auto put_glb = [&](float *dst, const f32x4 (&acc)[NCT], int rt, float sign) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[base + (size_t)(16 * rt + 4 * g + r) * D + 16 * ct + l16] = sign * acc[ct][r];
  };
  auto put_lds = [&](float *dst, const f32x4 (&acc)[NCT], int rt) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * rt + 4 * g + r) * SP + 16 * ct + l16] = acc[ct][r];
  };
  f32x4 acc[NCT], acc2[NCT], acs[NTC];
  f32x4 af[NKB], dof[NKB], tf[NTC];

  // (1) S0 phase: R = V_hat - K_a S0 (-> LDS), dQ_a = dO S0^T
  if (tid < D) xs[tid] = 0.f;
  bf16x8 pa[NE][NS], pb[NE][NS];  // planes: S0 now; then X (pa) and S0 (pb) for phase 3
  load_planes(S0p, pa);
  store_planes(ss, pa, pa, false);
  const bool arow = ar < st.valid;
  const size_t orow = (st.row + (arow ? ar : 0)) * D;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const size_t o = base + (size_t)ar * D + 16 * kb + 4 * g;
    const float4 kh = *reinterpret_cast<const float4 *>(a.KH + o), la = *reinterpret_cast<const float4 *>(a.LAM + o);
    af[kb] = f32x4{kh.x * __expf(la.x), kh.y * __expf(la.y), kh.z * __expf(la.z), kh.w * __expf(la.w)};
    dof[kb] = arow ? ld_do4(a.dO, orow + 16 * kb + 4 * g, a.do_bf16) : zero4();
  }
  float vh[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) vh[ct][r] = a.VH[base + (size_t)(16 * w + 4 * g + r) * D + 16 * ct + l16];
#pragma unroll
  for (int kb = 0; kb < NTC; ++kb)
    tf[kb] = *reinterpret_cast<const f32x4 *>(a.TI + cbase + (size_t)ar * C + 16 * kb + 4 * g);
  // phase 3's states, in flight during phases 1 and 2 (issued last: the
  // load counter completes in order)
  load_planes(Xp, pa);
  load_planes(S0p, pb);
  __syncthreads();
  zero_acc(acc);
  mm_nn(acc, af, ss, SP, 0, NKB, g, l16);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) bt[(16 * w + 4 * g + r) * SP + 16 * ct + l16] = vh[ct][r] - acc[ct][r];
  zero_acc(acc);
  mm_nt(acc, dof, ss, SP, NCT, g, l16);
  put_glb(a.DQA, acc, w, 1.f);
  __syncthreads();

  // (2) U = T^-1 R (T^-1 lower triangular: k-blocks up to the row tile)
  zero_acc(acc);
  mm_nn(acc, tf, bt, SP, 0, w + 1, g, l16);
  put_lds(bu, acc, w);
  __syncthreads();

  // (3) X phase: dA = dO U^T, Z = A^T dO + K' X, dK' = U X^T
  store_planes(ss, pa, pb, true);
  for (int idx = tid; idx < C * D / 4; idx += 256) {
    const int t = idx / (D / 4), j4 = idx % (D / 4);
    *reinterpret_cast<f32x4 *>(bt + t * SP + 4 * j4) =
        t < st.valid ? ld_do4(a.dO, (st.row + t) * D + 4 * j4, a.do_bf16) : zero4();
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const size_t o = base + (size_t)ar * D + 16 * kb + 4 * g;
    const float4 kn = *reinterpret_cast<const float4 *>(a.KN + o), la = *reinterpret_cast<const float4 *>(a.LAM + o);
    const float4 lc = *reinterpret_cast<const float4 *>(a.LAM + base + (size_t)(C - 1) * D + 16 * kb + 4 * g);
    af[kb] = f32x4{kn.x * __expf(lc.x - la.x), kn.y * __expf(lc.y - la.y), kn.z * __expf(lc.z - la.z),
                   kn.w * __expf(lc.w - la.w)};
  }
#pragma unroll
  for (int kb = 0; kb < NTC; ++kb)  // A^T rows: A[t][ar] for t = 16 kb + 4 g + e
#pragma unroll
    for (int e = 0; e < 4; ++e) tf[kb][e] = a.AM[cbase + (size_t)(16 * kb + 4 * g + e) * C + ar];
  __syncthreads();
  zero_acc(acs);
  mm_nt(acs, dof, bu, SP, w + 1, g, l16);
#pragma unroll
  for (int ct = 0; ct < NTC; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * g + r, s2 = 16 * ct + l16;
      a.DA[cbase + (size_t)t * C + s2] = s2 <= t ? acs[ct][r] : 0.f;
    }
  zero_acc(acc);
  mm_nn(acc, tf, bt, SP, w, NTC, g, l16);  // A lower triangular: t >= s
  mm_nn(acc, af, ss, SP, 0, NKB, g, l16);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) af[kb] = *reinterpret_cast<const f32x4 *>(bu + ar * SP + 16 * kb + 4 * g);
  zero_acc(acc2);
  mm_nt(acc2, af, ss, SP, NCT, g, l16);
  put_glb(a.DKP, acc2, w, 1.f);
  __syncthreads();  // every read of dO and X is done
  put_lds(bt, acc, w);
  if (tid < D) a.XS[slot * D + tid] = xs[tid];
#pragma unroll
  for (int kb = 0; kb < NTC; ++kb)  // T^-T rows: T^-1[t][ar]
#pragma unroll
    for (int e = 0; e < 4; ++e) tf[kb][e] = a.TI[cbase + (size_t)(16 * kb + 4 * g + e) * C + ar];
  __syncthreads();

  // (4) dU~ = T^-T Z (upper triangular: k-blocks from the row tile on)
  zero_acc(acc);
  mm_nn(acc, tf, bt, SP, w, NTC, g, l16);
  put_glb(a.DU, acc, w, 1.f);
  put_lds(ss, acc, w);
  __syncthreads();

  // (5) dL = -dU~ U^T for row tile 3 - w, then dK_a = -dU~ S0^T
  const int tw = NTC - 1 - w;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    af[kb] = *reinterpret_cast<const f32x4 *>(ss + (16 * tw + l16) * SP + 16 * kb + 4 * g);
  zero_acc(acs);
  mm_nt(acs, af, bu, SP, tw + 1, g, l16);
#pragma unroll
  for (int ct = 0; ct < NTC; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tw + 4 * g + r, s2 = 16 * ct + l16;
      a.DL[cbase + (size_t)t * C + s2] = s2 < t ? -acs[ct][r] : 0.f;
    }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) af[kb] = *reinterpret_cast<const f32x4 *>(ss + ar * SP + 16 * kb + 4 * g);
  __syncthreads();  // every read of U and Z is done
  store_planes(bb, pb, pb, false);
  __syncthreads();
  zero_acc(acc);
  mm_nt(acc, af, bb, SP, NCT, g, l16);
  put_glb(a.DKA, acc, w, -1.f);
}

// sum over the 16 lanes of a lane group (lane bits 0-3)
__device__ __forceinline__ float group16_sum(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

template <bool BF, int N>
__device__ __forceinline__ void ldn(const void *p, size_t i, float (&o)[N]) {
  if constexpr (N == 8)
    ld8<BF>(p, i, o);
  else
    ld4<BF>(p, i, o);
}

template <int N>
__device__ __forceinline__ void stn(float *p, const float (&x)[N]) {
#pragma unroll
  for (int v = 0; v < N / 4; ++v)
    reinterpret_cast<float4 *>(p)[v] = float4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
}

// ---------------------------------------------------------------------------
// Gram backprop: per chunk slot, on the fp32 matrix cores.  With the pair
// decay p_ts = e^{Lambda_t - Lambda_s} (per channel), s <= t:
//   rows    RA_t = sum_s dA_ts kn_s p_ts,   RL_t = sum_s dL_ts kn_s p_ts
//   columns CS_s = sum_t (dA_ts q_tilde_t + dL_ts k_hat_t) p_ts
// Wave w owns token block w (16 tokens) of RA, RL and CS: the triangles give
// every wave five 16-token k-blocks.  Rows split the decay at Q = Lambda of
// the block's first token, RA_t = e^{Lambda_t - Q} sum_s dA_ts kn_s e^{Q -
// Lambda_s}; columns at R = Lambda of the block's last token, CS_s =
// e^{R - Lambda_s} sum_t (...) e^{Lambda_t - R}.  Every factor is <= 1 except
// over the own block, where it reaches e^{range}; past range 60 the own block
// is summed pair by pair instead.  Column j of MFMA tile ct is channel
// NCT j + ct, so a lane's values of one token are NCT consecutive channels.
// Then per token the gradients of q_tilde, k_hat, kn and Lambda, their chains
// back to the inputs (gates, read-out gain, SiLU + l2), and the reverse
// cumulative sum of dLambda over the chunk (= d log alpha); the chunk's
// partial sums of dgamma go to gpart.
// ---------------------------------------------------------------------------
template <int D, bool BF>
__global__ void __launch_bounds__(256) bwd_gramback_kernel(BwdArgs a) {
  constexpr int C = kBC, NCT = D / 16, NV = NCT / 4, SPD = D + 4;
  constexpr float kMaxRange = 60.f;
  constexpr int IKN = 0, ILA = 1, IQT = 2, IKH = 3;
  static_assert(C == 64, "four waves, one 16-token block each");
  // kn, Lambda, q_tilde and k_hat of the chunk, rows padded to SPD; once every
  // wave is past its products and per-token work, the first holds dLambda
  // (then d log alpha) and the second the per-(wave, lane group) partial sums
  __shared__ __align__(16) float stg[4][C * SPD];
  float *dl = stg[IKN], *sk = stg[ILA], *gp = stg[ILA] + 16 * D;
  const size_t slot = blockIdx.x;
  const SlotTokens st = slot_tokens(a, slot);
  const int hd = st.head;
  const size_t base = slot * (size_t)C * D, cbase = slot * (size_t)C * C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int c0 = NCT * l16;  // first channel of this lane
  {
    const float *src[4] = {a.KN, a.LAM, a.QT, a.KH};
    for (int idx = tid; idx < C * D / 4; idx += 256) {
      const int t = idx / (D / 4), j4 = idx % (D / 4);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(stg[q] + t * SPD + 4 * j4) =
            *reinterpret_cast<const float4 *>(src[q] + base + (size_t)t * D + 4 * j4);
    }
  }
  __syncthreads();
  auto row = [&](int q, int t, float (&o)[NCT]) {  // staged array q, token t
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float4 x = *reinterpret_cast<const float4 *>(stg[q] + t * SPD + c0 + 4 * v);
      o[4 * v] = x.x;
      o[4 * v + 1] = x.y;
      o[4 * v + 2] = x.z;
      o[4 * v + 3] = x.w;
    }
  };
  auto rowg = [&](const float *p, int t, float (&o)[NCT]) {  // [C][D] workspace array, token t
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float4 x = *reinterpret_cast<const float4 *>(p + base + (size_t)t * D + c0 + 4 * v);
      o[4 * v] = x.x;
      o[4 * v + 1] = x.y;
      o[4 * v + 2] = x.z;
      o[4 * v + 3] = x.w;
    }
  };
  float qv[NCT], rv[NCT];
  row(ILA, 16 * w, qv);
  row(ILA, 16 * w + 15, rv);
  float rng = 0.f;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) rng = fmaxf(rng, qv[ct] - rv[ct]);
  const bool steep = wave_max(rng) > kMaxRange;
  const int kend = steep ? w : w + 1, kbeg = steep ? w + 1 : w;
  f32x4 ra[NCT], rl[NCT], cs[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) ra[ct] = rl[ct] = cs[ct] = zero4();
#pragma unroll 1
  for (int kb = 0; kb < 4; ++kb) {
    if (kb < kend) {  // rows: s = 16 kb + 4 g + e
      const float4 da4 = *reinterpret_cast<const float4 *>(a.DA + cbase + (size_t)(16 * w + l16) * C + 16 * kb + 4 * g);
      const float4 dl4 = *reinterpret_cast<const float4 *>(a.DL + cbase + (size_t)(16 * w + l16) * C + 16 * kb + 4 * g);
      const float av[4] = {da4.x, da4.y, da4.z, da4.w}, lv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float kn[NCT], ls[NCT];
        row(IKN, 16 * kb + 4 * g + e, kn);
        row(ILA, 16 * kb + 4 * g + e, ls);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float b = kn[ct] * __expf(qv[ct] - ls[ct]);
          ra[ct] = mfma4(av[e], b, ra[ct]);
          rl[ct] = mfma4(lv[e], b, rl[ct]);
        }
      }
    }
    if (kb >= kbeg) {  // columns: t = 16 kb + 4 g + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * kb + 4 * g + e;
        const float dat = a.DA[cbase + (size_t)t * C + 16 * w + l16], dlt = a.DL[cbase + (size_t)t * C + 16 * w + l16];
        float q[NCT], h[NCT], lt[NCT];
        row(IQT, t, q);
        row(IKH, t, h);
        row(ILA, t, lt);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float f = __expf(lt[ct] - rv[ct]);
          cs[ct] = mfma4(dat, q[ct] * f, cs[ct]);
          cs[ct] = mfma4(dlt, h[ct] * f, cs[ct]);
        }
      }
    }
  }
  float lc[NCT], skp[NCT], gac[NCT], dlv[4][NCT];
  row(ILA, C - 1, lc);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) skp[ct] = gac[ct] = 0.f;
#pragma unroll 1
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * w + 4 * g + r;
    float lt[NCT], q[NCT], h[NCT], kn[NCT], dqa[NCT], dka[NCT], dkp[NCT];
    row(ILA, t, lt);
    row(IQT, t, q);
    row(IKH, t, h);
    row(IKN, t, kn);
    rowg(a.DQA, t, dqa);
    rowg(a.DKA, t, dka);
    rowg(a.DKP, t, dkp);
    float RA[NCT], RL[NCT], CS[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float up = __expf(lt[ct] - qv[ct]);
      RA[ct] = up * ra[ct][r];
      RL[ct] = up * rl[ct][r];
      CS[ct] = __expf(rv[ct] - lt[ct]) * cs[ct][r];
    }
    if (steep) {  // the own block pair by pair
      for (int s2 = 16 * w; s2 <= t; ++s2) {
        const float dat = a.DA[cbase + (size_t)t * C + s2], dlt = a.DL[cbase + (size_t)t * C + s2];
        float k2[NCT], l2[NCT];
        row(IKN, s2, k2);
        row(ILA, s2, l2);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float x = k2[ct] * __expf(lt[ct] - l2[ct]);
          RA[ct] += dat * x;
          RL[ct] += dlt * x;
        }
      }
      for (int t2 = t; t2 < 16 * w + 16; ++t2) {
        const float dat = a.DA[cbase + (size_t)t2 * C + t], dlt = a.DL[cbase + (size_t)t2 * C + t];
        float q2[NCT], h2[NCT], l2[NCT];
        row(IQT, t2, q2);
        row(IKH, t2, h2);
        row(ILA, t2, l2);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) CS[ct] += (dat * q2[ct] + dlt * h2[ct]) * __expf(l2[ct] - lt[ct]);
      }
    }
    // the chains back to the inputs (q, k through SiLU and l2, the gain,
    // the gates); reductions over a token's channels stay in its 16 lanes
    const bool live = t < st.valid;
    const size_t grow = st.row + (live ? t : 0);
    float qx[NCT], kx[NCT], vx[NCT], zx[NCT], bg[NCT], wg[NCT], du[NCT];
    ldn<BF, NCT>(a.q, grow * D + c0, qx);
    ldn<BF, NCT>(a.k, grow * D + c0, kx);
    ldn<BF, NCT>(a.v, grow * D + c0, vx);
    if (a.z) {
      ldn<BF, NCT>(a.z, grow * D + c0, zx);
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) zx[ct] = 0.f;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      gate4<BF>(a.b, a.b_mode, grow, c0 + 4 * v, D, bg + 4 * v);
      gate4<BF>(a.w, a.w_mode, grow, c0 + 4 * v, D, wg + 4 * v);
    }
    rowg(a.DU, t, du);
    float sq[NCT], sn[NCT], nq = 0.f, nk = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      sq[ct] = a.normalize_qk ? silu(qx[ct]) : qx[ct];
      sn[ct] = a.normalize_qk ? silu(kx[ct]) : kx[ct];
      nq += sq[ct] * sq[ct];
      nk += sn[ct] * sn[ct];
    }
    float rq = 1.f, rk = 1.f;
    if (a.normalize_qk) {
      rq = fmaxf(sqrtf(group16_sum(nq)), 1e-12f);
      rk = fmaxf(sqrtf(group16_sum(nk)), 1e-12f);
    }
    float dqh[NCT], dkn[NCT], dzv[NCT], dbv[NCT], dwv[NCT], dvv[NCT];
    float dotq = 0.f, dotk = 0.f, sdb = 0.f, sdw = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float at = __expf(lt[ct]), rat = __expf(lc[ct] - lt[ct]);
      const float dqt = at * dqa[ct] + RA[ct], dkh = at * dka[ct] + RL[ct], dkw = rat * dkp[ct] + CS[ct];
      dlv[r][ct] = q[ct] * at * dqa[ct] + h[ct] * at * dka[ct] - kn[ct] * rat * dkp[ct] + q[ct] * RA[ct] +
                   h[ct] * RL[ct] - kn[ct] * CS[ct];
      skp[ct] += kn[ct] * rat * dkp[ct];
      const float qh = sq[ct] / rq, knv = sn[ct] / rk;
      const float gam = a.gamma ? a.gamma[(size_t)hd * D + c0 + ct] : 1.f;
      const float sg = 1.f / (1.f + expf(-zx[ct]));
      const float dyn = a.z ? 2.f * sg : 1.f;
      dqh[ct] = dqt * a.scale * gam * dyn;
      if (live) gac[ct] += dqt * a.scale * dyn * qh;
      dzv[ct] = dqt * a.scale * gam * qh * 2.f * sg * (1.f - sg);
      dkn[ct] = dkw + dkh * bg[ct];
      dbv[ct] = dkh * knv;
      dwv[ct] = du[ct] * vx[ct];
      dvv[ct] = du[ct] * wg[ct];
      sdb += dbv[ct];
      sdw += dwv[ct];
      dotq += qh * dqh[ct];
      dotk += knv * dkn[ct];
    }
    if (a.normalize_qk) {
      dotq = group16_sum(dotq);
      dotk = group16_sum(dotk);
    }
    if (a.b_mode == GDR_GATE_PER_TOKEN) sdb = group16_sum(sdb);
    if (a.w_mode == GDR_GATE_PER_TOKEN) sdw = group16_sum(sdw);
    float gq[NCT], gk[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      gq[ct] = dqh[ct];
      gk[ct] = dkn[ct];
      if (a.normalize_qk) {
        // through y = s / max(|s|, 1e-12), then s = SiLU(x)
        const float qh = sq[ct] / rq, knv = sn[ct] / rk;
        gq[ct] = rq > 1e-12f ? (gq[ct] - qh * dotq) / rq : gq[ct] / 1e-12f;
        gk[ct] = rk > 1e-12f ? (gk[ct] - knv * dotk) / rk : gk[ct] / 1e-12f;
        const float sgq = 1.f / (1.f + expf(-qx[ct])), sgk = 1.f / (1.f + expf(-kx[ct]));
        gq[ct] *= sgq * (1.f + qx[ct] * (1.f - sgq));
        gk[ct] *= sgk * (1.f + kx[ct] * (1.f - sgk));
      }
    }
    if (live) {
      const size_t o = grow * D + c0;
      if (a.dq) stn<NCT>(a.dq + o, gq);
      if (a.dk) stn<NCT>(a.dk + o, gk);
      if (a.dv) stn<NCT>(a.dv + o, dvv);
      if (a.dz && a.z) stn<NCT>(a.dz + o, dzv);
      if (a.db && a.b_mode == GDR_GATE_PER_CHANNEL) stn<NCT>(a.db + o, dbv);
      if (a.dw && a.w_mode == GDR_GATE_PER_CHANNEL) stn<NCT>(a.dw + o, dwv);
      if (l16 == 0) {
        if (a.db && a.b_mode == GDR_GATE_PER_TOKEN) a.db[grow] = sdb;
        if (a.dw && a.w_mode == GDR_GATE_PER_TOKEN) a.dw[grow] = sdw;
      }
    }
  }
  __syncthreads();  // the staged arrays are read for the last time
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[(16 * w + 4 * g + r) * SPD + c0 + ct] = dlv[r][ct];
    sk[(4 * w + g) * D + c0 + ct] = skp[ct];
    gp[(4 * w + g) * D + c0 + ct] = gac[ct];
  }
  __syncthreads();
  if (tid < D) {
    // the chunk-end decay: K' and Diag(a_C) S0 in the end state; then d log
    // alpha = the reverse cumulative sum of dLambda over the chunk
    const int ch = tid;
    float run = __expf(a.LAM[base + (size_t)(C - 1) * D + ch]) * a.XS[slot * D + ch], gs = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < 16; ++p2) {
      run += sk[p2 * D + ch];
      gs += gp[p2 * D + ch];
    }
    a.gpart[slot * D + ch] = gs;
    const bool per_ch = a.dla && a.alpha_mode == GDR_GATE_PER_CHANNEL;
    for (int t = C - 1; t >= 0; --t) {
      run += dl[t * SPD + ch];
      dl[t * SPD + ch] = run;
      if (per_ch && t < st.valid) a.dla[(st.row + t) * D + ch] = run;
    }
  }
  if (a.dla && a.alpha_mode == GDR_GATE_PER_TOKEN) {
    __syncthreads();
    const int t = tid >> 2, qq = tid & 3;
    float sv = 0.f;
    for (int j = 0; j < D / 4; ++j) sv += dl[t * SPD + qq * (D / 4) + j];
    sv += __shfl_xor(sv, 1, kWave);
    sv += __shfl_xor(sv, 2, kWave);
    if (qq == 0 && t < st.valid) a.dla[st.row + t] = sv;
  }
}

// dgamma[h][c] = sum over the batch and the chunks of the partial sums;
// one workgroup per (head, 32 channels), 8 threads per channel.
template <int D>
__global__ void __launch_bounds__(256) bwd_dgamma_kernel(BwdArgs a) {
  __shared__ float part[8][32];
  const int h = blockIdx.x / (D / 32), cl = threadIdx.x & 31, j = threadIdx.x >> 5;
  const int ch = (blockIdx.x % (D / 32)) * 32 + cl;
  float s = 0.f;
  if (a.ctab) {  // packed batch: slots entry * H + h (entries past the end hold zeros)
#pragma unroll 8
    for (int k = j; k < a.ctab_len; k += 8) s += a.gpart[((size_t)k * a.H + h) * D + ch];
  } else {
#pragma unroll 8
    for (int k = j; k < a.B * a.NC; k += 8) {
      const int b = k / a.NC, c = k % a.NC;
      s += a.gpart[((size_t)(b * a.H + h) * a.NC + c) * D + ch];
    }
  }
  part[j][cl] = s;
  __syncthreads();
  if (j == 0) {
#pragma unroll
    for (int i = 1; i < 8; ++i) s += part[i][cl];
    a.dgamma[h * D + ch] = s;
  }
}

// ---------------------------------------------------------------------------
// Output gate backward: y = n * weight * s with n = o r, r = (mean_c o_c^2 +
// eps)^(-1/2), s = sigmoid(g) (the fused gate of the forward).  For the loss
// <dy, y>: dg = dy n weight s (1 - s), do = r (u - n sum_c(u_c n_c) / dv) with
// u = dy weight s, and per workgroup the partial sums of dy n s for the
// weight's gradient.  One workgroup per (stream, 64 tokens); a wave per 16
// tokens, a lane per D / 64 channels.
// ---------------------------------------------------------------------------
template <int D, bool BF>
__global__ void __launch_bounds__(256) out_gate_bwd_kernel(OgBwdArgs a) {
  constexpr int CPL = D / 64, TB = 64, TW = TB / 4;
  __shared__ float wp[4][D];
  const size_t bh = blockIdx.x / a.ntb;
  const int tb = (int)(blockIdx.x % a.ntb), b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c0 = CPL * lane;
  float nw[CPL], acc[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    nw[u] = a.nw ? a.nw[(size_t)h * D + c0 + u] : 1.f;
    acc[u] = 0.f;
  }
#pragma unroll 4
  for (int j = 0; j < TW; ++j) {
    const int t = tb * TB + w * TW + j;
    if (t >= a.T) continue;  // uniform over the wave
    const size_t row = bh * a.T + t, yrow = ((size_t)b * a.T + t) * a.H + h;
    float o[CPL], gv[CPL], dy[CPL], ss = 0.f;
    if constexpr (CPL == 2) {  // paired channels: 8- and 4-byte loads
      const float2 o2 = *reinterpret_cast<const float2 *>(a.o + row * D + c0);
      o[0] = o2.x;
      o[1] = o2.y;
      ldc<BF, 2>(a.g, row * D + c0, gv);
      if (a.dy_bf16)
        ldc<true, 2>(a.dy, yrow * D + c0, dy);
      else
        ldc<false, 2>(a.dy, yrow * D + c0, dy);
    } else {
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        o[u] = a.o[row * D + c0 + u];
        gv[u] = ld1<BF>(a.g, row * D + c0 + u);
        dy[u] = a.dy_bf16 ? ld1<true>(a.dy, yrow * D + c0 + u) : ld1<false>(a.dy, yrow * D + c0 + u);
      }
    }
#pragma unroll
    for (int u = 0; u < CPL; ++u) ss += o[u] * o[u];
    const float r = 1.f / sqrtf(wave_sum(ss) / D + a.eps);
    float n[CPL], sg[CPL], uu[CPL], dot = 0.f;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      n[u] = o[u] * r;
      sg[u] = 1.f / (1.f + expf(-gv[u]));
      uu[u] = dy[u] * nw[u] * sg[u];
      dot += uu[u] * n[u];
    }
    dot = wave_sum(dot) / D;
    float xo[CPL], xg[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      xo[u] = r * (uu[u] - n[u] * dot);
      xg[u] = dy[u] * n[u] * nw[u] * sg[u] * (1.f - sg[u]);
      acc[u] += dy[u] * n[u] * sg[u];
    }
    stc<CPL>(a.dO + row * D + c0, xo);
    if (a.dg) stc<CPL>(a.dg + row * D + c0, xg);
  }
  if (!a.part) return;  // uniform over the block
#pragma unroll
  for (int u = 0; u < CPL; ++u) wp[w][c0 + u] = acc[u];
  __syncthreads();
  if (tid < D)
    a.part[(((size_t)b * a.ntb + tb) * a.H + h) * D + tid] = wp[0][tid] + wp[1][tid] + wp[2][tid] + wp[3][tid];
}

// d weight[h][c] = sum of the partials of every (batch, token block)
template <int D>
__global__ void __launch_bounds__(256) out_gate_dw_kernel(OgBwdArgs a) {
  __shared__ float part[8][32];
  const int h = blockIdx.x / (D / 32), cl = threadIdx.x & 31, j = threadIdx.x >> 5;
  const int ch = (blockIdx.x % (D / 32)) * 32 + cl;
  float s = 0.f;
#pragma unroll 8
  for (int k = j; k < a.B * a.ntb; k += 8) s += a.part[((size_t)k * a.H + h) * D + ch];
  part[j][cl] = s;
  __syncthreads();
  if (j == 0) {
#pragma unroll
    for (int i = 1; i < 8; ++i) s += part[i][cl];
    a.dnw[h * D + ch] = s;
  }
}

template <int D, bool BF>
hipError_t launch_out_gate_bwd_t(const OgBwdArgs &a, hipStream_t st) {
  const size_t nblk = (size_t)a.B * a.H * a.ntb;
  if (nblk > 0) hipLaunchKernelGGL((out_gate_bwd_kernel<D, BF>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  if (a.dnw) hipLaunchKernelGGL((out_gate_dw_kernel<D>), dim3((unsigned)(a.H * (D / 32))), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int NS, bool BF>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
  const unsigned nch = (unsigned)(a.ctab ? (size_t)a.H * a.ctab_len : (size_t)a.B * a.H * a.NC);
  if (nch == 0) {  // empty sequences: only dgamma (zeros)
    if (a.dgamma && a.gamma)
      hipLaunchKernelGGL((bwd_dgamma_kernel<D>), dim3((unsigned)(a.H * (D / 32))), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_prepass_kernel<D, BF>), dim3(nch), dim3(256), 0, st, a);
  hipLaunchKernelGGL((bwd_gram_kernel<D>), dim3(nch), dim3(256), 0, st, a);
  hipLaunchKernelGGL((bwd_mm_kernel<D, NS>), dim3(nch), dim3(256), 0, st, a);
  hipLaunchKernelGGL((bwd_gramback_kernel<D, BF>), dim3(nch), dim3(256), 0, st, a);
  if (a.dgamma && a.gamma)
    hipLaunchKernelGGL((bwd_dgamma_kernel<D>), dim3((unsigned)(a.H * (D / 32))), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int NS>
hipError_t launch_bwd_prep_t(const BwdArgs &a, hipStream_t st) {
  const unsigned nch = (unsigned)(a.ctab ? (size_t)a.H * a.ctab_len : (size_t)a.B * a.H * a.NC);
  hipLaunchKernelGGL((bwd_prep_kernel<D, NS>), dim3(nch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace(BwdArgs *a, ChunkArgs *f, void *ws, int B, int H, int T, int D, int NS, int nseq) {
  const int C = kBC;
  // chunk slots: uniform B * H * NC; packed H * (chunk-list length bound)
  const size_t nch = nseq > 0 ? (size_t)H * ((size_t)((T + C - 1) / C) + (size_t)nseq)
                              : (size_t)B * H * ((T + C - 1) / C);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t total = al(chunk_workspace(f, ws, nseq > 0 ? 1 : B, H, T, C, D, NS, nseq));
  unsigned char *base = static_cast<unsigned char *>(ws);
  auto take = [&](size_t bytes) {
    void *p = ws ? base + total : nullptr;
    total += al(bytes);
    return p;
  };
  void *mt = take(nch * NS * (size_t)D * D * 2), *xc = take(nch * NS * (size_t)D * D * 2);
  void *gn = take(nch * (size_t)D * D * 4);
  float **cd[9] = {&a->KN, &a->KH, &a->QT, &a->VH, &a->LAM, &a->DU, &a->DQA, &a->DKA, &a->DKP};
  float *cdp[9];
  for (int i = 0; i < 9; ++i) cdp[i] = static_cast<float *>(take(nch * (size_t)kBC * D * 4));
  float *ccp[4];
  for (int i = 0; i < 4; ++i) ccp[i] = static_cast<float *>(take(nch * (size_t)kBC * kBC * 4));
  float *gp = static_cast<float *>(take(nch * (size_t)D * 4));
  float *xs = static_cast<float *>(take(nch * (size_t)D * 4));
  if (a) {
    a->ctab = (ws && f) ? f->ctab : nullptr;
    a->ctab_len = (ws && f) ? f->ctab_len : 0;
    a->XS = xs;
    a->Mt = static_cast<uint16_t *>(mt);
    a->Xc = static_cast<uint16_t *>(xc);
    a->Gn = static_cast<float *>(gn);
    for (int i = 0; i < 9; ++i) *cd[i] = cdp[i];
    a->AM = ccp[0];
    a->TI = ccp[1];
    a->DA = ccp[2];
    a->DL = ccp[3];
    a->gpart = gp;
  }
  return total;
}

hipError_t launch_bwd_prep(const BwdArgs &a, int D, int NS, hipStream_t st) {
  if (D == 128 && NS == 2) return launch_bwd_prep_t<128, 2>(a, st);
  if (D == 128) return launch_bwd_prep_t<128, 3>(a, st);
  if (NS == 2) return launch_bwd_prep_t<64, 2>(a, st);
  return launch_bwd_prep_t<64, 3>(a, st);
}

hipError_t launch_out_gate_bwd(const OgBwdArgs &a, int D, bool g_bf16, hipStream_t st) {
  if (D == 128) return g_bf16 ? launch_out_gate_bwd_t<128, true>(a, st) : launch_out_gate_bwd_t<128, false>(a, st);
  return g_bf16 ? launch_out_gate_bwd_t<64, true>(a, st) : launch_out_gate_bwd_t<64, false>(a, st);
}

hipError_t launch_bwd(const BwdArgs &a, int D, int NS, hipStream_t st) {
  if (D == 128 && NS == 2) return launch_bwd_t<128, 2, true>(a, st);
  if (D == 128) return launch_bwd_t<128, 3, false>(a, st);
  if (NS == 2) return launch_bwd_t<64, 2, true>(a, st);
  return launch_bwd_t<64, 3, false>(a, st);
}

}  // namespace gdr
