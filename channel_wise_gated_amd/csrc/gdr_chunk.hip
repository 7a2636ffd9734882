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
// affine map (Q', O_bar, M, N); kernel 2 ("chain") carries S in fp32 through
// the chunks of one stream, split over value-column slices, and records each
// chunk-start state; kernel 3 ("output", parallel over chunks) forms
// O = Q' S_c + O_bar.
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
//   Sc : [D/16 slices][D/32][NS][64][8] bf16            B-fragments of S_c
// The contraction index of Q' and M (a state row) is in tile-pair order, the
// order in which the scan kernel's accumulator tiles of S hold it.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

constexpr float kMaxDiagRange = 40.0f;



__device__ __forceinline__ int tidx(int i, int j) { return i * (i + 1) / 2 + j; }

// Index of the pair (s-tile st, k-step kt >= st / 2) in st-major order: row
// st' holds NKC - st'/2 pairs, and sum_{st' < st} st'/2 = m (m - 1 + st % 2)
// with m = st / 2.
template <int NKC>
__device__ __forceinline__ constexpr int tf_pair(int st, int kt) {
  return st * NKC - (st / 2) * (st / 2 - 1 + st % 2) + kt - st / 2;
}

// Four fp32 values as NS bf16 planes (a 16x16x16 operand fragment).
template <int NS>
struct Split4 {
  s16x4 p[NS];
};
template <int NS>
__device__ __forceinline__ Split4<NS> split4(const float x[4]) {
  Split4<NS> r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t h[NS];
    split<NS>(x[e], h);
#pragma unroll
    for (int p = 0; p < NS; ++p) r.p[p][e] = (short)h[p];
  }
  return r;
}
// Product of pre-split operands, smallest plane products first.
template <int NS>
__device__ __forceinline__ f32x4 mfma16_pre(const Split4<NS> &a, const Split4<NS> &b, f32x4 c) {
#pragma unroll
  for (int s = NS - 1; s >= 0; --s)
#pragma unroll
    for (int pa = 0; pa <= s; ++pa)
      c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.p[pa], b.p[s - pa], c, 0, 0, 0);
  return c;
}

template <int NS>
__device__ __forceinline__ f32x4 mfma16_split(const float a[4], const float b[4], f32x4 c) {
  return mfma16_pre<NS>(split4<NS>(a), split4<NS>(b), c);
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
  static constexpr int NB = C / 16, NKC = C / 32, NKD = D / 32;
  static constexpr int TILE_LD = 20;       // padded 16 x 16 fp32 tiles
  static constexpr int TILE_SZ = 16 * TILE_LD;
  static constexpr int NTILES = NB * (NB + 1) / 2;
  static constexpr int FRAG = 64 * 8;      // bf16 per fragment plane
  static constexpr int STAGE = NKC * 2 * NS * FRAG;
  // (s-tile st, token k-step kt) pairs with kt >= st / 2, in st-major order:
  // the A-fragments of T^-T that are not identically zero
  static constexpr int NPAIR = NB * NKC - (NB / 2) * (NB / 2 - 1);
  static constexpr int TF_HALVES = NPAIR * NS * FRAG / 2;  // in floats
  static constexpr int LT_SZ = NTILES * TILE_SZ > TF_HALVES ? NTILES * TILE_SZ : TF_HALVES;
  static constexpr int STG_SZ = NTILES * D > STAGE / 2 ? NTILES * D : STAGE / 2;  // in floats
  // float offsets
  static constexpr int KCF = 0;                        // [NB][NKD][64][8]  kn * Cf
  static constexpr int LT = KCF + C * D;               // [NTILES][TILE_SZ] L, then T^-1 fragments
  static constexpr int CUM = LT + LT_SZ;               // [NB + 1][D]      block-start log decay
  static constexpr int NRM = CUM + (NB + 1) * D;       // [2][C]           inverse norms of q, k
  static constexpr int STG = NRM + 2 * C;              // pair decay table, then R staging (bf16)
  // In the last phase the KCF region is dead and holds v_hat = w * v (fp32,
  // same layout), loaded during the pre-pass.
  static constexpr size_t bytes = sizeof(float) * ((size_t)STG + STG_SZ) + sizeof(int) * NB;
  static constexpr int WAVES = NB > D / 16 ? NB : D / 16;
  // The backward's recompute (PP) also forms G = Q'^T dO: dO of the chunk
  // [C][D + 4] and one column pair's Q' [C][36] in fp32, after the rest.
  static constexpr int DOS_LD = D + 4, QS_LD = 36;
  static constexpr int DOS = (int)((bytes + 15) / 16 * 4);  // float offset, 16-byte aligned
  static constexpr int QS = DOS + C * DOS_LD;
  static constexpr size_t pp_bytes = sizeof(float) * ((size_t)QS + C * QS_LD);
};

// Channel held by (lane group g, k-step ks, element e) in tile-pair order.
__device__ __forceinline__ int tp_chan(int ks, int g, int e) { return 32 * ks + 16 * (e >> 2) + 4 * g + (e & 3); }

// ============================================================================
// Kernel 1: one workgroup per (stream, chunk); each wave owns one token block
// i (16 tokens; a permutation of the waves balances the SIMDs) and channel
// tile m = wave.  Per-token values live in the registers of
// the owning wave in "row-operand" layout: lane (t = l%16, g = l/16) holds
// channels tp_chan(ks, g, e) of token t.
// ============================================================================
// SA (scalar decay): log alpha is one value per token (GDN, DeltaNet), given
// per token or as ONES.  Every decay factor is then a scalar per token or per
// block pair, which leaves the channel dimension of the Gram products free of
// per-pair factors: kn * Cf is split into bf16 planes once, in the pre-pass,
// and the pair factor D_ij scales the accumulated tile.
// PP: also write what the backward reads of the chunk: the per-token vectors
// kn, k_hat, q_tilde, v_hat and the in-chunk cumulative log decay ([slot][C][D]
// fp32 each, zero on padding rows), the chunk system's A and T^-1
// ([slot][C][C] fp32 each), M^T in M's A-fragment plane layout and G =
// Q'^T dO in N's accumulator-tile layout (for the reverse chain of state
// gradients, X <- M^T X + G); Q' itself is not written.
// DOBF (PP only): dO is bf16 (else fp32).
template <int C, int D, int NS, bool BF, bool SA, bool PP = false, bool DOBF = false>
__global__ void __launch_bounds__(512) chunk_intra_kernel(ChunkArgs a) {
  static_assert(!SA || NS == 2, "the scalar-decay kernel keeps kn * Cf as two bf16 planes in the kn * Cf region");
  using Lds = IntraLds<C, D, NS>;
  constexpr int NB = C / 16, NKC = C / 32, NKD = D / 32, NMT = D / 16;
  constexpr int TILE_LD = Lds::TILE_LD, TILE_SZ = Lds::TILE_SZ, FRAG = Lds::FRAG;
  static_assert(NB <= 8 && NMT <= 8, "one wave per token block and per channel tile");
  // off-diagonal L tiles are stored as NS bf16 planes of A-fragments when those
  // fit the fp32 tile slot (NS = 2), else in fp32
  constexpr bool LPRE = NS * 256 <= 2 * TILE_SZ;

  extern __shared__ __align__(16) unsigned char smem[];
  float *sm = reinterpret_cast<float *>(smem);
  float *kcf = sm + Lds::KCF;
  uint16_t *kcs = reinterpret_cast<uint16_t *>(kcf);  // scalar decay: kn * Cf as bf16 planes
  float *cum = sm + Lds::CUM;
  float *inq = sm + Lds::NRM;
  float *ink = inq + C;
  float *Lt = sm + Lds::LT;
  uint16_t *tf = reinterpret_cast<uint16_t *>(Lt);  // T^-1 fragments, once C2 is done
  uint16_t *rst = reinterpret_cast<uint16_t *>(sm + Lds::STG);
  int *dflag = reinterpret_cast<int *>(sm + Lds::STG + Lds::STG_SZ);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int l16 = lane & 15, g = lane >> 4;
  const size_t ch = blockIdx.x;  // chunk slot in the workspace
  int h, tvalid;
  size_t row0;  // first token row
  if (a.ctab) {  // packed batch: slot = entry * H + head
    const int4 e = a.ctab[ch / a.H];
    if (e.x < 0) {  // past the last chunk (the grid is an upper bound)
      if constexpr (PP) {  // the backward still reads the slot: zeros
        float *pp[8] = {a.pp_kn, a.pp_kh, a.pp_qt, a.pp_vh, a.pp_lam, a.pp_am, a.pp_ti, a.pp_g};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int n4 = q < 5 ? C * D / 4 : (q < 7 ? C * C / 4 : D * D / 4);
          float4 *dst = reinterpret_cast<float4 *>(pp[q] + ch * (size_t)n4 * 4);
          for (int x = threadIdx.x; x < n4; x += blockDim.x) dst[x] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      return;
    }
    h = (int)(ch % a.H);
    row0 = (size_t)h * a.T + e.z;
    tvalid = e.w;
  } else {
    const size_t bh = ch / a.ncs;
    const int c = a.c0 + (int)(ch % a.ncs);
    h = (int)(bh % a.H);
    row0 = bh * (size_t)a.T + (size_t)c * C;
    tvalid = min(C, a.T - c * C);
  }
  // The last chunk of a sequence may be short: its tokens from `tvalid` on
  // are padding, read at the last real row and turned into identity steps
  // (log alpha = 0, no erase, no write); their outputs are never stored.
  const bool norm = a.normalize_qk != 0;
  const bool rowwave = wave < NB;
  // Token block of this wave.  The triangular phases give block i work in
  // proportion to i + 1 (or to NB - i); waves w and w + 4 are dealt to one
  // SIMD, so with 8 blocks wave w >= 4 takes block 11 - w and every SIMD holds
  // a pair of blocks whose work sums to the same total.
  const int i = (NB == 8 && wave >= 4) ? (wave ^ 3) : wave;
  const int t = 16 * i + l16;               // token of this lane (row-operand layout)
  const bool tok_ok = t < tvalid;
  const size_t rowt = row0 + min(t, tvalid - 1);  // row the lane's inputs are read from
  auto rowc = [&](int tt) { return row0 + min(tt, tvalid - 1); };

  // PP: the lane's 8 values of k-step ks (channels tp_chan(ks, g, 0..7): two
  // runs of 4) into row t of a [slot][C][D] array
  auto pp_store = [&](float *arr, int ks, const float x[8]) {
    float *r = arr + (ch * (size_t)C + t) * D + 32 * ks + 4 * g;
    *reinterpret_cast<float4 *>(r) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(r + 16) = make_float4(x[4], x[5], x[6], x[7]);
  };
  float pp_lam[PP ? NKD : 1][8];  // PP: the in-block decay prefix, kept for Lambda

  // ----------------------------------------------------------- A: pre-pass
  // QRp / KRp: NS bf16 planes of qt * R and k_hat * R, R = exp(P_t), P the
  // inclusive log-decay prefix inside the block (<= 0).
  bf16x8 QRp[NKD][NS], KRp[NKD][NS];
  Raw4<BF> vraw[NKD][2];    // v of this lane's token and channels
  Gate4<BF> wraw[NKD][2];   // w of the same
  const void *any = a.q;    // a valid 16-byte-aligned address for unused loads
  if (rowwave) {
    float qv[NKD][8], kv[NKD][8], lv[NKD][8];
    Raw4<BF> zg[NKD][2];
    Raw4<false> gm[NKD][2];
    Gate4<BF> bg[NKD][2];
    Gate4<false> lg[NKD][2];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c0 = 32 * ks + 16 * hh + 4 * g;
        ld4<BF>(a.q, rowt * D + c0, &qv[ks][4 * hh]);
        ld4<BF>(a.k, rowt * D + c0, &kv[ks][4 * hh]);
        // optional tensors: the pointer is selected, the load is unconditional
        zg[ks][hh] = *reinterpret_cast<const Raw4<BF> *>(
            a.z ? reinterpret_cast<const char *>(a.z) + (rowt * D + c0) * (BF ? 2 : 4) : reinterpret_cast<const char *>(any));
        gm[ks][hh] = *reinterpret_cast<const Raw4<false> *>(
            a.gamma ? reinterpret_cast<const char *>(a.gamma + (size_t)h * D + c0) : reinterpret_cast<const char *>(any));
        bg[ks][hh] = gate_load<BF>(a.b, a.b_mode, rowt, c0, D, any);
        if constexpr (!SA) lg[ks][hh] = gate_load<false>(a.log_alpha, a.alpha_mode, rowt, c0, D, any);
      }
    // scalar decay: one log alpha per token (0 in ONES mode and for padding)
    float la1 = 0.f;
    if constexpr (SA) {
      const bool tokm = a.alpha_mode == GDR_GATE_PER_TOKEN;
      la1 = ld1<false>(tokm ? reinterpret_cast<const void *>(a.log_alpha) : any, tokm ? rowt : 0);
      la1 = tokm && tok_ok ? la1 : 0.f;
    }
    const float bconst = tok_ok ? gate_const(a.b_mode) : 0.f;
    if constexpr (!SA) {
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) gate8<false>(lg[ks], a.alpha_mode, 0.f, tok_ok, lv[ks]);
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (norm) { qv[ks][e] = silu(qv[ks][e]); kv[ks][e] = silu(kv[ks][e]); }
        sq += qv[ks][e] * qv[ks][e];
        sk += kv[ks][e] * kv[ks][e];
      }
    sq += __shfl_xor(sq, 16, kWave); sq += __shfl_xor(sq, 32, kWave);
    sk += __shfl_xor(sk, 16, kWave); sk += __shfl_xor(sk, 32, kWave);
    const float nq = norm ? inv_norm(sq) : 1.f, nk = norm ? inv_norm(sk) : 1.f;
    if (g == 0) { inq[t] = nq; ink[t] = nk; }
    // inclusive prefix of log alpha over the 16 tokens of the block: a scan
    // within each row of 16 lanes by DPP row shifts of 1, 2, 4, 8 (lanes
    // without a source add 0)
    auto row_scan = [](float x) {
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, false));
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, false));
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, false));
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, false));
      return x;
    };
    // block total (lane 15 of the row), broadcast within each row of 16 lanes
    // by a DPP row broadcast (no trip through the LDS unit)
    auto row_total = [](float x) {
      return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xF, 0xF, false));
    };
    float P1 = 0.f, tot1 = 0.f, R1 = 1.f, Cf1 = 1.f;  // scalar decay: per token
    if constexpr (SA) {
      P1 = row_scan(la1);
      tot1 = row_total(P1);
      R1 = __expf(P1);
      Cf1 = __expf(tot1 - P1);
    } else {
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) lv[ks][e] = row_scan(lv[ks][e]);
    }
    float range = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      // per-channel factors of this k-step: the erase gate, and the read-out
      // multiplier 2 sigma(z) gamma (optional inputs tested once per k-step)
      float bbv[8], fq[8];
      gate8<BF>(bg[ks], a.b_mode, bconst, tok_ok, bbv);
      if (a.z) {
#pragma unroll
        for (int e = 0; e < 8; ++e) fq[e] = a.scale * two_sigmoid(raw_elem<BF>(zg[ks][e / 4], e % 4));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) fq[e] = a.scale;
      }
      if (a.gamma) {
#pragma unroll
        for (int e = 0; e < 8; ++e) fq[e] *= raw_elem<false>(gm[ks][e / 4], e % 4);
      }
      float QR[8], KR[8], KC[8], tot[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float R, Cf;
        if constexpr (SA) {
          tot[e] = tot1;
          R = R1;
          Cf = Cf1;
        } else {
          const float P = lv[ks][e];
          tot[e] = row_total(P);
          R = __expf(P);
          Cf = __expf(tot[e] - P);
        }
        range = fmaxf(range, -tot[e]);
        const float qt = fq[e] * qv[ks][e] * nq;
        const float kn = kv[ks][e] * nk;
        QR[e] = qt * R;
        KR[e] = bbv[e] * kn * R;
        KC[e] = kn * Cf;
      }
      if constexpr (PP) {
        float kn8[8], kh8[8], qt8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kn = tok_ok ? kv[ks][e] * nk : 0.f;
          kn8[e] = kn;
          kh8[e] = bbv[e] * kn;
          qt8[e] = tok_ok ? fq[e] * qv[ks][e] * nq : 0.f;
          if constexpr (SA) pp_lam[ks][e] = P1;
          else pp_lam[ks][e] = lv[ks][e];
        }
        pp_store(a.pp_kn, ks, kn8);
        pp_store(a.pp_kh, ks, kh8);
        pp_store(a.pp_qt, ks, qt8);
      }
      if (l16 == 15) {  // channels tp_chan(ks, g, 0..3) and (ks, g, 4..7) are two runs of 4
        float *cb = cum + (i + 1) * D + 32 * ks + 4 * g;
        *reinterpret_cast<float4 *>(cb) = make_float4(tot[0], tot[1], tot[2], tot[3]);
        *reinterpret_cast<float4 *>(cb + 16) = make_float4(tot[4], tot[5], tot[6], tot[7]);
      }
      split8<NS>(QR, QRp[ks]);
      split8<NS>(KR, KRp[ks]);
      if constexpr (SA) {  // A-fragment planes of kn * Cf for the Gram products
        bf16x8 kp[NS];
        split8<NS>(KC, kp);
#pragma unroll
        for (int p = 0; p < NS; ++p)
          *reinterpret_cast<bf16x8 *>(kcs + (((i * NKD + ks) * NS + p) * 64 + lane) * 8) = kp[p];
      } else {
        float4 *dst = reinterpret_cast<float4 *>(kcf + ((i * NKD + ks) * 64 + lane) * 8);
        dst[0] = make_float4(KC[0], KC[1], KC[2], KC[3]);
        dst[1] = make_float4(KC[4], KC[5], KC[6], KC[7]);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) range = fmaxf(range, __shfl_xor(range, off, kWave));
    if (lane == 0) dflag[i] = range > kMaxDiagRange;
  }
  __syncthreads();
  // cumulative block-start log decay: cum[m][c] = sum_{m' < m} total_{m'}[c]
  if (tid < D) {
    float s = 0.f;
    cum[tid] = 0.f;
    for (int m = 1; m <= NB; ++m) {
      s += cum[m * D + tid];
      cum[m * D + tid] = s;
    }
  }
  __syncthreads();

  if constexpr (PP) {  // Lambda_t = block-start cumulative log decay + in-block prefix
    if (rowwave) {
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        float x[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4 f = *reinterpret_cast<const float4 *>(cum + i * D + 32 * ks + 16 * hh + 4 * g);
          x[4 * hh] = f.x + pp_lam[ks][4 * hh];
          x[4 * hh + 1] = f.y + pp_lam[ks][4 * hh + 1];
          x[4 * hh + 2] = f.z + pp_lam[ks][4 * hh + 2];
          x[4 * hh + 3] = f.w + pp_lam[ks][4 * hh + 3];
        }
        pp_store(a.pp_lam, ks, x);
      }
    }
  }

  // pair decay factors D_ij[c] = exp(cum_i - cum_{j+1}) for j <= i, one
  // exponential per (pair, channel), kept in the (still unused) staging area
  float *dtab = reinterpret_cast<float *>(rst);
  if constexpr (!SA) {  // scalar decay: D_ij is one exponential per pair, formed in B
    // thread <-> channel c; the pairs are dealt out over the P groups of D
    // threads (a group is whole waves, so the pair test is a scalar branch)
    constexpr int P = 64 * Lds::WAVES / D;
    static_assert(D % 64 == 0 && (64 * Lds::WAVES) % D == 0, "whole waves per channel group");
    const int c = tid % D, part = wave / (D / 64);
    float cm[NB + 1];
#pragma unroll
    for (int m = 0; m <= NB; ++m) cm[m] = cum[m * D + c];
#pragma unroll
    for (int ii = 0; ii < NB; ++ii)
#pragma unroll
      for (int jj = 0; jj <= ii; ++jj) {
        const int pr = tidx(ii, jj);
        if (pr % P != part) continue;
        const float dd = cm[ii] - cm[jj + 1];
        dtab[pr * D + c] = __expf(jj < ii ? fminf(dd, 0.f) : dd);
      }
    __syncthreads();
  }

  // per-lane factor vectors for this wave's channels (row-operand layout)
  auto cum8 = [&](int m, int ks, float out[8]) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float4 f = *reinterpret_cast<const float4 *>(cum + m * D + 32 * ks + 16 * hh + 4 * g);
      out[4 * hh] = f.x; out[4 * hh + 1] = f.y; out[4 * hh + 2] = f.z; out[4 * hh + 3] = f.w;
    }
  };

  // ----------------------------------------------------------- B: L and A tiles
  // Tiles are computed transposed (rows s, cols t) so that the accumulator
  // lane <-> t:  L^T[s][t] = sum_c (kn_s Cf_s D_ij)_c (k_hat_t R_t)_c with
  // Cf_s = exp(Lambda_end(j) - Lambda_s), R_t = exp(Lambda_t - Lambda_start(i))
  // and D_ij = exp(Lambda_start(i) - Lambda_end(j)); the product is
  // exp(Lambda_t - Lambda_s).  For j < i every factor is in (0, 1].
  bf16x8 afr[NKC][NS];  // A-fragments of A (row block i), tile-pair order over s
#pragma unroll
  for (int kk = 0; kk < NKC; ++kk)
#pragma unroll
    for (int p = 0; p < NS; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) afr[kk][p][e] = (__bf16)0.f;

  if (rowwave) {
#pragma unroll 1
    for (int j = 0; j <= i; ++j) {
      f32x4 accL = zero4(), accA = zero4();
      if constexpr (SA) {
        // kn * Cf of block j as ready A-fragments; the scalar pair factor
        // D_ij scales the accumulated tiles
        bf16x8 kc[NKD][NS];
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) load_frag<NS>(kcs + ((j * NKD + ks) * NS * 64 + lane) * 8, FRAG, kc[ks]);
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) {
          accL = mfma32_split<NS>(kc[ks], KRp[ks], accL);
          accA = mfma32_split<NS>(kc[ks], QRp[ks], accA);
        }
        const float dd = cum[i * D] - cum[(j + 1) * D];
        const float dij = __expf(j < i ? fminf(dd, 0.f) : dd);
#pragma unroll
        for (int r = 0; r < 4; ++r) { accL[r] *= dij; accA[r] *= dij; }
      } else {
      // every LDS operand of the pair is read first, so the reads overlap and
      // each k-step waits only for its own
      float4 kf[NKD][2], df[NKD][2];
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const float4 *src = reinterpret_cast<const float4 *>(kcf + ((j * NKD + ks) * 64 + lane) * 8);
        kf[ks][0] = src[0];
        kf[ks][1] = src[1];
        // D_ij = exp(cum_i - cum_{j+1}): <= 1 for j < i (clamped against
        // rounding); for j = i it is exp(-total_i) >= 1, bounded by the
        // block's decay range (wide ranges take the exact path below).
        const float4 *dp = reinterpret_cast<const float4 *>(dtab + tidx(i, j) * D + 32 * ks + 4 * g);
        df[ks][0] = dp[0];  // channels tp_chan(ks, g, 0..3)
        df[ks][1] = dp[4];  // and (ks, g, 4..7)
      }
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const float4 f0 = kf[ks][0], f1 = kf[ks][1], d0 = df[ks][0], d1 = df[ks][1];
        float x[8] = {f0.x * d0.x, f0.y * d0.y, f0.z * d0.z, f0.w * d0.w,
                      f1.x * d1.x, f1.y * d1.y, f1.z * d1.z, f1.w * d1.w};
        bf16x8 kc[NS];
        split8<NS>(x, kc);
        accL = mfma32_split<NS>(kc, KRp[ks], accL);
        accA = mfma32_split<NS>(kc, QRp[ks], accA);
      }
      }
      // lane (col t, group g) holds rows s = 16j + 4g + r
      if (j == i) {
        if (dflag[i]) {
          // a block whose decay range is too wide for one pivot: exact
          // pairwise exponentials exp(sum_{x=s+1}^{t} log alpha_x)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s2 = 16 * j + 4 * g + r;
            float lsum = 0.f, asum = 0.f;
            if (s2 <= t) {
              const size_t r2 = rowc(s2);
              for (int c = 0; c < D; ++c) {
                float dec = 0.f;
                for (int xx = s2 + 1; xx <= t; ++xx)
                  if (xx < tvalid) dec += log_alpha_at(a.log_alpha, a.alpha_mode, row0 + xx, c, D);
                const float pi = __expf(dec);
                const float kraw_s = ld1<BF>(a.k, r2 * D + c), kraw_t = ld1<BF>(a.k, rowt * D + c);
                const float kns = (norm ? silu(kraw_s) : kraw_s) * ink[s2];
                const float knt = (norm ? silu(kraw_t) : kraw_t) * ink[t];
                const float bb = tok_ok ? gate_at<BF>(a.b, a.b_mode, rowt, c, D) : 0.f;
                const float qraw = ld1<BF>(a.q, rowt * D + c);
                const float dy = a.z ? two_sigmoid(ld1<BF>(a.z, rowt * D + c)) : 1.f;
                const float gg = a.gamma ? a.gamma[(size_t)h * D + c] : 1.f;
                const float qt = a.scale * gg * dy * (norm ? silu(qraw) : qraw) * inq[t];
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
      if constexpr (PP) {  // A[t][s] (s = 16 j + 4 g + r), zero on padding rows and columns
        float4 av;
        av.x = tok_ok && 16 * j + 4 * g < tvalid ? accA[0] : 0.f;
        av.y = tok_ok && 16 * j + 4 * g + 1 < tvalid ? accA[1] : 0.f;
        av.z = tok_ok && 16 * j + 4 * g + 2 < tvalid ? accA[2] : 0.f;
        av.w = tok_ok && 16 * j + 4 * g + 3 < tvalid ? accA[3] : 0.f;
        *reinterpret_cast<float4 *>(a.pp_am + (ch * (size_t)C + t) * C + 16 * j + 4 * g) = av;
      }
      if (j == i || !LPRE) {  // diagonal tile: fp32, row-major [t][s], for the leaf inverse
        *reinterpret_cast<float4 *>(Lt + tidx(i, j) * TILE_SZ + l16 * TILE_LD + 4 * g) =
            make_float4(accL[0], accL[1], accL[2], accL[3]);
      } else {  // off-diagonal: this lane's A-fragment (row t, k = 4g..4g+3) as NS bf16 planes
        const float lv4[4] = {accL[0], accL[1], accL[2], accL[3]};
        const Split4<NS> ls = split4<NS>(lv4);
        uint16_t *lt = reinterpret_cast<uint16_t *>(Lt + tidx(i, j) * TILE_SZ);
#pragma unroll
        for (int p = 0; p < NS; ++p) *reinterpret_cast<s16x4 *>(lt + p * 256 + lane * 4) = ls.p[p];
      }
      uint16_t hp[4][NS];
#pragma unroll
      for (int r = 0; r < 4; ++r) split<NS>(accA[r], hp[r]);
      // afr[j/2] elements 4*(j%2) + r  (j is uniform: compares, no dynamic indexing)
#pragma unroll
      for (int kk = 0; kk < NKC; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          if (j == 2 * kk + hf) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int p = 0; p < NS; ++p) afr[kk][p][4 * hf + r] = __builtin_bit_cast(__bf16, hp[r][p]);
          }
    }
    if constexpr (PP) {  // A's tiles above the diagonal
      for (int j = i + 1; j < NB; ++j)
        *reinterpret_cast<float4 *>(a.pp_am + (ch * (size_t)C + t) * C + 16 * j + 4 * g) =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();

  // v and w of this lane's token and channels, only needed in the last phase:
  // issued here so that their latency hides behind the triangular inverse
  if (rowwave) {
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c0 = 32 * ks + 16 * hh + 4 * g;
        vraw[ks][hh] = *reinterpret_cast<const Raw4<BF> *>(reinterpret_cast<const char *>(a.v) +
                                                          (rowt * D + c0) * (BF ? 2 : 4));
        wraw[ks][hh] = gate_load<BF>(a.w, a.w_mode, rowt, c0, D, any);  // padding: zeroed at use
      }
  }

  // -------------------------------------------------- C1: leaf inverses
  // X = (I + N)^-1 for the strictly lower 16 x 16 diagonal block N, by fp32
  // forward substitution (column-parallel, right-looking): once rows < s are
  // done, row s of X is final; it is broadcast and every later row t takes
  // off N[t][s] X[s][:].  Lane (column j = l16, group g) holds rows 4g..4g+3
  // of X.  Unlike a Neumann-product form (whose powers of N grow
  // combinatorially and cancel), this keeps the rounding error at the level
  // of the system's conditioning.
  if (rowwave) {
    float *Tii = Lt + tidx(i, i) * TILE_SZ;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (4 * g + r) == l16 ? 1.f : 0.f;
#pragma unroll
    for (int s_ = 0; s_ < 16; ++s_) {
      // X[s][j] from the lane of group s/4 that holds column j
      const float xs = __shfl(x[s_ % 4], l16 + 16 * (s_ / 4), kWave);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] -= Tii[(4 * g + r) * TILE_LD + s_] * xs;  // N[t][s] = 0 for t <= s
    }
    __builtin_amdgcn_wave_barrier();  // every lane has read N before X overwrites it
#pragma unroll
    for (int r = 0; r < 4; ++r) Tii[(4 * g + r) * TILE_LD + l16] = x[r];
  }
  __syncthreads();

  // -------------------------------------------------- C2: blocked forward substitution
  // X[i][q] = -X[i][i] sum_{j=q}^{i-1} L[i][j] X[j][q].  The owner wave of
  // token block q owns column block q and keeps X[j][q] in accumulator layout -- the B-operand layout of
  // the 16x16x16 product -- so the waves need no barrier until the write-back.
  {
    f32x4 Xc[NB];
    Split4<NS> Xs[NB];  // the planes of each finished X[j][q]
#pragma unroll
    for (int j = 0; j < NB; ++j) Xc[j] = zero4();
    const int q = i;  // column block of this wave
    if (rowwave) {
#pragma unroll
      for (int jj = 0; jj < NB; ++jj)
        if (jj == q) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Xc[jj][r] = Lt[tidx(jj, jj) * TILE_SZ + (4 * g + r) * TILE_LD + l16];
          const float xv[4] = {Xc[jj][0], Xc[jj][1], Xc[jj][2], Xc[jj][3]};
          Xs[jj] = split4<NS>(xv);
        }
#pragma unroll
      for (int ii = 1; ii < NB; ++ii) {
        if (ii <= q) continue;
        f32x4 W = zero4();
#pragma unroll
        for (int j = 0; j < NB - 1; ++j) {
          if (j < q || j >= ii) continue;
          Split4<NS> la;  // L[ii][j], pre-split when the planes fit the tile slot
          if constexpr (LPRE) {
            const uint16_t *lt = reinterpret_cast<const uint16_t *>(Lt + tidx(ii, j) * TILE_SZ);
#pragma unroll
            for (int p = 0; p < NS; ++p) la.p[p] = *reinterpret_cast<const s16x4 *>(lt + p * 256 + lane * 4);
          } else {
            float av[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) av[e] = Lt[tidx(ii, j) * TILE_SZ + l16 * TILE_LD + 4 * g + e];
            la = split4<NS>(av);
          }
          W = mfma16_pre<NS>(la, Xs[j], W);
        }
        float av[4], bw[4] = {W[0], W[1], W[2], W[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = Lt[tidx(ii, ii) * TILE_SZ + l16 * TILE_LD + 4 * g + e];
        const f32x4 Xn = mfma16_split<NS>(av, bw, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) Xc[ii][r] = -Xn[r];
        const float xv[4] = {Xc[ii][0], Xc[ii][1], Xc[ii][2], Xc[ii][3]};
        Xs[ii] = split4<NS>(xv);
      }
      if constexpr (PP) {  // column block q of T^-1: tile (ii, q) holds rows 4g..4g+3, column l16
#pragma unroll
        for (int ii = 0; ii < NB; ++ii)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.pp_ti[(ch * (size_t)C + 16 * ii + 4 * g + r) * C + 16 * q + l16] = ii >= q ? Xc[ii][r] : 0.f;
      }
    }
    __syncthreads();  // every L and X tile has been read before the fragments overwrite them
    // Column block q of T^-1 leaves as A-fragments of T^-T, pre-split into NS
    // bf16 planes: for pair (st = q, kt), lane (s = l16, g) holds tokens
    // t = 16 (2 kt + e/4) + 4g + e%4 -- exactly rows 4g..4g+3 of the tiles
    // X[2kt][q], X[2kt+1][q] that this lane holds.  The tile above the
    // diagonal (2kt = q - 1 for odd q) is written as zeros.
    if (rowwave) {
#pragma unroll
      for (int ii = 0; ii < NB; ++ii) {
        if (ii < q - q % 2) continue;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = ii >= q ? Xc[ii][r] : 0.f;
        store4_planes<NS>(tf + (tf_pair<NKC>(q, ii / 2) * NS) * FRAG + lane * 8 + 4 * (ii % 2), FRAG, x);
      }
    }
    __syncthreads();
  }

  // -------------------------------------------------- D: the chunk map
  // PP: dO of the chunk, loaded here (in flight while W and P are formed)
  // and staged in LDS before the column loop; rows past the chunk's tokens
  // read its last real row and are zeroed
  constexpr int NDO = PP ? C * D / 4 / (64 * Lds::WAVES) : 1;
  static_assert(!PP || NDO * 4 * 64 * Lds::WAVES == C * D, "whole float4s of dO per thread");
  using DoRaw = std::conditional_t<DOBF, uint2, float4>;
  DoRaw dor[NDO];
  if constexpr (PP) {
#pragma unroll
    for (int it = 0; it < NDO; ++it) {
      const int idx = tid + 64 * Lds::WAVES * it, tt = idx / (D / 4), j4 = idx % (D / 4);
      const size_t off = rowc(tt) * D + 4 * j4;
      if constexpr (DOBF)
        dor[it] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.pp_do) + off);
      else
        dor[it] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.pp_do) + off);
    }
  }
  // With W = K'^T T^-1 (D x C) and P = A T^-1 (C x C, lower triangular):
  //   N = W V_hat,  M = Diag(e^Lambda_C) - W K_hat e^Lambda,
  //   O_bar = P V_hat,  Q' = Qt e^Lambda - P K_hat e^Lambda,
  // so the column loop multiplies the staged R = [V_hat | K_hat e^Lambda]
  // directly, with no Z = T^-1 R round trip.  W and P are formed once per
  // chunk from the T^-1 tiles in LDS.
  // K'^T fragments for channel tile m = wave (lane <-> c), tile-pair order
  // over s: K'[s][c] = kn_s,c Cf_s,c exp(cum_NB - cum_{blk(s)+1}).
  bf16x8 kpf[NKC][NS];
  float gdiag = 0.f;
  if (wave < NMT) {
    const int c = 16 * wave + l16;
    const int ksc = c / 32, cw = c % 32;
    const int ec = 4 * (cw / 16) + (cw % 4), gc = (cw % 16) / 4;
    const float cend = cum[NB * D + c];
    gdiag = __expf(cend);
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int blk = 2 * ks + e / 4, ts = 4 * g + (e % 4);
        float kc;
        if constexpr (SA) {
          kc = 0.f;
#pragma unroll
          for (int p = NS - 1; p >= 0; --p)
            kc += __builtin_bit_cast(float, (uint32_t)kcs[(((blk * NKD + ksc) * NS + p) * 64 + ts + 16 * gc) * 8 + ec] << 16);
        } else {
          kc = kcf[((blk * NKD + ksc) * 64 + ts + 16 * gc) * 8 + ec];
        }
        x[e] = kc * __expf(fminf(cend - cum[(blk + 1) * D + c], 0.f));
      }
      split8<NS>(x, kpf[ks]);
    }
  }

  // W^T (rows s, cols c of this channel tile) = T^-T K' and P^T (rows s, cols
  // t of block i) = T^-T A^T, one s-tile at a time; the accumulators of
  // s-tiles 2ks, 2ks+1 form the A-fragment of W (lane <-> c) and of P
  // (lane <-> t) for k-step ks in tile-pair order over s.  P^T is zero for
  // s-tiles beyond block i, and A^T for token k-steps beyond it.
  bf16x8 wf[NKC][NS], pf[NKC][NS];
  {
    f32x4 accW[2], accP[2];
#pragma unroll
    for (int st = 0; st < NB; ++st) {
      accW[st % 2] = zero4();
      accP[st % 2] = zero4();
#pragma unroll
      for (int kt = st / 2; kt < NKC; ++kt) {
        bf16x8 ta[NS];
        load_frag<NS>(tf + (tf_pair<NKC>(st, kt) * NS) * FRAG + lane * 8, FRAG, ta);
        if (wave < NMT) accW[st % 2] = mfma32_split<NS>(ta, kpf[kt], accW[st % 2]);
        if (rowwave && st <= i && 2 * kt <= i) accP[st % 2] = mfma32_split<NS>(ta, afr[kt], accP[st % 2]);
      }
      if (st % 2 == 1) {
        const int ks = st / 2;
        float x[8] = {accW[0][0], accW[0][1], accW[0][2], accW[0][3],
                      accW[1][0], accW[1][1], accW[1][2], accW[1][3]};
        split8<NS>(x, wf[ks]);
        float y[8] = {accP[0][0], accP[0][1], accP[0][2], accP[0][3],
                      accP[1][0], accP[1][1], accP[1][2], accP[1][3]};
        split8<NS>(y, pf[ks]);
      }
    }
  }

  // every wave has read kcf: the region now takes v_hat = w * v (fp32, kcf
  // layout), read back by the same wave in the first half of the loop below
  __syncthreads();
  if constexpr (PP) {  // dO -> [C][D + 4] fp32 (read after the first half's barriers)
    float *dos = sm + Lds::DOS;
#pragma unroll
    for (int it = 0; it < NDO; ++it) {
      const int idx = tid + 64 * Lds::WAVES * it, tt = idx / (D / 4), j4 = idx % (D / 4);
      float4 v;
      if constexpr (DOBF)
        v = make_float4(__uint_as_float(dor[it].x << 16), __uint_as_float(dor[it].x & 0xffff0000u),
                        __uint_as_float(dor[it].y << 16), __uint_as_float(dor[it].y & 0xffff0000u));
      else
        v = dor[it];
      if (tt >= tvalid) v = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4 *>(dos + tt * Lds::DOS_LD + 4 * j4) = v;
    }
  }
  float *vhat = sm + Lds::KCF;
  if (rowwave) {
    const float wconst = gate_const(a.w_mode);
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      float x[8];
      gate8<BF>(wraw[ks], a.w_mode, wconst, true, x);
#pragma unroll
      for (int e = 0; e < 8; ++e)  // padding tokens write nothing
        x[e] = tok_ok ? raw_elem<BF>(vraw[ks][e / 4], e % 4) * x[e] : 0.f;
      float4 *dst = reinterpret_cast<float4 *>(vhat + ((i * NKD + ks) * 64 + lane) * 8);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
      if constexpr (PP) pp_store(a.pp_vh, ks, x);
    }
  }

  const size_t chq = ch * NS;
  uint16_t *Qp = a.Qp + chq * (size_t)C * D;
  uint16_t *Mm = a.Mm + chq * (size_t)D * D;
  float *Ob = a.Ob + ch * (size_t)C * D;
  float *Nn = a.Nn + ch * (size_t)D * D;

  // one column pair; QRs, KRs = QRp[kq], KRp[kq] (the K half is unrolled, so
  // they are indexed at compile time)
  auto pair_iter = [&](const int cp, const bf16x8 (&QRs)[NS], const bf16x8 (&KRs)[NS]) {
    const bool vhalf = cp < D / 32;
    const int kq = vhalf ? 0 : cp - D / 32;  // channel k-step of the K_hat / Q' half
    // e^{cum_i} of this lane's channels in the K_hat / Q' half (both D1 and
    // the Q' products use it)
    float eci[8];
    if (rowwave && !vhalf) {
      cum8(i, kq, eci);
#pragma unroll
      for (int e = 0; e < 8; ++e) eci[e] = __expf(eci[e]);
    }
    // D1: the owner wave of each token block writes its 16 rows of
    // R[:, 32cp .. 32cp+32) into the B-fragment staging (lane <-> column,
    // tile-pair order over tokens).
    if (rowwave) {
      float val[8];
      if (vhalf) {
        const float4 *src = reinterpret_cast<const float4 *>(vhat + ((i * NKD + cp) * 64 + lane) * 8);
        const float4 f0 = src[0], f1 = src[1];
        val[0] = f0.x; val[1] = f0.y; val[2] = f0.z; val[3] = f0.w;
        val[4] = f1.x; val[5] = f1.y; val[6] = f1.z; val[7] = f1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float kr = 0.f;
#pragma unroll
          for (int p = 0; p < NS; ++p) kr += (float)KRs[p][e];
          val[e] = kr * eci[e];  // k_hat e^Lambda = (k_hat R) e^{cum_i}
        }
      }
      // Value e sits in column 16*(e/4) + 4g + e%4 and token t = 16i + l16.
      // The B-fragment wants, per column, the 4 tokens of a lane quad as 4
      // consecutive bf16: transpose 4 x 4 inside each quad (DPP), then every
      // lane writes 8 contiguous bytes per plane (no bank conflicts).
      const int r = l16 & 3, q4 = l16 >> 2;
      const bool b0 = (r & 1) != 0, b1 = (r & 2) != 0;
      const int ksr = i / 2;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // 4 x 4 transpose over (lane r of the quad, element k): swap the
        // off-diagonal 2 x 2 blocks across lanes r ^ 2, then the off-diagonal
        // elements of each 2 x 2 block across lanes r ^ 1 (selects on lane
        // bits, no lane-dependent indexing).
        const float *w = &val[4 * hf];
        const float s0 = b1 ? w[0] : w[2], s1 = b1 ? w[1] : w[3];
        const float t0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0), 0x4E, 0xF, 0xF, false));
        const float t1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1), 0x4E, 0xF, 0xF, false));
        const float n0 = b1 ? t0 : w[0], n1 = b1 ? t1 : w[1];
        const float n2 = b1 ? w[2] : t0, n3 = b1 ? w[3] : t1;
        const float u0 = b0 ? n0 : n1, u1 = b0 ? n2 : n3;
        const float v0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(u0), 0xB1, 0xF, 0xF, false));
        const float v1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(u1), 0xB1, 0xF, 0xF, false));
        // column 16hf + 4g + r, tokens 4q + 0..3
        const float tok[4] = {b0 ? v0 : n0, b0 ? n1 : v0, b0 ? v1 : n2, b0 ? n3 : v1};
        const int ln = 4 * g + r + 16 * q4;
        store4_planes<NS>(rst + ((ksr * 2 + hf) * NS) * FRAG + ln * 8 + 4 * (i % 2), FRAG, tok);
      }
    }
    __syncthreads();
    // D3: products with R (the chunk map).  Every wave multiplies the same
    // staged fragments of R into its tile of N or M (channel tile `wave`)
    // and of O_bar or Q' (token block i): each fragment is read from LDS once
    // for both.
    const bool mw = wave < NMT;
    f32x4 accC[2] = {zero4(), zero4()}, accT[2] = {zero4(), zero4()};  // channel-tile, token-block products
    f32x4 accMt[PP ? 2 : 1] = {};  // PP, K half: K'^T Y itself (M^T up to the diagonal)
    // both column tiles of a k-step together: their fragments read at once
    // (one k-step ahead) and their two accumulators' products interleaved
    // (each accumulator still sums the k-steps in order)
    bf16x8 n0[NS], n1[NS];
    load_frag<NS>(rst + 0 * NS * FRAG + lane * 8, FRAG, n0);
    load_frag<NS>(rst + 1 * NS * FRAG + lane * 8, FRAG, n1);
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      bf16x8 z0[NS], z1[NS];
#pragma unroll
      for (int p = 0; p < NS; ++p) { z0[p] = n0[p]; z1[p] = n1[p]; }
      if (ks + 1 < NKC) {
        load_frag<NS>(rst + ((ks * 2 + 2) * NS) * FRAG + lane * 8, FRAG, n0);
        load_frag<NS>(rst + ((ks * 2 + 3) * NS) * FRAG + lane * 8, FRAG, n1);
      }
      const bool tw = rowwave && 2 * ks <= i && (!vhalf || a.Ob);  // O_bar only when it is stored
      if (!mw && !tw) continue;
      if (vhalf) {
        if (mw) mfma32_split2<NS>(wf[ks], z0, accC[0], wf[ks], z1, accC[1]);  // N = K'^T U_bar
        if (tw) mfma32_split2<NS>(z0, pf[ks], accT[0], z1, pf[ks], accT[1]);  // O_bar^T = U_bar^T A^T
      } else {
        if (mw) mfma32_split2<NS>(z0, wf[ks], accC[0], z1, wf[ks], accC[1]);  // (K'^T Y)^T = Y^T K'
        if (tw) mfma32_split2<NS>(z0, pf[ks], accT[0], z1, pf[ks], accT[1]);  // (A Y)^T = Y^T A^T
        if constexpr (PP)
          if (mw) mfma32_split2<NS>(wf[ks], z0, accMt[0], wf[ks], z1, accMt[1]);
      }
    }
    if (vhalf) {
      if (mw) {
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl)
          *reinterpret_cast<f32x4 *>(Nn + ((size_t)(wave * NMT + 2 * cp + ctl) * 64 + lane) * 4) = accC[ctl];
      }
      if (rowwave && a.Ob) {
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl)
          *reinterpret_cast<f32x4 *>(Ob + ((size_t)(i * NMT + 2 * cp + ctl) * 64 + lane) * 4) = accT[ctl];
      }
    } else {
      const int ksy = cp - D / 32;  // k-step of the state-row index covered by this pair
      if (mw) {                     // M = Diag(e^Lambda_C) - K'^T Y
        const int c = 16 * wave + l16;
        float mv[8];
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cpr = 32 * ksy + 16 * ctl + 4 * g + r;
            mv[4 * ctl + r] = (cpr == c ? gdiag : 0.f) - accC[ctl][r];
          }
        store8_planes<NS>(Mm + ((size_t)(wave * NKD + ksy) * 64 + lane) * 8, (size_t)D * D, mv);
        if constexpr (PP) {
          // M^T[j][c] for j = 32 ksy + 16 ctl + l16 (its A-fragment row) and
          // c = 16 wave + 4 g + r: half of the fragment entry of row tile
          // 2 ksy + ctl and k-step wave / 2 (the diagonal, j = c, falls on the
          // lanes whose own channel 16 wave + l16 is j)
#pragma unroll
          for (int ctl = 0; ctl < 2; ++ctl) {
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x[r] = (2 * ksy + ctl == wave && l16 == 4 * g + r ? gdiag : 0.f) - accMt[ctl][r];
            store4_planes<NS>(a.pp_mt + chq * (size_t)D * D +
                                  ((size_t)((2 * ksy + ctl) * NKD + wave / 2) * 64 + lane) * 8 + 4 * (wave % 2),
                              (size_t)D * D, x);
          }
        }
      }
      if (rowwave) {  // Q' = Qt e^Lambda - A Y
        float qv8[8];
#pragma unroll
        for (int ctl = 0; ctl < 2; ++ctl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * ctl + r;  // channel tp_chan(ksy, g, e)
            float qr = 0.f;
#pragma unroll
            for (int p = 0; p < NS; ++p) qr += (float)QRs[p][e];
            qv8[e] = qr * eci[e] - accT[ctl][r];
          }
        if constexpr (PP) {  // this pair's 32 channels of Q' for G (row t, channel 16 ctl + 4 g + r)
          float *qs = sm + Lds::QS + t * Lds::QS_LD + 4 * g;
          *reinterpret_cast<float4 *>(qs) = make_float4(qv8[0], qv8[1], qv8[2], qv8[3]);
          *reinterpret_cast<float4 *>(qs + 16) = make_float4(qv8[4], qv8[5], qv8[6], qv8[7]);
        } else {
          store8_planes<NS>(Qp + ((size_t)(i * NKD + ksy) * 64 + lane) * 8, (size_t)C * D, qv8);
        }
      }
    }
    __syncthreads();
    if constexpr (PP) {
      // G rows of this pair's 32 channels (state-row tiles 2 ksy, 2 ksy + 1)
      // = Q'[:, channels]^T dO on the fp32 matrix cores, k = token; wave w
      // takes row tile 2 ksy + (w & 1) and value tiles 2 (w >> 1), + 1.  The
      // next pair writes Q' only after its own first barrier.
      if (!vhalf) {
        static_assert(NMT == Lds::WAVES, "two G tiles per wave");
        const float *qs = sm + Lds::QS, *dos = sm + Lds::DOS;
        const int rl = wave & 1, jt0 = 2 * (wave >> 1);
        f32x4 g0 = zero4(), g1 = zero4();
#pragma unroll
        for (int kb = 0; kb < C / 4; ++kb) {
          const int tt = 4 * kb + g;
          const float av = qs[tt * Lds::QS_LD + 16 * rl + l16];
          const float b0 = dos[tt * Lds::DOS_LD + 16 * jt0 + l16];
          const float b1 = dos[tt * Lds::DOS_LD + 16 * (jt0 + 1) + l16];
          g0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b0, g0, 0, 0, 0);
          g1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1, g1, 0, 0, 0);
        }
        const int rt = 2 * (cp - D / 32) + rl;
        float *G = a.pp_g + ch * (size_t)D * D;
        *reinterpret_cast<f32x4 *>(G + ((size_t)(rt * NMT + jt0) * 64 + lane) * 4) = g0;
        *reinterpret_cast<f32x4 *>(G + ((size_t)(rt * NMT + jt0 + 1) * 64 + lane) * 4) = g1;
      }
    }
  };
  if constexpr (NS == 2) {
#pragma unroll 1
    for (int cp = 0; cp < D / 32; ++cp) pair_iter(cp, QRp[0], KRp[0]);
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk) pair_iter(D / 32 + kk, QRp[kk], KRp[kk]);
  } else {  // fp32 mode: unrolling the K half would spill; select at run time
#pragma unroll 1
    for (int cp = 0; cp < 2 * D / 32; ++cp) {
      const int kq = cp < D / 32 ? 0 : cp - D / 32;
      bf16x8 QRs[NS], KRs[NS];  // QRp[kq], KRp[kq], selected without dynamic indexing
#pragma unroll
      for (int p = 0; p < NS; ++p) { QRs[p] = QRp[0][p]; KRs[p] = KRp[0][p]; }
#pragma unroll
      for (int kk = 1; kk < NKD; ++kk)
        if (kq == kk) {
#pragma unroll
          for (int p = 0; p < NS; ++p) { QRs[p] = QRp[kk][p]; KRs[p] = KRp[kk][p]; }
        }
      pair_iter(cp, QRs, KRs);
    }
  }
}

// ============================================================================
// Kernel 2 (chain): one workgroup per (stream, 16-column value slice); wave w
// owns state row tile w.  Per chunk: S <- M S + N, with the fp32 slice in the
// accumulator tiles and its NS bf16 planes shared through LDS as
// B-fragments.  Those planes -- the chunk-start state S_c -- are also written
// to the workspace for the output kernel.  M and N of chunks c+1 .. c+3 are
// in flight while chunk c is computed (four register buffers; three, holding
// c+1 and c+2, in fp32 mode); every wave
// issues its loads without a branch, so that the wait counts stay exact.
// ============================================================================
template <int D, int NS>
struct ChainBuf {
  bf16x8 m[D / 32][NS];  // A-fragments of M (state row tile)
  f32x4 nn;              // accumulator tile of N
};

// S_c planes, double-buffered by chunk parity: step c reads buffer c & 1 and
// writes buffer (c + 1) & 1, so one barrier per step suffices
template <int D, int NS>
using ChainLds = uint16_t[2][(D / 32) * NS * 64 * 8];

// The chain of workgroup `id` of a launch over the chain `a`.
template <int C, int D, int NS>
__device__ __forceinline__ void chain_run(const ChunkArgs &a, int id, ChainLds<D, NS> &sfr2) {
  constexpr int NMT = D / 16, NKD = D / 32, NSL = D / 16;
  constexpr int FRAG = 64 * 8, NFR = NKD * NS;

  // all slices of one stream on the same XCD (workgroups go round-robin over 8)
  const int grp = id / (8 * NSL), rem = id % (8 * NSL);
  const int slice = rem / 8;
  const size_t bh = (size_t)grp * 8 + rem % 8;
  if (bh >= (size_t)a.B * a.H) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // chunks of this stream and their workspace slots
  int NC;
  size_t slot0, slot_step;
  if (a.ctab) {  // packed batch: stream = sequence * H + head, slot = entry * H + head
    const int n = (int)(bh / a.H);
    NC = a.coff[n + 1] - a.coff[n];  // the sequence's entries of the chunk list
    slot0 = (size_t)a.coff[n] * a.H + bh % a.H;
    slot_step = a.H;
  } else {
    NC = a.ncs;  // chunks c0 .. c0 + ncs - 1 (the last chunk of a stream may be short)
    slot0 = bh * NC;
    slot_step = 1;
  }
  auto slot = [&](int c) { return slot0 + (size_t)(a.rev ? NC - 1 - c : c) * slot_step; };
  const int col = 16 * slice + l16;

  f32x4 S = zero4();
  if (a.S0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) S[r] = a.S0[(bh * D + 16 * wave + 4 * g + r) * D + col];
  }
  auto publish = [&](uint16_t *sfr) {
    float x[4] = {S[0], S[1], S[2], S[3]};
    store4_planes<NS>(sfr + ((wave / 2) * NS) * FRAG + lane * 8 + 4 * (wave % 2), FRAG, x);
  };
  const uint32_t off_m = (uint32_t)((wave * NKD * 64 + lane) * 8);
  const uint32_t off_nn = (uint32_t)(((wave * NMT + slice) * 64 + lane) * 4);
  // buffer loads: the chunk base goes in scalar registers and the lane
  // offsets never change, so no address register is rewritten while a load
  // into another buffer is still in flight (that would cost a wait)
  auto load = [&](int c, ChainBuf<D, NS> &bf) {
    c = c < NC ? c : NC - 1;  // clamped instead of skipped: no conditional load
    const size_t ch = slot(c);
    const auto rm = buffer_rsrc(a.Mm + ch * NS * (size_t)D * D, (uint32_t)(NS * D * D * 2));
    const auto rn = buffer_rsrc(a.Nn + ch * (size_t)D * D, (uint32_t)(D * D * 4));
    bf.nn = buffer_load16<f32x4>(rn, 4 * off_nn);
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
      for (int p = 0; p < NS; ++p) bf.m[ks][p] = buffer_load16<bf16x8>(rm, 2 * (p * D * D + off_m + ks * 512));
  };
  // step c with the state planes in LDS buffer `par`
  auto step = [&](int c, const ChainBuf<D, NS> &cur, int par) {
    const uint16_t *sfr = sfr2[par];
    // chunk-start state planes -> workspace (fragment f = ks * NS + p)
    uint16_t *Sc = a.Sc + slot(c) * (size_t)NS * D * D + (size_t)slice * NFR * FRAG;
    if constexpr (NFR == NMT) {  // one fragment per wave, no branch (keeps the wait counts exact)
      *reinterpret_cast<bf16x8 *>(Sc + wave * FRAG + lane * 8) =
          *reinterpret_cast<const bf16x8 *>(sfr + wave * FRAG + lane * 8);
    } else {
      for (int f = wave; f < NFR; f += NMT)
        *reinterpret_cast<bf16x8 *>(Sc + f * FRAG + lane * 8) =
            *reinterpret_cast<const bf16x8 *>(sfr + f * FRAG + lane * 8);
    }
    bf16x8 sf[NKD][NS];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) load_frag<NS>(sfr + (ks * NS) * FRAG + lane * 8, FRAG, sf[ks]);
    __builtin_amdgcn_sched_barrier(0);  // all fragment reads in flight before the products
    // independent accumulation chains over the k-steps (one per k-step; two
    // in fp32 mode, where registers are short)
    constexpr int NACC = NS == 3 ? 2 : NKD;
    f32x4 acc[NACC];
#pragma unroll
    for (int ks = 0; ks < NACC; ++ks) acc[ks] = ks == 0 ? cur.nn : zero4();
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) acc[ks % NACC] = mfma32_split<NS>(cur.m[ks], sf[ks], acc[ks % NACC]);
#pragma unroll
    for (int ks = 1; ks < NACC; ++ks)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[0][r] += acc[ks][r];
    S = acc[0];
    publish(sfr2[par ^ 1]);
    __syncthreads();
  };

  publish(sfr2[0]);
  __syncthreads();
  if (NC <= 0) {
    // no chunk: S_T = S0 below
  } else if constexpr (NS == 3) {  // fp32 mode: wider buffers, three of them
    ChainBuf<D, NS> b0, b1, b2;
    load(0, b0);
    load(1, b1);
    for (int c = 0; c < NC; c += 3) {
      load(c + 2, b2);
      step(c, b0, c & 1);
      if (c + 1 >= NC) break;
      load(c + 3, b0);
      step(c + 1, b1, (c + 1) & 1);
      if (c + 2 >= NC) break;
      load(c + 4, b1);
      step(c + 2, b2, c & 1);
    }
  } else {
    ChainBuf<D, NS> b0, b1, b2, b3;
    load(0, b0);
    load(1, b1);
    load(2, b2);
    for (int c = 0; c < NC; c += 4) {
      load(c + 3, b3);
      step(c, b0, 0);
      if (c + 1 >= NC) break;
      load(c + 4, b0);
      step(c + 1, b1, 1);
      if (c + 2 >= NC) break;
      load(c + 5, b1);
      step(c + 2, b2, 0);
      if (c + 3 >= NC) break;
      load(c + 6, b2);
      step(c + 3, b3, 1);
    }
  }
  if (a.S_T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a.S_T[(bh * D + 16 * wave + 4 * g + r) * D + col] = S[r];
  }
}

template <int C, int D, int NS>
__global__ void __launch_bounds__(64 * (D / 16)) chunk_chain_kernel(ChunkArgs a) {
  __shared__ __align__(16) ChainLds<D, NS> sfr2;
  chain_run<C, D, NS>(a, blockIdx.x, sfr2);
}

// Two independent chains in one launch: workgroups [0, na) run `a`, the rest
// `b` (na a multiple of 8, so both keep their XCD placement).
template <int C, int D, int NS>
__global__ void __launch_bounds__(64 * (D / 16)) chunk_chain2_kernel(ChunkArgs a, ChunkArgs b, int na) {
  __shared__ __align__(16) ChainLds<D, NS> sfr2;
  const bool first = (int)blockIdx.x < na;
  chain_run<C, D, NS>(first ? a : b, first ? (int)blockIdx.x : (int)blockIdx.x - na, sfr2);
}

// ============================================================================
// Kernel 3 (output): one workgroup per (stream, chunk); wave w owns output row
// tile w and sweeps the value slices: O = Q' S_c + O_bar, formed transposed
// (O^T = S_c^T Q'^T: the S_c fragments in the A operand, Q''s in the B
// operand, O_bar stored transposed by the intra-chunk kernel) so that a lane
// holds 4 consecutive value channels of one token and stores them as one
// vector.  S_c (all slices, NS bf16 planes in B-fragment layout, which is the
// A-fragment layout of S_c^T) is staged in LDS once.
// ============================================================================
// Dynamic LDS of the output kernel: the S_c planes of all slices, and with a
// gated output also the normalised rows [C][D + 4] fp32 (staged after the
// planes are read).
template <int C, int D, int NS>
constexpr size_t out_lds_gated() {
  constexpr size_t planes = (size_t)(D / 16) * (D / 32) * NS * 512 * 2, rows = (size_t)C * (D + 4) * 4;
  return planes > rows ? planes : rows;
}

// OG: gated output -- per token, the RMS over the dv channels of o is reduced
// across the 4 lanes that hold the token's columns, and y = o / rms * onw *
// sigmoid(og) is written token-major; o itself is not written.
template <int C, int D, int NS, bool OB16, bool OG>
__global__ void __launch_bounds__(64 * (C / 16)) chunk_out_kernel(ChunkArgs a) {
  constexpr int NRT = C / 16, NMT = D / 16, NKD = D / 32, NSL = D / 16;
  constexpr int FRAG = 64 * 8, NFR = NKD * NS;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *sc = reinterpret_cast<uint16_t *>(smem);  // [NSL][NFR][FRAG]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t ch = blockIdx.x;  // chunk slot (layout as in the intra-chunk kernel)
  size_t rbase;                   // first token row of the chunk
  int tvalid;
  if (a.ctab) {
    const int4 e = a.ctab[ch / a.H];
    if (e.x < 0) return;
    rbase = (ch % a.H) * (size_t)a.T + e.z;
    tvalid = e.w;
  } else {
    const int c = a.c0 + (int)(ch % a.ncs);  // the last chunk of a stream may be short
    rbase = (ch / a.ncs) * (size_t)a.T + (size_t)c * C;
    tvalid = min(C, a.T - c * C);
  }

  const uint16_t *Scg = a.Sc + ch * (size_t)NS * D * D;
  // all of a thread's 16-byte vectors loaded before any is stored, so their
  // loads are in flight together
  constexpr int NV = NSL * NFR * FRAG / 8, NVT = NV / (64 * NRT);
  static_assert(NVT * 64 * NRT == NV, "whole vectors per thread");
  u32x4 scv[NVT];  // a vector type: an array of structs would stay in scratch
#pragma unroll
  for (int v = 0; v < NVT; ++v) scv[v] = *reinterpret_cast<const u32x4 *>(Scg + (tid + v * 64 * NRT) * 8);
#pragma unroll
  for (int v = 0; v < NVT; ++v) *reinterpret_cast<u32x4 *>(sc + (tid + v * 64 * NRT) * 8) = scv[v];
  const uint16_t *Qp = a.Qp + ch * NS * (size_t)C * D;
  bf16x8 qf[NKD][NS];
#pragma unroll
  for (int ks = 0; ks < NKD; ++ks)
#pragma unroll
    for (int p = 0; p < NS; ++p)
      qf[ks][p] = *reinterpret_cast<const bf16x8 *>(Qp + (size_t)p * C * D + ((wave * NKD + ks) * 64 + lane) * 8);
  const float *Ob = a.Ob + ch * (size_t)C * D;
  // gated output: all of the wave's O_bar tiles loaded with the other loads
  // (its products come before any store, so they are waited for once)
  f32x4 obg[OG ? NSL : 1];
  if constexpr (OG) {
#pragma unroll
    for (int jt = 0; jt < NSL; ++jt) obg[jt] = *reinterpret_cast<const f32x4 *>(Ob + ((size_t)(wave * NMT + jt) * 64 + lane) * 4);
  }
  __syncthreads();
  const int tok = 16 * wave + l16;  // this lane's token within the chunk
  const bool live = tok < tvalid;   // padding rows are never stored
  const size_t orow = rbase + tok;
  // lane (l16, g): token tok, value channels 16 jt + 4 g .. + 3
  auto product = [&](int jt) {
    f32x4 acc = *reinterpret_cast<const f32x4 *>(Ob + ((size_t)(wave * NMT + jt) * 64 + lane) * 4);
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      bf16x8 sf[NS];
      load_frag<NS>(sc + (jt * NFR + ks * NS) * FRAG + lane * 8, FRAG, sf);
      acc = mfma32_split<NS>(sf, qf[ks], acc);
    }
    return acc;
  };
  if constexpr (!OG) {
#pragma unroll 1
    for (int jt = 0; jt < NSL; ++jt) {
      const f32x4 acc = product(jt);
      if (live) st4_stream<OB16>(a.o, orow * D + 16 * jt + 4 * g, acc);
    }
  } else {
    // this lane's 4 value channels of every slice
    f32x4 ov[NSL];
#pragma unroll
    for (int jt = 0; jt < NSL; ++jt) ov[jt] = obg[jt];
#pragma unroll
    for (int jt = 0; jt < NSL; ++jt)
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        bf16x8 sf[NS];
        load_frag<NS>(sc + (jt * NFR + ks * NS) * FRAG + lane * 8, FRAG, sf);
        ov[jt] = mfma32_split<NS>(sf, qf[ks], ov[jt]);
      }
    float ss = 0.f;
#pragma unroll
    for (int jt = 0; jt < NSL; ++jt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ss += ov[jt][r] * ov[jt][r];
      if (a.oraw && live)  // o before the norm and the gate, for the gate's backward
        *reinterpret_cast<f32x4 *>(a.oraw + orow * D + 16 * jt + 4 * g) = ov[jt];
    }
    ss += __shfl_xor(ss, 16, kWave);  // the 4 lanes of the token
    ss += __shfl_xor(ss, 32, kWave);
    const float inv = rsqrtf(ss / (float)D + a.oeps);
    // normalised rows through LDS (the S_c planes are no longer read), then
    // each thread takes 8 consecutive columns of one token: the gate loads
    // and the token-major stores are whole 16- or 32-byte vectors
    __syncthreads();
    float *ys = reinterpret_cast<float *>(smem);  // [C][D + 4] fp32
    constexpr int YLD = D + 4;
#pragma unroll
    for (int jt = 0; jt < NSL; ++jt) *reinterpret_cast<f32x4 *>(ys + tok * YLD + 16 * jt + 4 * g) = ov[jt] * inv;
    __syncthreads();
    const size_t T = (size_t)a.T;
    constexpr int PT = D / 8;  // threads per token
    for (int idx = tid; idx < C * PT; idx += 64 * NRT) {
      const int tk = idx / PT, c8 = (idx % PT) * 8;
      if (tk >= tvalid) continue;  // no padding rows
      const size_t row = rbase + tk;  // row of [B,H,T] (head-major)
      const size_t bh = row / T, t = row % T;
      const size_t hh = bh % (size_t)a.H, b = bh / (size_t)a.H;
      const size_t yrow = (b * T + t) * (size_t)a.H + hh;  // row of [B,T,H]
      float gl[8], nw[8], yv[8];
      ld8<NS == 2>(a.og, row * D + c8, gl);
      if (a.onw) {
        ld8<false>(a.onw, hh * D + c8, nw);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) nw[e] = 1.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] = ys[tk * YLD + c8 + e] * nw[e] * (1.f / (1.f + __expf(-gl[e])));
      st8<OB16>(a.y, yrow * D + c8, yv);
    }
  }
}

// ============================================================================
// Packed batches: the per-head chunk list.  One workgroup scans the chunk
// counts ceil(len_n / C) of the sequences (1024 at a time), writes the
// offsets coff[0..nseq] and, per sequence, its entries {n, c, first packed
// row, valid tokens}; entries past the last chunk get sequence -1.
// The offsets are read defensively: each is clamped to [0, T] and the end of
// a sequence to no less than its start, and no entry is written at or past
// ctab_len (coff is capped there too), so offsets that break the documented
// contract give wrong results but never an access outside the tensors or
// the workspace.  Sequence n owns the coff[n + 1] - coff[n] entries from
// coff[n] on: ceil(len_n / C) whenever the offsets are valid.
// ============================================================================
template <int C>
__global__ void __launch_bounds__(1024) chunk_table_kernel(ChunkArgs a) {
  __shared__ long long wsum[16];
  __shared__ long long carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long cap = a.ctab_len;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base <= a.nseq; base += 1024) {
    const int n = base + tid;
    int len = 0, r0 = 0;
    long long cnt = 0;
    if (n < a.nseq) {
      r0 = min(max(a.cu[n], 0), a.T);
      const int r1 = min(max(a.cu[n + 1], r0), a.T);
      len = r1 - r0;
      cnt = (len + C - 1) / C;
    }
    long long x = cnt;  // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (tid == 0) {  // wave totals -> exclusive offsets of the waves
      long long acc = 0;
      for (int w = 0; w < 16; ++w) { const long long t = wsum[w]; wsum[w] = acc; acc += t; }
    }
    __syncthreads();
    const long long excl = carry + wsum[wave] + x - cnt;  // chunks before sequence n
    if (n <= a.nseq) a.coff[n] = (int)min(excl, cap);
    if (n < a.nseq) {
      const long long stop = min(excl + cnt, cap);
      for (long long j = excl; j < stop; ++j) {
        const int c = (int)(j - excl);
        a.ctab[j] = make_int4(n, c, r0 + c * C, min(C, len - c * C));
      }
    }
    __syncthreads();
    if (tid == 1023) carry = excl + cnt;  // running total after this block of sequences
    __syncthreads();
  }
  for (long long j = min(carry, cap) + tid; j < cap; j += 1024) a.ctab[j] = make_int4(-1, 0, 0, 0);
}

// ============================================================================
// host side
// ============================================================================
size_t chunk_workspace(ChunkArgs *a, void *ws, int B, int H, int T, int C, int D, int NS, int nseq) {
  const size_t per_head = (size_t)((T + C - 1) / C) + (nseq > 0 ? (size_t)nseq : 0);
  const size_t nch = nseq > 0 ? (size_t)H * per_head : (size_t)B * H * ((T + C - 1) / C);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t sz[8] = {nch * NS * (size_t)C * D * 2, nch * NS * (size_t)D * D * 2, nch * (size_t)C * D * 4,
                        nch * (size_t)D * D * 4, nch * NS * (size_t)D * D * 2,
                        nseq > 0 ? per_head * sizeof(int4) : 0, nseq > 0 ? ((size_t)nseq + 1) * sizeof(int) : 0,
                        nseq > 0 || T == 0 ? 0 : (size_t)B * H * D * D * sizeof(float)};
  size_t off[8], total = 0;
  for (int r = 0; r < 8; ++r) { off[r] = total; total += al(sz[r]); }
  if (ws && a) {
    unsigned char *base = static_cast<unsigned char *>(ws);
    a->Qp = reinterpret_cast<uint16_t *>(base + off[0]);
    a->Mm = reinterpret_cast<uint16_t *>(base + off[1]);
    a->Ob = reinterpret_cast<float *>(base + off[2]);
    a->Nn = reinterpret_cast<float *>(base + off[3]);
    a->Sc = reinterpret_cast<uint16_t *>(base + off[4]);
    a->ctab = nseq > 0 ? reinterpret_cast<int4 *>(base + off[5]) : nullptr;
    a->coff = nseq > 0 ? reinterpret_cast<int *>(base + off[6]) : nullptr;
    a->ctab_len = nseq > 0 ? (int)per_head : 0;
    a->Sst = nseq > 0 ? nullptr : reinterpret_cast<float *>(base + off[7]);
  }
  return total;
}

// Configurations with an instantiated kernel whose workgroup fits in LDS.
// C = 128, d = 128 with fp32 inputs (three planes) is not instantiated; the
// C = 64 kernel serves that input type at d = 128.
bool chunk_intra_fits(int C, int D, int NS) {
  size_t b = 0;
#define GDR_FIT(CC, DD, NN) if (C == CC && D == DD && NS == NN) b = IntraLds<CC, DD, NN>::bytes;
  GDR_FIT(64, 64, 2) GDR_FIT(64, 64, 3) GDR_FIT(64, 128, 2) GDR_FIT(64, 128, 3)
  GDR_FIT(128, 64, 2) GDR_FIT(128, 64, 3) GDR_FIT(128, 128, 2)
#undef GDR_FIT
  return b > 0 && b <= 160 * 1024;
}

// Chunks per stream in one segment of a whole-call launch.  Each kernel of a
// segment reads what the previous one wrote to the workspace (Q', M, O_bar, N,
// S_c: `chunk_bytes` per chunk); a segment of at most kSegmentBytes keeps that
// traffic inside MI355X's 256 MB last-level cache instead of HBM.  The count
// is a multiple of 256 / gcd(streams, 256), so that every intra-chunk launch
// fills whole rounds of the 256 CUs, and at least kMinSegment chunks (launch
// cost); NC (one segment) when the whole workspace is small enough.
constexpr size_t kSegmentBytes = (size_t)160 << 20;
constexpr size_t kMinSegment = 8;
constexpr size_t seg_chunk_bytes(int C, int D, int NS) {
  return (size_t)NS * C * D * 2 + (size_t)NS * D * D * 2 * 2 + (size_t)C * D * 4 + (size_t)D * D * 4;
}
static int segment_chunks(size_t nbh, int NC, size_t chunk_bytes) {
  if (nbh == 0 || NC <= 0 || nbh * (size_t)NC * chunk_bytes <= kSegmentBytes) return NC > 0 ? NC : 1;
  size_t g = 256, x = nbh % 256;
  while (x) { const size_t t = g % x; g = x; x = t; }  // gcd(256, nbh)
  const size_t q = 256 / g;
  size_t seg = kSegmentBytes / (nbh * chunk_bytes);
  seg -= seg % q;
  if (seg < kMinSegment) return NC;  // too short to pay for the extra launches
  return seg >= (size_t)NC ? NC : (int)seg;
}

// One pass of the kernels over `nch` chunk slots (phases: bit 0 intra-chunk,
// bit 1 chain + output).
template <int C, int D, int NS, bool BF, bool OB16>
static hipError_t launch_chunk_pass(const ChunkArgs &a, size_t nch, int phases, hipStream_t st) {
  using Lds = IntraLds<C, D, NS>;
  const size_t nbh = (size_t)a.B * a.H;
  if (nch > 0 && (phases & 1)) {
    const bool sa = NS == 2 && a.alpha_mode != GDR_GATE_PER_CHANNEL;  // scalar decay
    const dim3 grid((unsigned)nch), block(64 * Lds::WAVES);
    bool pp = false;
    if constexpr (C == 64) {
      if (a.pp_kn) {  // the backward's recompute: the per-token vectors and G as well
        pp = true;
        if (a.pp_do_bf16) {
          if (sa)
            hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF, NS == 2, true, true>), grid, block, Lds::pp_bytes, st, a);
          else
            hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF, false, true, true>), grid, block, Lds::pp_bytes, st, a);
        } else {
          if (sa)
            hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF, NS == 2, true>), grid, block, Lds::pp_bytes, st, a);
          else
            hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF, false, true>), grid, block, Lds::pp_bytes, st, a);
        }
      }
    }
    if (!pp) {
      if (sa)
        hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF, NS == 2>), grid, block, Lds::bytes, st, a);
      else
        hipLaunchKernelGGL((chunk_intra_kernel<C, D, NS, BF, false>), grid, block, Lds::bytes, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phases & 6)) return hipSuccess;
  constexpr int NSL = D / 16;
  const size_t nblk = ((nbh + 7) / 8) * 8 * NSL;
  hipLaunchKernelGGL((chunk_chain_kernel<C, D, NS>), dim3((unsigned)nblk), dim3(64 * (D / 16)), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nch == 0 || !(phases & 2)) return e;
  constexpr size_t out_lds = (size_t)NSL * (D / 32) * NS * 512 * 2;
  constexpr size_t og_lds = out_lds_gated<C, D, NS>();
  if (a.og)
    hipLaunchKernelGGL((chunk_out_kernel<C, D, NS, OB16, true>), dim3((unsigned)nch), dim3(64 * (C / 16)), og_lds,
                       st, a);
  else
    hipLaunchKernelGGL((chunk_out_kernel<C, D, NS, OB16, false>), dim3((unsigned)nch), dim3(64 * (C / 16)), out_lds, st, a);
  return hipGetLastError();
}

constexpr int kMaxDevices = 64;

int chunk_segment(int B, int H, int T, int C, int D, int NS) {
  const int NC = (T + C - 1) / C;
  return segment_chunks((size_t)B * H, NC, seg_chunk_bytes(C, D, NS));
}

// Scratch of the allocation-free whole call (gdr_chunk_fwd_static): one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it only names the symbol): the device
// address of the current device's copy is looked up once per device and
// used everywhere instead.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr) {
  static std::once_flag once[kMaxDevices];
  static void *addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void *p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = err[dev] == hipSuccess ? p : nullptr;
  });
  if (err[dev] != hipSuccess) return err[dev];
  if (!addr[dev]) return hipErrorInvalidSymbol;
  *ptr = addr[dev];
  return hipSuccess;
}

template <int C, int D, int NS, bool BF, bool OB16>
static hipError_t launch_chunk_t(const ChunkArgs &a, int phases, hipStream_t st, int seg_force) {
  using Lds = IntraLds<C, D, NS>;
  static_assert(Lds::bytes <= 160 * 1024 || NS == 3, "intra-chunk LDS budget");
  if constexpr (Lds::bytes <= 160 * 1024) {
    // the dynamic-LDS limits, once per device (a function attribute may be
    // held per device)
    static std::once_flag once[kMaxDevices];
    static hipError_t attr_err[kMaxDevices];
    int dev = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 != hipSuccess) return e0;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] {
      constexpr size_t out_lds = (size_t)(D / 16) * (D / 32) * NS * 512 * 2;
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF, false>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lds::bytes);
      if (e == hipSuccess && NS == 2)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF, NS == 2>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lds::bytes);
      if constexpr (C == 64) {
        static_assert(Lds::pp_bytes <= 160 * 1024, "the recompute's LDS budget");
        const void *pk[4] = {reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF, false, true>),
                             reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF, false, true, true>),
                             reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF, NS == 2, true>),
                             reinterpret_cast<const void *>(&chunk_intra_kernel<C, D, NS, BF, NS == 2, true, true>)};
        for (int q = 0; q < (NS == 2 ? 4 : 2) && e == hipSuccess; ++q)
          e = hipFuncSetAttribute(pk[q], hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lds::pp_bytes);
      }
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_out_kernel<C, D, NS, OB16, false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)out_lds);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_out_kernel<C, D, NS, OB16, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(out_lds_gated<C, D, NS>()));
      attr_err[dev] = e;
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    const size_t nbh = (size_t)a.B * a.H;
    if (a.ctab) {  // packed batch: one pass over the device-built chunk list
      if (phases & 1) {
        hipLaunchKernelGGL((chunk_table_kernel<C>), dim3(1), dim3(1024), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      return launch_chunk_pass<C, D, NS, BF, OB16>(a, (size_t)a.H * a.ctab_len, phases, st);
    }
    // Uniform batch: the whole call (phases 3) runs in segments of `seg`
    // chunks per stream, the state carried between segments in Sst; the
    // separate intra / scan calls exchange the whole workspace and are not
    // segmented.
    const int NC = (a.T + C - 1) / C;
    constexpr size_t chunk_bytes = seg_chunk_bytes(C, D, NS);
    const int seg = seg_force > 0 ? seg_force : (phases == 3 ? segment_chunks(nbh, NC, chunk_bytes) : NC);
    const int nseg = NC > 0 ? (NC + seg - 1) / seg : 1;
    for (int sgi = 0; sgi < nseg; ++sgi) {
      ChunkArgs sa = a;
      sa.c0 = sgi * seg;
      sa.ncs = NC > 0 ? std::min(seg, NC - sa.c0) : 0;
      if (sgi > 0) sa.S0 = a.Sst;
      if (sgi + 1 < nseg) sa.S_T = a.Sst;
      hipError_t e = launch_chunk_pass<C, D, NS, BF, OB16>(sa, nbh * (size_t)sa.ncs, phases, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else {
    return hipErrorInvalidValue;
  }
}

template <int C, int D, int NS>
static hipError_t launch_chain_pair_t(const ChunkArgs &a, const ChunkArgs &b, hipStream_t st) {
  constexpr int NSL = D / 16;
  const size_t na = (((size_t)a.B * a.H + 7) / 8) * 8 * NSL, nb = (((size_t)b.B * b.H + 7) / 8) * 8 * NSL;
  hipLaunchKernelGGL((chunk_chain2_kernel<C, D, NS>), dim3((unsigned)(na + nb)), dim3(64 * (D / 16)), 0, st, a, b,
                     (int)na);
  return hipGetLastError();
}

hipError_t launch_chain_pair(const gdr_desc &d, const ChunkArgs &a, const ChunkArgs &b, hipStream_t st) {
  const bool ib = d.in_dtype == GDR_BF16;
  if (d.chunk != 64) return hipErrorInvalidValue;
  if (d.dk == 128) return ib ? launch_chain_pair_t<64, 128, 2>(a, b, st) : launch_chain_pair_t<64, 128, 3>(a, b, st);
  if (d.dk == 64) return ib ? launch_chain_pair_t<64, 64, 2>(a, b, st) : launch_chain_pair_t<64, 64, 3>(a, b, st);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk(const gdr_desc &d, const ChunkArgs &a, int phases, hipStream_t st, int seg) {
  const bool ib = d.in_dtype == GDR_BF16, ob = d.out_dtype == GDR_BF16;
  if (seg > 0 && (phases != 3 || a.ctab)) return hipErrorInvalidValue;
#define GDR_CH(CC, DD, IB, OBB)                                                            \
  if (d.chunk == CC && d.dk == DD && ib == IB && ob == OBB)                                \
    return launch_chunk_t<CC, DD, (IB ? 2 : 3), IB, OBB>(a, phases, st, seg);
  GDR_CH(64, 64, true, false) GDR_CH(64, 64, true, true) GDR_CH(64, 64, false, false)
  GDR_CH(64, 64, false, true) GDR_CH(64, 128, true, false) GDR_CH(64, 128, true, true)
  GDR_CH(64, 128, false, false) GDR_CH(64, 128, false, true) GDR_CH(128, 64, true, false)
  GDR_CH(128, 64, true, true) GDR_CH(128, 64, false, false) GDR_CH(128, 64, false, true)
  GDR_CH(128, 128, true, false) GDR_CH(128, 128, true, true)
#undef GDR_CH
  return hipErrorInvalidValue;
}

}  // namespace gdr
