// gdr_decode.hip -- one decode step of the channel-wise gated delta rule.
//
// One token per (sequence, head) (the "Kimi3 = GPT2 x 22580" blog, section 3
// "DeltaNet", forward() with a one-token x and cache = S; the update and the
// gated read-out of the Muir reading notes, arXiv:2611.08376, section 2.1).
//
// The state is read once and written once.  Both reductions over the key
// channels come from the same read of S:
//   r_j = sum_i (k_hat_i alpha_i) S_ij          (u = v_hat - r)
//   p_j = sum_i (qt_i alpha_i) S_ij             (o = p + (qt . kn) u)
// because o = qt (Diag(alpha) S + kn^T u).  Then S_ij <- alpha_i S_ij + kn_i u_j.
//
// Work layout: one 256-thread workgroup per (b, h).  Thread (rg, cg) owns
// rows [rg*RPT, rg*RPT+RPT) and the 4 columns [4cg, 4cg+4) of S: every row
// of S is read by D/4 consecutive threads as float4, fully coalesced, and the
// loads are issued before the pre-pass so that they are in flight meanwhile.
// HBM traffic per (b, h): 2 * D * D * 4 bytes of state plus the token inputs.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <int D, bool IN_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(256) decode_kernel(
    float *__restrict__ S, const void *__restrict__ q, const void *__restrict__ k,
    const void *__restrict__ v, const float *__restrict__ log_alpha,
    const void *__restrict__ bgate, const void *__restrict__ wgate,
    const float *__restrict__ gamma, const void *__restrict__ z, void *__restrict__ o,
    int H, int alpha_mode, int b_mode, int w_mode, int normalize_qk, float scale) {
  constexpr int NT = 256;
  constexpr int CG = D / 4;       // column groups (float4 each)
  constexpr int RG = NT / CG;     // row groups
  constexpr int RPT = D / RG;     // rows per thread
  static_assert(CG * RG == NT && RG * RPT == D, "decode tiling");

  __shared__ float s_qa[D];       // qt_i * alpha_i
  __shared__ float s_ka[D];       // k_hat_i * alpha_i
  __shared__ float s_a[D];        // alpha_i
  __shared__ float s_kn[D];       // unit key
  __shared__ float s_vh[D];       // v_hat
  __shared__ float s_red[4][4];   // cross-wave partial sums
  __shared__ float s_r[RG][D];    // partial r_j per row group
  __shared__ float s_p[RG][D];    // partial p_j per row group

  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x;   // (b, h) flattened
  const int h = (int)(bh % H);
  const int cg = tid % CG, rg = tid / CG;
  float *Sb = S + bh * (size_t)D * D;

  // 1. the token's inputs first, then the state: waiting for the former
  // leaves the state loads in flight.  Every thread loads channel tid % D
  // (threads beyond D duplicate), and each load is unconditional -- gates of
  // a constant mode read a dummy valid address -- so that no branch forces a
  // wait for every load in flight.
  const int c = tid % D;
  const size_t ix = bh * D + c;
  const void *any = q;
  const bool a_ld = alpha_mode == GDR_GATE_PER_CHANNEL || alpha_mode == GDR_GATE_PER_TOKEN;
  const bool b_ld = b_mode == GDR_GATE_PER_CHANNEL || b_mode == GDR_GATE_PER_TOKEN;
  const bool w_ld = w_mode == GDR_GATE_PER_CHANNEL || w_mode == GDR_GATE_PER_TOKEN;
  float qv = ld1<IN_BF16>(q, ix);
  float kv = ld1<IN_BF16>(k, ix);
  const float vv = ld1<IN_BF16>(v, ix);
  const float zr = ld1<IN_BF16>(z ? z : any, z ? ix : 0);
  const float gr = ld1<false>(gamma ? gamma : any, gamma ? (size_t)h * D + c : 0);
  const float lr = ld1<false>(a_ld ? log_alpha : any,
                              alpha_mode == GDR_GATE_PER_CHANNEL ? ix : (alpha_mode == GDR_GATE_PER_TOKEN ? bh : 0));
  const float br = ld1<IN_BF16>(b_ld ? bgate : any,
                                b_mode == GDR_GATE_PER_CHANNEL ? ix : (b_mode == GDR_GATE_PER_TOKEN ? bh : 0));
  const float wr = ld1<IN_BF16>(w_ld ? wgate : any,
                                w_mode == GDR_GATE_PER_CHANNEL ? ix : (w_mode == GDR_GATE_PER_TOKEN ? bh : 0));
  f32x4 sreg[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    sreg[r] = *reinterpret_cast<const f32x4 *>(Sb + (size_t)(rg * RPT + r) * D + 4 * cg);

  // 2. pre-pass: thread i < D owns channel i
  const int lane = tid % kWave, wave = tid / kWave;
  if (normalize_qk) { qv = silu(qv); kv = silu(kv); }
  float qs = tid < D ? qv * qv : 0.f, ks = tid < D ? kv * kv : 0.f;
  qs = wave_sum(qs);
  ks = wave_sum(ks);
  if (lane == 0) { s_red[0][wave] = qs; s_red[1][wave] = ks; }
  __syncthreads();
  float qkd = 0.f;
  if (tid < D) {
    float nq = 1.f, nk = 1.f;
    if (normalize_qk) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int w = 0; w < (D + kWave - 1) / kWave; ++w) { sq += s_red[0][w]; sk += s_red[1][w]; }
      nq = inv_norm(sq);
      nk = inv_norm(sk);
    }
    const float g = gamma ? gr : 1.f;
    const float dyn = z ? two_sigmoid(zr) : 1.f;
    const float qt = scale * g * dyn * qv * nq;
    const float kn = kv * nk;
    const float a = __expf(a_ld ? lr : 0.f);
    const float bb = b_ld ? br : gate_const(b_mode);
    const float ww = w_ld ? wr : gate_const(w_mode);
    s_qa[tid] = qt * a;
    s_ka[tid] = bb * kn * a;
    s_a[tid] = a;
    s_kn[tid] = kn;
    s_vh[tid] = ww * vv;
    qkd = qt * kn;
  }
  qkd = wave_sum(qkd);
  if (lane == 0) s_red[2][wave] = qkd;
  __syncthreads();
  float qk = 0.f;
#pragma unroll
  for (int w = 0; w < (D + kWave - 1) / kWave; ++w) qk += s_red[2][w];

  // 3. partial column reductions over this thread's rows
  float r4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg * RPT + r;
    const float ka = s_ka[i], qa = s_qa[i];
    r4[0] += ka * sreg[r][0]; r4[1] += ka * sreg[r][1]; r4[2] += ka * sreg[r][2]; r4[3] += ka * sreg[r][3];
    p4[0] += qa * sreg[r][0]; p4[1] += qa * sreg[r][1]; p4[2] += qa * sreg[r][2]; p4[3] += qa * sreg[r][3];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) { s_r[rg][4 * cg + c] = r4[c]; s_p[rg][4 * cg + c] = p4[c]; }
  __syncthreads();

  // 4. u_j and o_j for this thread's 4 columns
  float u[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = 4 * cg + c;
    float rr = 0.f, pp = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) { rr += s_r[g2][j]; pp += s_p[g2][j]; }
    u[c] = s_vh[j] - rr;
    if (rg == 0) st1<OUT_BF16>(o, bh * D + j, pp + qk * u[c]);
  }

  // 5. write the new state, past the caches: nothing reads it again in this
  // step, and a batch's states rarely fit the last-level cache (4096 streams
  // of d = 128 hold 268 MB)
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg * RPT + r;
    const float a = s_a[i], kn = s_kn[i];
    f32x4 nv;
    nv[0] = a * sreg[r][0] + kn * u[0];
    nv[1] = a * sreg[r][1] + kn * u[1];
    nv[2] = a * sreg[r][2] + kn * u[2];
    nv[3] = a * sreg[r][3] + kn * u[3];
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(Sb + (size_t)i * D + 4 * cg));
  }
}

template <int D, bool IB, bool OB>
static hipError_t launch_decode_t(const gdr_desc &d, float *S, const void *q, const void *k,
                                  const void *v, const float *la, const void *b, const void *w,
                                  const float *gamma, const void *z, void *o, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, IB, OB>), dim3((unsigned)((size_t)d.B * d.H)), dim3(256), 0,
                     st, S, q, k, v, la, b, w, gamma, z, o, d.H, (int)d.alpha_mode, (int)d.b_mode,
                     (int)d.w_mode, d.normalize_qk, d.scale);
  return hipGetLastError();
}

hipError_t launch_decode(const gdr_desc &d, float *S, const void *q, const void *k, const void *v,
                         const float *la, const void *b, const void *w, const float *gamma,
                         const void *z, void *o, hipStream_t st) {
  const bool ib = d.in_dtype == GDR_BF16, ob = d.out_dtype == GDR_BF16;
#define GDR_DEC(DD, IB, OB)                                                              \
  if (d.dk == DD && ib == IB && ob == OB)                                                \
    return launch_decode_t<DD, IB, OB>(d, S, q, k, v, la, b, w, gamma, z, o, st);
  GDR_DEC(128, true, false) GDR_DEC(128, true, true) GDR_DEC(128, false, false)
  GDR_DEC(128, false, true) GDR_DEC(64, true, false) GDR_DEC(64, true, true)
  GDR_DEC(64, false, false) GDR_DEC(64, false, true)
#undef GDR_DEC
  return hipErrorInvalidValue;
}

}  // namespace gdr
