// gdr_gate.hip -- the five-gate low-rank projection that feeds the pre-pass
// (Muir reading notes, arXiv:2611.08376, section 2.3: one shared down-
// projection of the layer input, then per gate an up-projection and a channel
// bias give the logits of decay f, erase b, output gate g, write w and query
// gain q; ranks (r_f, r_b, r_g, r_w, r_q)).  Activations and layouts are this
// library's reading (stated in gdr.h).
//
// Two kernels:
//   down: Hlat[N, R] fp32 = X[N, dm] Wd^T       (bf16 operands, exact products)
//   up:   per gate, logits[N, H*d] = Hlat[:, gate's ranks] Wu_g^T + bias_g,
//         activation, written head-major [B, H, T, d]
// Weights use the [out, in] row-major convention, so every MFMA operand
// fragment is 16 contiguous bytes of one row.
#include <stdint.h>

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

namespace {

constexpr int kGates = 5;

// ---------------------------------------------------------------------------
// down: workgroup tile 128 tokens x 128 latent columns, 8 waves (wave w: tokens
// 16w .. 16w+15), k-steps of 32.  The Wd tile of a k-step (128 rows x 32) is
// staged in LDS (double-buffered, one barrier per step); X fragments come
// straight from global memory.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) gate_down_kernel(GateArgs a) {
  __shared__ __align__(16) uint16_t wt[2][128 * 32];  // [buffer][latent row][k]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 128, c0 = blockIdx.y * 128;
  const int n = min(n0 + 16 * wave + l16, a.N - 1);  // clamped: rows past N are not stored
  const uint16_t *xrow = a.x + (size_t)n * a.dm + 8 * g;
  // staging: thread -> (latent row tid / 4, 8 k values (tid % 4) * 8); rows
  // past R (a last, partial column tile) read row R - 1 and are not stored
  const int sr = tid >> 2, sk = (tid & 3) * 8;
  const uint16_t *wsrc = a.wd + (size_t)min(c0 + sr, a.R - 1) * a.dm + sk;
  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = zero4();
  const int nk = a.dm / 32;
  *reinterpret_cast<uint4 *>(&wt[0][sr * 32 + sk]) = *reinterpret_cast<const uint4 *>(wsrc);
  __syncthreads();
#pragma unroll 1
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    // the next k-step's tile (the last step re-reads its own: no branch around the load)
    const uint4 wnext = *reinterpret_cast<const uint4 *>(wsrc + min(ks + 1, nk - 1) * 32);
    const bf16x8 xa = *reinterpret_cast<const bf16x8 *>(xrow + ks * 32);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const bf16x8 wb = *reinterpret_cast<const bf16x8 *>(&wt[cur][(16 * ct + l16) * 32 + 8 * g]);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, acc[ct], 0, 0, 0);
    }
    if (ks + 1 < nk) *reinterpret_cast<uint4 *>(&wt[cur ^ 1][sr * 32 + sk]) = wnext;
    __syncthreads();
  }
  // accumulator: lane (column l16, rows 4g .. 4g+3) of each 16 x 16 tile
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int nr = n0 + 16 * wave + 4 * g + r;
    if (nr >= a.N) continue;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      if (c0 + 16 * ct + l16 < a.R) a.hlat[(size_t)nr * a.R + c0 + 16 * ct + l16] = acc[ct][r];
  }
}

// ---------------------------------------------------------------------------
// up: workgroup = 128 tokens x one gate, looping over the heads; 8 waves (wave
// w: tokens 16w .. 16w+15).  The latent fragments of the gate's ranks are
// loaded once, split into hi / lo bf16 planes (the weights are exact bf16, so
// two products per fragment keep ~16 bits of the fp32 latent), and reused for
// every head's d output channels.
// ---------------------------------------------------------------------------
template <int D, bool OB16>
__global__ void __launch_bounds__(512) gate_up_kernel(GateArgs a) {
  constexpr int NCT = D / 16;
  const int gate = blockIdx.y;
  void *outp = a.out[gate];
  if (!outp) return;  // this gate is not wanted
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 128;
  const int n = min(n0 + 16 * wave + l16, a.N - 1);
  const int rank = a.rank[gate], roff = a.roff[gate];
  const int nk = rank / 32;  // <= 4
  bf16x8 hf[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks >= nk) continue;
    const float4 *src = reinterpret_cast<const float4 *>(a.hlat + (size_t)n * a.R + roff + 32 * ks + 8 * g);
    const float4 f0 = src[0], f1 = src[1];
    const float x[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    split8<2>(x, hf[ks]);
  }
  const uint16_t *wu = a.wu + a.wuoff[gate];  // [H*D, rank]
  const size_t T = (size_t)a.T;
#pragma unroll 1
  for (int hh = 0; hh < a.H; ++hh) {
    f32x4 acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks >= nk) continue;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int j = hh * D + 16 * ct + l16;
        const bf16x8 wb = *reinterpret_cast<const bf16x8 *>(wu + (size_t)j * rank + 32 * ks + 8 * g);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hf[ks][1], wb, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hf[ks][0], wb, acc[ct], 0, 0, 0);
      }
    }
    // epilogue: bias, activation, head-major store of token rows 4g + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nr = n0 + 16 * wave + 4 * g + r;
      if (nr >= a.N) continue;
      const size_t b = (size_t)nr / T, t = (size_t)nr % T;
      const size_t orow = (b * a.H + hh) * T + t;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int c = 16 * ct + l16;
        float l = acc[ct][r] + (a.bias ? a.bias[(size_t)gate * a.H * D + hh * D + c] : 0.f);
        if (gate == 0) {  // log alpha = log sigmoid(l) = -softplus(-l), fp32
          const float u = -l;
          reinterpret_cast<float *>(outp)[orow * D + c] = -(fmaxf(u, 0.f) + __logf(1.f + __expf(-fabsf(u))));
          continue;
        }
        if (gate == 1) l = 2.f / (1.f + __expf(-l));  // erase b in (0, 2)
        if (gate == 3) l = 1.f / (1.f + __expf(-l));  // write w in (0, 1)
        st1<OB16>(outp, orow * D + c, l);              // g and q stay logits
      }
    }
  }
}

}  // namespace

hipError_t launch_gate_proj(const GateArgs &a, int d, bool out_bf16, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const dim3 gdown((a.N + 127) / 128, (a.R + 127) / 128);
  hipLaunchKernelGGL(gate_down_kernel, gdown, dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gup((a.N + 127) / 128, kGates);
  if (d == 128 && out_bf16) hipLaunchKernelGGL((gate_up_kernel<128, true>), gup, dim3(512), 0, st, a);
  else if (d == 128) hipLaunchKernelGGL((gate_up_kernel<128, false>), gup, dim3(512), 0, st, a);
  else if (out_bf16) hipLaunchKernelGGL((gate_up_kernel<64, true>), gup, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((gate_up_kernel<64, false>), gup, dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdr
