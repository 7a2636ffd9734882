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
// fragment is 16 contiguous bytes of one row.  Both kernels put the weight
// rows in the MFMA's A operand and the tokens in its B operand: a lane's
// accumulator then holds four output columns of one token (the up kernel
// orders its weight rows so that two tiles give a lane eight consecutive
// columns).
#include <stdint.h>

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

namespace {

constexpr int kGates = 5;

// ---------------------------------------------------------------------------
// down: workgroup tile 256 tokens x 256 latent columns, 8 waves as 4 token
// groups x 2 latent halves (wave tile: 64 tokens x 128 latent, 4 x 8 MFMA
// tiles: 12 fragment reads from LDS per 32 products).  k-steps of 32: both
// operand tiles of a step are staged in LDS (double-buffered, rows padded to
// 40 elements so that the 16 rows of a fragment read fall in distinct
// banks); 80 KB, one workgroup per CU.  The x tile of step k + 4 (streamed
// from HBM) and the Wd tile of step k + 2 (L2-resident) are fetched into
// registers at the start of step k, so enough bytes are in flight to cover
// the memory latency; step k commits the tiles of step k + 1 after its
// products.  The loop runs four steps per iteration with the register slots
// named, so no register copy waits for a load in flight.
// ---------------------------------------------------------------------------
constexpr int kDnTok = 256, kDnLat = 256, kDnK = 32, kDnRow = kDnK + 8;
constexpr int kDnWaveTok = 64, kDnWaveLat = 128;  // wave tile
constexpr int kDnMT = kDnWaveTok / 16, kDnNT = kDnWaveLat / 16;

__global__ void __launch_bounds__(512) gate_down_kernel(GateArgs a) {
  __shared__ __align__(16) uint16_t xs[2][kDnTok * kDnRow];  // [buffer][token][k]
  __shared__ __align__(16) uint16_t ws[2][kDnLat * kDnRow];  // [buffer][latent][k]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int wt = wave & 3, wl = wave >> 2;  // token group, latent half
  const int n0 = blockIdx.x * kDnTok, c0 = blockIdx.y * kDnLat;
  // staging: thread -> rows tid / 4 and 128 + tid / 4 of each tile, 8 k
  // values (tid % 4) * 8; rows past N or R read the last row and are never
  // stored
  const int sr = tid >> 2, sk = (tid & 3) * 8;
  const uint16_t *xsrc0 = a.x + (size_t)min(n0 + sr, a.N - 1) * a.dm + sk;
  const uint16_t *xsrc1 = a.x + (size_t)min(n0 + 128 + sr, a.N - 1) * a.dm + sk;
  const uint16_t *wsrc0 = a.wd + (size_t)min(c0 + sr, a.R - 1) * a.dm + sk;
  const uint16_t *wsrc1 = a.wd + (size_t)min(c0 + 128 + sr, a.R - 1) * a.dm + sk;
  const int so = sr * kDnRow + sk;
  const int nk = a.dm / kDnK;  // d_model is a multiple of 32
  struct Pair {
    u32x4 r0, r1;
  };
  // steps past the last are clamped to it (re-loads, no branch around a load)
  auto ld2 = [&](const uint16_t *p0, const uint16_t *p1, int ks) {
    const int k = min(ks, nk - 1) * kDnK;
    return Pair{*reinterpret_cast<const u32x4 *>(p0 + k), *reinterpret_cast<const u32x4 *>(p1 + k)};
  };
  auto ldx = [&](int ks) { return ld2(xsrc0, xsrc1, ks); };
  auto ldw = [&](int ks) { return ld2(wsrc0, wsrc1, ks); };
  auto commit = [&](int buf, const Pair &rx, const Pair &rw) {
    *reinterpret_cast<u32x4 *>(&xs[buf][so]) = rx.r0;
    *reinterpret_cast<u32x4 *>(&xs[buf][so + 128 * kDnRow]) = rx.r1;
    *reinterpret_cast<u32x4 *>(&ws[buf][so]) = rw.r0;
    *reinterpret_cast<u32x4 *>(&ws[buf][so + 128 * kDnRow]) = rw.r1;
  };
  f32x4 acc[kDnMT][kDnNT];
#pragma unroll
  for (int tt = 0; tt < kDnMT; ++tt)
#pragma unroll
    for (int ct = 0; ct < kDnNT; ++ct) acc[tt][ct] = zero4();
  auto products = [&](int buf) {
    const uint16_t *xc = &xs[buf][(wt * kDnWaveTok + l16) * kDnRow + 8 * g];
    const uint16_t *wc = &ws[buf][(wl * kDnWaveLat + l16) * kDnRow + 8 * g];
    bf16x8 xb[kDnMT];
#pragma unroll
    for (int tt = 0; tt < kDnMT; ++tt) xb[tt] = *reinterpret_cast<const bf16x8 *>(xc + 16 * tt * kDnRow);
#pragma unroll
    for (int ct = 0; ct < kDnNT; ++ct) {
      const bf16x8 wa = *reinterpret_cast<const bf16x8 *>(wc + 16 * ct * kDnRow);
#pragma unroll
      for (int tt = 0; tt < kDnMT; ++tt)
        acc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb[tt], acc[tt][ct], 0, 0, 0);
    }
  };
  // step ks: fetch x(ks + 4) into the slot x(ks) left, Wd(ks + 2) into the
  // slot Wd(ks) left; products of step ks; commit x(ks + 1), Wd(ks + 1)
  auto step = [&](int ks, Pair &x_ld, const Pair &x_cm, Pair &w_ld, const Pair &w_cm) {
    x_ld = ldx(ks + 4);
    w_ld = ldw(ks + 2);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (ks < nk) products(ks & 1);  // uniform; no load inside
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // buffer (ks + 1) & 1 was last read in step ks - 1, before the barrier that ended it
    commit((ks + 1) & 1, x_cm, w_cm);
    __syncthreads();
  };
  Pair x0 = ldx(0), x1 = ldx(1), x2 = ldx(2), x3 = ldx(3);
  Pair w0 = ldw(0), w1 = ldw(1);
  commit(0, x0, w0);
  __syncthreads();
#pragma unroll 1
  for (int ks = 0; ks < nk; ks += 4) {
    step(ks + 0, x0, x1, w0, w1);
    step(ks + 1, x1, x2, w1, w0);
    step(ks + 2, x2, x3, w0, w1);
    step(ks + 3, x3, x0, w1, w0);
  }
  // accumulator: lane (token l16 of tile tt, latent columns 16 ct + 4g .. +3)
#pragma unroll
  for (int tt = 0; tt < kDnMT; ++tt) {
    const int n = n0 + wt * kDnWaveTok + 16 * tt + l16;
    if (n >= a.N) continue;
    float *dst = a.hlat + (size_t)n * a.R + c0 + wl * kDnWaveLat + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kDnNT; ++ct)
      if (c0 + wl * kDnWaveLat + 16 * ct + 4 * g < a.R) *reinterpret_cast<f32x4 *>(dst + 16 * ct) = acc[tt][ct];
  }
}

// ---------------------------------------------------------------------------
// up: workgroup = 16 kUpWaves tokens x one gate, looping over the heads (wave
// w: tokens 16w .. 16w+15).  The latent fragments of the gate's ranks are
// loaded once, split into hi / lo bf16 planes (the weights are exact bf16, so
// two products per fragment keep ~16 bits of the fp32 latent), and reused for
// every head's d output channels.  A head's weight tile (d rows x rank, one
// contiguous block) and bias go through LDS, double-buffered: the workgroup
// fetches head h + 1's tile from global memory while its waves multiply head
// h's, one barrier per head.
// ---------------------------------------------------------------------------
struct ActLogSigmoid {  // log alpha = log sigmoid(l), fp32
  __device__ float operator()(float l) const { return fminf(l, 0.f) - __logf(1.f + __expf(-fabsf(l))); }
};
struct ActTwoSigmoid {  // erase b in (0, 2)
  __device__ float operator()(float l) const { return two_sigmoid(l); }
};
struct ActSigmoid {  // write w in (0, 1)
  __device__ float operator()(float l) const { return fast_rcp(1.f + __expf(-l)); }
};
struct ActLogit {  // g and q stay logits
  __device__ float operator()(float l) const { return l; }
};

__device__ __align__(16) float kZeroBias[128] = {};  // read only; global, like the bias

constexpr int kUpWaves = 8;            // waves (16 tokens each) per up workgroup
constexpr int kUpThreads = 64 * kUpWaves;
constexpr int kWRowMax = 128 + 8;      // LDS weight row: rank + 8 (16-byte pad), rank <= 128

template <int D, typename OT, int NK>
__device__ __forceinline__ void gate_up_heads(const GateArgs &a, int gate, OT *out, uint16_t *wl, float *bl, int n0,
                                              int tid) {
  constexpr int NCT = D / 16;
  constexpr bool F32 = sizeof(OT) == 4;
  constexpr int RANK = 32 * NK;
  constexpr int WROW = RANK + 8;               // padded row: the 16 rows of a fragment read hit distinct banks
  constexpr int WBUF = D * WROW;               // elements per weight buffer
  constexpr int PIECES = D * RANK / 8;         // 16-byte pieces of one head's weight tile
  constexpr int PPT = (PIECES + kUpThreads - 1) / kUpThreads;
  static_assert(WROW <= kWRowMax, "weight rows exceed the LDS buffer");
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  // latent fragments of this gate's ranks (B operand: token l16, k 8g .. 8g+7)
  bf16x8 hf[NK][2];
  {
    const int n = min(n0 + l16, a.N - 1);
    const float *hsrc = a.hlat + (size_t)n * a.R + a.roff[gate] + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const float4 f0 = *reinterpret_cast<const float4 *>(hsrc + 32 * ks);
      const float4 f1 = *reinterpret_cast<const float4 *>(hsrc + 32 * ks + 4);
      const float x[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      split8<2>(x, hf[ks]);
    }
  }
  // this lane's output row: (b H + 0) T + t; the head adds h T
  const int nt = n0 + l16;
  const bool live = nt < a.N;
  const uint32_t bq = (uint32_t)nt / (uint32_t)a.T;
  const uint32_t rb = bq * (uint32_t)a.H * (uint32_t)a.T + ((uint32_t)nt - bq * (uint32_t)a.T);
  const uint16_t *wu = a.wu + a.wuoff[gate];  // [H*D, RANK]; head h's tile starts at h D RANK
  const float *bias0 = a.bias ? a.bias + (size_t)gate * a.H * D : kZeroBias;
  const int bstep = a.bias ? D : 0;
  // head tile fetch (global -> registers) and commit (registers -> LDS buffer);
  // surplus pieces are clamped to the last one (same value written twice)
  // (plain vector types: a struct-typed array here is not promoted to registers)
  u32x4 pw[PPT];
  f32x4 pb;
  auto fetch = [&](int hh) {
    const uint16_t *src = wu + (size_t)hh * D * RANK;
#pragma unroll
    for (int p = 0; p < PPT; ++p) pw[p] = *reinterpret_cast<const u32x4 *>(src + 8 * min(tid + p * kUpThreads, PIECES - 1));
    pb = *reinterpret_cast<const f32x4 *>(bias0 + hh * bstep + 4 * min(tid, D / 4 - 1));
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int i = min(tid + p * kUpThreads, PIECES - 1);
      *reinterpret_cast<u32x4 *>(wl + buf * WBUF + (i / (RANK / 8)) * WROW + 8 * (i % (RANK / 8))) = pw[p];
    }
    if (tid < D / 4) *reinterpret_cast<f32x4 *>(bl + buf * D + 4 * tid) = pb;
  };
  // epilogue: bias and activation, stored straight from the accumulator
  // layout (lane: token l16; tiles 2j, 2j + 1 hold its channels 32 j + 8 g ..
  // + 7: one 16-byte store in bf16, two in fp32; the four lanes of a token
  // cover 64 or 128 contiguous bytes)
  auto epilogue = [&](const f32x4 (&acc)[NCT], const float *bb, int hh, auto act) {
    OT *orow = out + ((size_t)rb + (size_t)hh * a.T) * D + 8 * g;
#pragma unroll
    for (int j = 0; j < NCT / 2; ++j) {
      const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bb + 32 * j + 8 * g);
      const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bb + 32 * j + 8 * g + 4);
      float y[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = act(acc[2 * j][r] + b0[r]);
        y[4 + r] = act(acc[2 * j + 1][r] + b1[r]);
      }
      if (live) {
        if constexpr (F32) {
          *reinterpret_cast<f32x4 *>(orow + 32 * j) = f32x4{y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4 *>(orow + 32 * j + 4) = f32x4{y[4], y[5], y[6], y[7]};
        } else {
          uint4 pk;
          pk.x = pack_bf16x2(y[0], y[1]);
          pk.y = pack_bf16x2(y[2], y[3]);
          pk.z = pack_bf16x2(y[4], y[5]);
          pk.w = pack_bf16x2(y[6], y[7]);
          *reinterpret_cast<uint4 *>(orow + 32 * j) = pk;
        }
      }
    }
  };
  fetch(0);
  commit(0);
  __syncthreads();
#pragma unroll 1
  for (int hh = 0; hh < a.H; ++hh) {
    const int cur = hh & 1;
    fetch(min(hh + 1, a.H - 1));  // the last head re-fetches its own tile: no branch around a load
    // the fetch is issued before the products and committed after them, so
    // its latency hides behind them: keep the compiler from moving either
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = zero4();
    // tile ct, row i holds channel 32 (ct / 2) + 8 (i / 4) + 4 (ct % 2) + i % 4, so
    // that a lane's accumulators of tiles 2j, 2j + 1 are 8 consecutive channels
    const uint16_t *wc = wl + cur * WBUF + (8 * (l16 >> 2) + (l16 & 3)) * WROW + 8 * g;
    // per k-step and pair of tiles: the pair's weight fragments read first,
    // then its lo products and its hi products, so that an LDS read and the
    // previous product on the same accumulator overlap other products (pairs
    // keep the kernel within 128 registers; groups of 4 spilled)
    constexpr int TG = 2;
    static_assert(NCT % TG == 0, "whole pairs of tiles");
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int c0 = 0; c0 < NCT; c0 += TG) {
        bf16x8 wb[TG];
#pragma unroll
        for (int u = 0; u < TG; ++u) {
          const int ct = c0 + u;
          wb[u] = *reinterpret_cast<const bf16x8 *>(wc + (32 * (ct >> 1) + 4 * (ct & 1)) * WROW + 32 * ks);
        }
#pragma unroll
        for (int u = 0; u < TG; ++u)
          acc[c0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[u], hf[ks][1], acc[c0 + u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < TG; ++u)
          acc[c0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[u], hf[ks][0], acc[c0 + u], 0, 0, 0);
      }
    // buffer cur ^ 1 was last read in head hh - 1, which every wave finished
    // before the barrier that ended it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    commit(cur ^ 1);
    const float *bb = bl + cur * D;
    if (gate == 0) epilogue(acc, bb, hh, ActLogSigmoid{});
    else if (gate == 1) epilogue(acc, bb, hh, ActTwoSigmoid{});
    else if (gate == 3) epilogue(acc, bb, hh, ActSigmoid{});
    else epilogue(acc, bb, hh, ActLogit{});
    __syncthreads();
  }
}

template <int D, typename OT>
__device__ __forceinline__ void gate_up_ranks(const GateArgs &a, int gate, OT *out, uint16_t *wl, float *bl, int n0,
                                              int tid) {
  switch (a.rank[gate] / 32) {
    case 1: gate_up_heads<D, OT, 1>(a, gate, out, wl, bl, n0, tid); break;
    case 2: gate_up_heads<D, OT, 2>(a, gate, out, wl, bl, n0, tid); break;
    case 3: gate_up_heads<D, OT, 3>(a, gate, out, wl, bl, n0, tid); break;
    default: gate_up_heads<D, OT, 4>(a, gate, out, wl, bl, n0, tid); break;
  }
}

template <int D, bool OB16>
__global__ void __launch_bounds__(kUpThreads) __attribute__((amdgpu_waves_per_eu(4))) gate_up_kernel(GateArgs a) {
  __shared__ __align__(16) uint16_t wl[2 * D * kWRowMax];
  __shared__ __align__(16) float bl[2 * D];
  const int gate = blockIdx.y;
  void *outp = a.out[gate];
  if (!outp) return;  // this gate is not wanted (uniform over the workgroup)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * (16 * kUpWaves) + 16 * wave;
  if (gate == 0 || !OB16)
    gate_up_ranks<D, float>(a, gate, static_cast<float *>(outp), wl, bl, n0, tid);
  else
    gate_up_ranks<D, uint16_t>(a, gate, static_cast<uint16_t *>(outp), wl, bl, n0, tid);
}

}  // namespace

hipError_t launch_gate_proj(const GateArgs &a, int d, bool out_bf16, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const dim3 gdown((a.N + kDnTok - 1) / kDnTok, (a.R + kDnLat - 1) / kDnLat);
  hipLaunchKernelGGL(gate_down_kernel, gdown, dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gup((a.N + 16 * kUpWaves - 1) / (16 * kUpWaves), kGates);
  const dim3 bup(kUpThreads);
  if (d == 128 && out_bf16) hipLaunchKernelGGL((gate_up_kernel<128, true>), gup, bup, 0, st, a);
  else if (d == 128) hipLaunchKernelGGL((gate_up_kernel<128, false>), gup, bup, 0, st, a);
  else if (out_bf16) hipLaunchKernelGGL((gate_up_kernel<64, true>), gup, bup, 0, st, a);
  else hipLaunchKernelGGL((gate_up_kernel<64, false>), gup, bup, 0, st, a);
  return hipGetLastError();
}

}  // namespace gdr
