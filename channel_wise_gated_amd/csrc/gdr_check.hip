// gdr_check.hip -- the opt-in precondition check of the token inputs.
//
// The chunkwise forward, its backward and the decode step take their inputs
// as the caller hands them over: a non-finite gate or a log-decay outside
// the range the pivots are built for is not looked for on the hot path.
// This kernel counts such elements, per tensor, so that a caller can test a
// batch off the hot path (a debugging or data-validation step).  Preconditions
// (the recurrence's decay is a product of factors alpha in (0, 1], so log
// alpha <= 0; the pivoted factors stay in fp32 range for log alpha >= -30):
//   q, k, v, b, w, z, gamma: finite;  log alpha: finite and in [-30, 0].
#include <stdint.h>

#include <algorithm>

#include "gdr_launch.h"

namespace gdr {

namespace {

constexpr float kLogAlphaMin = -30.f;
constexpr int kCheckThreads = 256;

__device__ __forceinline__ unsigned bad_bf16(uint32_t h) { return (h & 0x7F80u) == 0x7F80u; }
__device__ __forceinline__ unsigned bad_f32(float x, bool range) {
  if ((__float_as_uint(x) & 0x7F800000u) == 0x7F800000u) return 1u;  // NaN or +-inf
  return range && (x > 0.f || x < kLogAlphaMin) ? 1u : 0u;
}

struct CheckArgs {
  CheckTensor t[kCheckCounts];
  unsigned long long *counts;
};

__global__ void __launch_bounds__(kCheckThreads) check_zero_kernel(unsigned long long *counts) {
  if (threadIdx.x < kCheckCounts) counts[threadIdx.x] = 0ull;
}

// blockIdx.y: the tensor; the blocks along x stride over its elements in
// 16-byte groups, then the elements past the last whole group one by one.
__global__ void __launch_bounds__(kCheckThreads) check_kernel(CheckArgs a) {
  const CheckTensor t = a.t[blockIdx.y];
  const size_t stride = (size_t)gridDim.x * kCheckThreads;
  const size_t first = (size_t)blockIdx.x * kCheckThreads + threadIdx.x;
  unsigned cnt = 0;
  if (t.p) {
    if (t.bf16) {
      const uint16_t *p = static_cast<const uint16_t *>(t.p);
      const size_t ng = t.n / 8;
      for (size_t i = first; i < ng; i += stride) {
        const uint4 u = reinterpret_cast<const uint4 *>(p)[i];
        cnt += bad_bf16(u.x) + bad_bf16(u.x >> 16) + bad_bf16(u.y) + bad_bf16(u.y >> 16) + bad_bf16(u.z) +
               bad_bf16(u.z >> 16) + bad_bf16(u.w) + bad_bf16(u.w >> 16);
      }
      for (size_t i = ng * 8 + first; i < t.n; i += stride) cnt += bad_bf16(p[i]);
    } else {
      const float *p = static_cast<const float *>(t.p);
      const bool range = t.range != 0;
      const size_t ng = t.n / 4;
      for (size_t i = first; i < ng; i += stride) {
        const float4 f = reinterpret_cast<const float4 *>(p)[i];
        cnt += bad_f32(f.x, range) + bad_f32(f.y, range) + bad_f32(f.z, range) + bad_f32(f.w, range);
      }
      for (size_t i = ng * 4 + first; i < t.n; i += stride) cnt += bad_f32(p[i], range);
    }
  }
  // workgroup sum (with the grid below a thread visits at most 2^21
  // elements for n <= 2^40, a wave at most 2^27), one 64-bit atomic add per
  // workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  __shared__ unsigned part[kCheckThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
#pragma unroll
    for (int w = 0; w < kCheckThreads / 64; ++w) s += part[w];
    if (s) atomicAdd(a.counts + blockIdx.y, s);
  }
}

}  // namespace

hipError_t launch_check(const CheckTensor (&t)[kCheckCounts], unsigned long long *counts, hipStream_t st) {
  hipLaunchKernelGGL(check_zero_kernel, dim3(1), dim3(kCheckThreads), 0, st, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long nmax = 0;
  CheckArgs a{};
  for (int i = 0; i < kCheckCounts; ++i) {
    a.t[i] = t[i];
    if (t[i].p && t[i].n > nmax) nmax = t[i].n;
  }
  if (nmax == 0) return hipSuccess;
  a.counts = counts;
  // about 8 groups of 16 bytes per thread for the largest tensor, at most
  // 2048 workgroups per tensor
  const unsigned long long per_block = (unsigned long long)kCheckThreads * 8 * 8;
  const unsigned nx = (unsigned)std::min<unsigned long long>(2048, (nmax + per_block - 1) / per_block);
  hipLaunchKernelGGL(check_kernel, dim3(nx, kCheckCounts), dim3(kCheckThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdr
