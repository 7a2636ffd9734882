// gdr_device.h -- device helpers shared by the gfx950 kernels of libgdr.
//
// bf16 storage, fp32 arithmetic, hi/lo bf16 operand splits for the matrix
// cores, and the two MFMA shapes the kernels use.
//
// MFMA lane layouts (wave64, verified on gfx950 by an in-bounds probe):
//   v_mfma_f32_16x16x32_bf16   A (16 x 32): lane l holds row l%16, k = 8*(l/16) + e, e < 8
//                              B (32 x 16): lane l holds col l%16, k = 8*(l/16) + e
//                              D (16 x 16): lane l holds col l%16, rows 4*(l/16) + r, r < 4
//   v_mfma_f32_16x16x16_bf16   same with k = 4*(l/16) + e, e < 4
// The contraction index k may be permuted freely as long as A and B use the
// same permutation; the kernels use that to feed accumulator tiles (rows
// 4*(l/16)+r) straight back in as operands: within a 32-wide k-step that
// covers 16-row tiles m0 and m0+1, lane group g = l/16 and element e stand for
// row 16*(m0 + e/4) + 4*g + e%4 ("tile-pair order").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/gdr.h"

namespace gdr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, b);
}
// Two floats to two bf16 (round to nearest even, as above) in one 32-bit word,
// x in the low half: one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}
__device__ __forceinline__ float round_bf16(float x) {
  return bf16_bits_to_f32(f32_to_bf16_bits(x));
}

// Load one element of a tensor stored as bf16 or f32.
template <bool BF16>
__device__ __forceinline__ float ld1(const void *p, size_t i) {
  if constexpr (BF16)
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
  else
    return reinterpret_cast<const float *>(p)[i];
}

// Load 4 consecutive elements (i multiple of 4; 8- or 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void ld4(const void *p, size_t i, float out[4]) {
  if constexpr (BF16) {
    uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
    out[0] = __uint_as_float(u.x << 16);
    out[1] = __uint_as_float(u.x & 0xffff0000u);
    out[2] = __uint_as_float(u.y << 16);
    out[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
    out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
  }
}

// Load 8 consecutive elements (i multiple of 8).
template <bool BF16>
__device__ __forceinline__ void ld8(const void *p, size_t i, float out[8]) {
  if constexpr (BF16) {
    uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p) + i);
    out[0] = __uint_as_float(u.x << 16); out[1] = __uint_as_float(u.x & 0xffff0000u);
    out[2] = __uint_as_float(u.y << 16); out[3] = __uint_as_float(u.y & 0xffff0000u);
    out[4] = __uint_as_float(u.z << 16); out[5] = __uint_as_float(u.z & 0xffff0000u);
    out[6] = __uint_as_float(u.w << 16); out[7] = __uint_as_float(u.w & 0xffff0000u);
  } else {
    const float4 *f = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
    float4 a = f[0], b = f[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

// Store 8 consecutive elements (i multiple of 8).
template <bool BF16>
__device__ __forceinline__ void st8(void *p, size_t i, const float x[8]) {
  if constexpr (BF16) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
    u.z = (uint32_t)f32_to_bf16_bits(x[4]) | ((uint32_t)f32_to_bf16_bits(x[5]) << 16);
    u.w = (uint32_t)f32_to_bf16_bits(x[6]) | ((uint32_t)f32_to_bf16_bits(x[7]) << 16);
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p) + i) = u;
  } else {
    float4 *f = reinterpret_cast<float4 *>(reinterpret_cast<float *>(p) + i);
    f[0] = make_float4(x[0], x[1], x[2], x[3]);
    f[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// Streaming stores of outputs the kernel never reads back (nontemporal: no
// reuse expected in the caches).
template <bool BF16>
__device__ __forceinline__ void st1_stream(void *p, size_t i, float x) {
  if constexpr (BF16)
    __builtin_nontemporal_store(f32_to_bf16_bits(x), reinterpret_cast<uint16_t *>(p) + i);
  else
    __builtin_nontemporal_store(x, reinterpret_cast<float *>(p) + i);
}

// ... and of 4 consecutive elements (i multiple of 4; 8- or 16-byte aligned).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ void st4_stream(void *p, size_t i, f32x4 x) {
  if constexpr (BF16)
    __builtin_nontemporal_store(u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])},
                                reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(p) + i));
  else
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p) + i));
}

template <bool BF16>
__device__ __forceinline__ void st1(void *p, size_t i, float x) {
  if constexpr (BF16)
    reinterpret_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(x);
  else
    reinterpret_cast<float *>(p)[i] = x;
}

// ---------------------------------------------------------------- math
// Hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE division.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// x * sigmoid(x); e^-x = inf for very negative x gives rcp(inf) = 0 and -0.
__device__ __forceinline__ float silu(float x) { return x * fast_rcp(1.0f + __expf(-x)); }
__device__ __forceinline__ float two_sigmoid(float x) { return 2.0f * fast_rcp(1.0f + __expf(-x)); }
// 1 / max(|x|_2, 1e-12) from a sum of squares (the l2 normalisation floor).
__device__ __forceinline__ float inv_norm(float sumsq) { return fast_rcp(fmaxf(sqrtf(sumsq), 1e-12f)); }

// ---------------------------------------------------------------- hi/lo splits
// x ~= sum_{p < NS} plane_p(x), each plane a bf16.  NS = 2 keeps ~16 mantissa
// bits, NS = 3 ~24 (fp32).
template <int NS>
__device__ __forceinline__ void split(float x, uint16_t out[NS]) {
  float r = x;
#pragma unroll
  for (int p = 0; p < NS; ++p) {
    uint16_t h = f32_to_bf16_bits(r);
    out[p] = h;
    r = r - bf16_bits_to_f32(h);
  }
}

// Eight fp32 values -> NS packed bf16x8 fragments.
template <int NS>
__device__ __forceinline__ void split8(const float x[8], bf16x8 out[NS]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint16_t h[NS];
    split<NS>(x[e], h);
#pragma unroll
    for (int p = 0; p < NS; ++p) out[p][e] = __builtin_bit_cast(__bf16, h[p]);
  }
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split product: sum over plane pairs (pa, pb) with pa + pb < NS.
template <int NS>
__device__ __forceinline__ f32x4 mfma32_split(const bf16x8 a[NS], const bf16x8 b[NS], f32x4 c) {
  // small terms first
#pragma unroll
  for (int s = NS - 1; s >= 0; --s)
#pragma unroll
    for (int pa = 0; pa <= s; ++pa) c = mfma32(a[pa], b[s - pa], c);
  return c;
}

// Two independent split products, c0 += a0 b0 and c1 += a1 b1, each in the
// order of mfma32_split (so bit-identical to two such calls), issued
// alternately so that neither waits for its own previous product.
template <int NS>
__device__ __forceinline__ void mfma32_split2(const bf16x8 a0[NS], const bf16x8 b0[NS], f32x4 &c0,
                                              const bf16x8 a1[NS], const bf16x8 b1[NS], f32x4 &c1) {
#pragma unroll
  for (int s = NS - 1; s >= 0; --s)
#pragma unroll
    for (int pa = 0; pa <= s; ++pa) {
      c0 = mfma32(a0[pa], b0[s - pa], c0);
      c1 = mfma32(a1[pa], b1[s - pa], c1);
    }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- gates
// Value of a gate for element (token row `row`, channel `c`) of a tensor with
// d channels, given its mode.  `row` indexes [B*H*T] (or [B*H] for decode).
template <bool BF16>
__device__ __forceinline__ float gate_at(const void *p, int mode, size_t row, int c, int d) {
  switch (mode) {
    case GDR_GATE_PER_CHANNEL: return ld1<BF16>(p, row * (size_t)d + c);
    case GDR_GATE_PER_TOKEN: return ld1<BF16>(p, row);
    case GDR_GATE_ONES: return 1.0f;
    default: return 0.0f;
  }
}

// Four consecutive channels c0..c0+3 of a gate (c0 multiple of 4).
template <bool BF16>
__device__ __forceinline__ void gate4(const void *p, int mode, size_t row, int c0, int d, float out[4]) {
  if (mode == GDR_GATE_PER_CHANNEL) {
    ld4<BF16>(p, row * (size_t)d + c0, out);
  } else {
    const float v = mode == GDR_GATE_PER_TOKEN ? ld1<BF16>(p, row) : (mode == GDR_GATE_ONES ? 1.0f : 0.0f);
    out[0] = out[1] = out[2] = out[3] = v;
  }
}

__device__ __forceinline__ void log_alpha4(const float *p, int mode, size_t row, int c0, int d, float out[4]) {
  if (mode == GDR_GATE_PER_CHANNEL) {
    float4 f = *reinterpret_cast<const float4 *>(p + row * (size_t)d + c0);
    out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
  } else {
    const float v = mode == GDR_GATE_PER_TOKEN ? p[row] : 0.0f;
    out[0] = out[1] = out[2] = out[3] = v;
  }
}

__device__ __forceinline__ float log_alpha_at(const float *p, int mode, size_t row, int c, int d) {
  switch (mode) {
    case GDR_GATE_PER_CHANNEL: return p[row * (size_t)d + c];
    case GDR_GATE_PER_TOKEN: return p[row];
    default: return 0.0f;
  }
}

// ---------------------------------------------------------------- branch-free gate loads
// Four raw storage elements (bf16 or fp32).
template <bool BF>
using Raw4 = typename std::conditional<BF, uint2, float4>::type;

// Element e (0..3, known at compile time) of a raw group.
template <bool BF>
__device__ __forceinline__ float raw_elem(const Raw4<BF> &r, int e) {
  if constexpr (BF) {
    const uint32_t w = (e < 2) ? r.x : r.y;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return e == 0 ? r.x : (e == 1 ? r.y : (e == 2 ? r.z : r.w));
  }
}

// Four gate values (channels c0..c0+3 of token row `row`) fetched without a
// branch whatever the gate mode -- a load under a branch makes the compiler
// wait for every load in flight where the paths join.  Two loads are always
// issued: the group of four channel values and the single token value; the
// one the mode does not use reads `any`, a valid 16-byte-aligned address.
//   per channel  p[row * d + c0 .. c0 + 3]
//   per token    p[row]
//   constant     neither (the value is a constant)
template <bool BF>
struct Gate4 {
  Raw4<BF> grp;
  float tok;
};
template <bool BF>
__device__ __forceinline__ Gate4<BF> gate_load(const void *p, int mode, size_t row, int c0, int d, const void *any) {
  const bool chan = mode == GDR_GATE_PER_CHANNEL, tokm = mode == GDR_GATE_PER_TOKEN;
  const char *gb = reinterpret_cast<const char *>(chan ? p : any);
  const char *tb = reinterpret_cast<const char *>(tokm ? p : any);
  Gate4<BF> g;
  g.grp = *reinterpret_cast<const Raw4<BF> *>(gb + (chan ? row * (size_t)d + c0 : 0) * (BF ? 2 : 4));
  g.tok = ld1<BF>(tb, tokm ? row : 0);
  return g;
}

// The 8 gate values of a lane's two 4-channel groups, zero where `ok` is
// false.  The mode is tested once for all 8 (uniform branches around plain
// moves), and `ok` is applied as a select afterwards, so no lane-divergent
// region encloses the mode test.
template <bool BF>
__device__ __forceinline__ void gate8(const Gate4<BF> g[2], int mode, float cval, bool ok, float out[8]) {
  if (mode == GDR_GATE_PER_CHANNEL) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = raw_elem<BF>(g[e / 4].grp, e % 4);
  } else if (mode == GDR_GATE_PER_TOKEN) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = g[e / 4].tok;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = cval;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = ok ? out[e] : 0.f;
}

// Value of the constant gate modes: ONES -> 1 (for log alpha: 0), ZEROS -> 0.
__device__ __forceinline__ float gate_const(int mode) { return mode == GDR_GATE_ONES ? 1.0f : 0.0f; }

// ---------------------------------------------------------------- buffer loads
// A raw buffer resource over [base, base + bytes) (gfx9 word 3: 32-bit data
// format).  Loads through it take the base from scalar registers and a
// 32-bit lane offset; offsets outside the range read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  static_assert(sizeof(T) == 16, "16-byte loads");
  return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

}  // namespace gdr
