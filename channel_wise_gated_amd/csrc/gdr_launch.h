// gdr_launch.h -- internal launch interface between the C ABI (gdr_abi.hip)
// and the kernel translation units.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

// Arguments of the two chunkwise kernels (device pointers; see gdr.h).
struct ChunkArgs {
  const void *q, *k, *v, *b, *w, *z;
  const float *log_alpha, *gamma, *S0;
  void *o;
  float *S_T;
  uint16_t *Qp, *Mm;  // workspace: A-fragment planes of Q' and M
  float *Ob, *Nn;     // workspace: accumulator tiles of O_bar and N
  uint16_t *Sc;       // workspace: chunk-start states as B-fragment planes
  int B, H, T, alpha_mode, b_mode, w_mode, normalize_qk;
  float scale;
};

hipError_t launch_decode(const gdr_desc &d, float *S, const void *q, const void *k, const void *v,
                         const float *la, const void *b, const void *w, const float *gamma,
                         const void *z, void *o, hipStream_t st);
// phases: bit 0 = intra-chunk kernel, bit 1 = scan kernel
hipError_t launch_chunk(const gdr_desc &d, const ChunkArgs &a, int phases, hipStream_t st);
size_t chunk_workspace_bytes(int B, int H, int T, int C, int D, int NS);
bool chunk_intra_fits(int C, int D, int NS);

}  // namespace gdr
