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
  float *Ob, *Nn;     // workspace: accumulator tiles of O_bar^T and N (intra-chunk
                      // kernel alone: Ob null skips O_bar, which only the output kernel reads)
  uint16_t *Sc;       // workspace: chunk-start states as B-fragment planes
  int B, H, T, alpha_mode, b_mode, w_mode, normalize_qk;
  float scale;
  // Packed variable-length batch (all null / 0 otherwise): B = 1, T = total
  // tokens, sequence n holds packed rows cu[n] .. cu[n+1]-1.  Chunk slot
  // g = j * H + h holds chunk j of the per-head chunk list ctab (entries
  // {sequence, chunk of the sequence, first packed row, valid tokens}, or
  // sequence -1 past the end); coff[n] is the first entry of sequence n.
  const int *cu;
  int *coff;
  int4 *ctab;
  int nseq, ctab_len;
  // Uniform batches: this launch covers chunks c0 .. c0 + ncs - 1 of every
  // stream; stream bh's chunk c sits in slot bh * ncs + (c - c0).
  int c0, ncs;
  float *Sst;  // workspace: fp32 states handed from one segment to the next
  // Chain only: walk each stream's chunks last to first (the backward's chain
  // of state gradients, X <- M^T X + G, with M^T and G in the M and N slots).
  int rev;
  // Gated output (og != null): instead of o, y[b,t,h,:] = RMSNorm(o[b,h,t,:])
  // * onw[h,:] * sigmoid(og[b,h,t,:]) in token-major [B,T,H,dv].
  const void *og;
  const float *onw;
  float oeps;
  float *oraw;  // gated output only: o itself as well ([B,H,T,dv] fp32), or null
  void *y;
  // Intra-chunk kernel at C = 64 for the backward (all null otherwise): the
  // per-token vectors kn, k_hat, q_tilde, v_hat and the in-chunk cumulative
  // log decay, [slot][C][D] fp32 each, zero on padding rows.
  float *pp_kn, *pp_kh, *pp_qt, *pp_vh, *pp_lam;
  // ... and the chunk system's A (diagonal included) and T^-1, [slot][C][C]
  // fp32 each, zero above the diagonal and on padding rows and columns of A;
  // and M^T as NS bf16 planes in M's A-fragment layout ([slot][NS][D][D]; not
  // written for an empty slot of a packed batch).
  float *pp_am, *pp_ti;
  uint16_t *pp_mt;
  // ... and G = Q'^T dO for the reverse chain, in N's accumulator-tile layout
  // ([slot][D][D] fp32), from dO ([B,H,T,dv] rows as q's, bf16 when
  // pp_do_bf16, else fp32); Q' itself is then not written.
  const void *pp_do;
  int pp_do_bf16;
  float *pp_g;
};

// The five-gate projection: x [N, dm] bf16 (N = B*T tokens), wd [R, dm]
// bf16, wu the gates' [H*d, rank] bf16 blocks at element offsets wuoff, bias
// [5, H*d] fp32 or null; hlat [N, R] fp32 workspace; out[gate] (gate order f,
// b, g, w, q) head-major [B, H, T, d] or null (not computed).
struct GateArgs {
  const uint16_t *x, *wd, *wu;
  const float *bias;
  float *hlat;  // [N][R] fp32 latent
  void *out[5];
  int N, T, dm, H, R;
  int rank[5], roff[5];
  size_t wuoff[5];
};
hipError_t launch_gate_proj(const GateArgs &a, int d, bool out_bf16, hipStream_t st);

// Backward pass (gdr_bwd.hip): chunks of 64 tokens, uniform or packed batches.
struct BwdArgs {
  const void *q, *k, *v, *b, *w, *z, *dO;
  const float *log_alpha, *gamma;
  int B, H, T, NC, alpha_mode, b_mode, w_mode, normalize_qk, do_bf16;
  float scale;
  const uint16_t *Mm, *Sc;       // the forward's M and chunk-start states (C = 64)
  uint16_t *Mt, *Xc;             // M^T for the reverse chain; the chunk-end state gradients
  float *Gn;                     // Q'^T dO for the reverse chain
  // per-chunk scratch, [slot][64][D] fp32
  float *KN, *KH, *QT, *VH, *LAM, *DU, *DQA, *DKA, *DKP;
  float *AM, *TI, *DA, *DL;      // [slot][64][64] fp32
  float *gpart;                  // [slot][D] partial sums of dgamma
  float *XS;                     // [slot][D] row dots sum_j X_ij S0_ij of each chunk's end-state gradient and start state
  const int4 *ctab;              // packed batch: the forward's chunk list (null for uniform batches)
  int ctab_len;
  float *dq, *dk, *dv, *dla, *db, *dw, *dz, *dgamma;  // outputs (each may be null)
};
// Workspace of the backward: the forward's chunk workspace (C = 64; its fields
// set in *f) followed by the backward's regions (set in *a); returns the size.
size_t bwd_workspace(BwdArgs *a, ChunkArgs *f, void *ws, int B, int H, int T, int D, int NS, int nseq);
hipError_t launch_bwd(const BwdArgs &a, int D, int NS, hipStream_t st);

// Backward of the fused output gate (gdr_bwd.hip): rows of [B,H,T,dv] in
// workgroups of 64 tokens; `part` holds [B][ntb][H][dv] partial sums of the
// norm weight's gradient (null without a weight).
struct OgBwdArgs {
  const float *o, *nw;
  const void *g, *dy;
  float *dO, *dg, *dnw, *part;
  int B, H, T, ntb, dy_bf16;
  float eps;
};
hipError_t launch_out_gate_bwd(const OgBwdArgs &a, int D, bool g_bf16, hipStream_t st);

// The opt-in precondition check (gdr_check.hip): per tensor its pointer (null:
// not checked), element count, storage (bf16 or fp32) and whether the
// log-decay range applies; counts[i] gets the number of elements of tensor i
// that break the preconditions (zeroed first, on the stream).
struct CheckTensor {
  const void *p;
  unsigned long long n;
  int bf16, range;
};
constexpr int kCheckCounts = 8;
hipError_t launch_check(const CheckTensor (&t)[kCheckCounts], unsigned long long *counts, hipStream_t st);

hipError_t launch_decode(const gdr_desc &d, float *S, const void *q, const void *k, const void *v,
                         const float *la, const void *b, const void *w, const float *gamma,
                         const void *z, void *o, hipStream_t st);
// phases: bit 0 = intra-chunk kernel, bit 1 = scan (chain + output kernels),
// bit 2 = chain kernel only (no output).  seg > 0 (whole calls of uniform
// batches only): segments of exactly `seg` chunks per stream, the workspace
// laid out for B*H*seg chunk slots (chunk_workspace with T = seg * C); 0: the
// library's own segment choice over a workspace for every chunk.
hipError_t launch_chunk(const gdr_desc &d, const ChunkArgs &a, int phases, hipStream_t st, int seg = 0);
// Chunks per stream in one segment of a whole call, as the library chooses it.
int chunk_segment(int B, int H, int T, int C, int D, int NS);
// The static scratch of the allocation-free whole call: its size, and the
// device address of the current device's copy (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void **ptr);
// Two independent chains (the chain kernel only) over uniform batches at C = 64
// in one launch; each ChunkArgs with c0 = 0 and ncs = its chunks per stream.
hipError_t launch_chain_pair(const gdr_desc &d, const ChunkArgs &a, const ChunkArgs &b, hipStream_t st);
// Workspace of the chunkwise forward: per chunk slot the maps Q', M, O_bar,
// N and the chunk-start state; for a packed batch (nseq > 0) the chunk list
// and sequence offsets, otherwise (T > 0) the fp32 states [B,H,D,D] handed
// between segments.  Slots: B*H*ceil(T/C), or H * (ceil(T/C) + nseq)
// for a packed batch (each sequence adds at most one short chunk).  Returns
// the size in bytes; with `ws` set, also points the fields of *a into it.
size_t chunk_workspace(ChunkArgs *a, void *ws, int B, int H, int T, int C, int D, int NS, int nseq);
bool chunk_intra_fits(int C, int D, int NS);

}  // namespace gdr
