// gdr_abi.hip -- the extern "C" entry points of libgdr.so (declared in
// include/gdr.h): host-side validation, workspace carving and launches.
// Validation is pure host code and returns before any HIP call.
#include <stdint.h>

#include "gdr_launch.h"



namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int d) { return d == GDR_BF16 || d == GDR_F32; }

bool valid_mode(int m) { return m >= GDR_GATE_PER_CHANNEL && m <= GDR_GATE_ZEROS; }

bool needs_ptr(int m) { return m == GDR_GATE_PER_CHANNEL || m == GDR_GATE_PER_TOKEN; }

// Checks shared by both calls; `tokens` = T for chunk_fwd, 1 for decode.
gdr_status check_common(const gdr_desc *d, long long tokens) {
  if (!d) return GDR_ERR_INVALID_ARG;
  if (d->B < 0 || d->H < 0 || tokens < 0) return GDR_ERR_INVALID_ARG;
  if (d->dk <= 0 || d->dv <= 0) return GDR_ERR_INVALID_ARG;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return GDR_ERR_INVALID_ARG;
  if (!valid_mode(d->alpha_mode) || !valid_mode(d->b_mode) || !valid_mode(d->w_mode))
    return GDR_ERR_INVALID_ARG;
  if (d->alpha_mode == GDR_GATE_ZEROS) return GDR_ERR_INVALID_ARG;  // log alpha = -inf
  if (d->normalize_qk != 0 && d->normalize_qk != 1) return GDR_ERR_INVALID_ARG;
  if (!(d->scale == d->scale) || d->scale > 3.0e38f || d->scale < -3.0e38f) return GDR_ERR_INVALID_ARG;
  // element counts must stay addressable
  const long long elems = (long long)d->B * d->H * tokens * (d->dk > d->dv ? d->dk : d->dv);
  if (d->B > 0 && d->H > 0 && tokens > 0 && elems / d->B / d->H / tokens <= 0) return GDR_ERR_INVALID_ARG;
  if (elems > (1LL << 40)) return GDR_ERR_INVALID_ARG;
  if (d->dk != d->dv) return GDR_ERR_UNSUPPORTED;
  if (d->dk != 64 && d->dk != 128) return GDR_ERR_UNSUPPORTED;
  return GDR_OK;
}

gdr_status check_inputs(const gdr_desc *d, const void *q, const void *k, const void *v,
                        const float *la, const void *b, const void *w, const float *gamma,
                        const void *z, const void *o) {
  if (!q || !k || !v || !o) return GDR_ERR_INVALID_ARG;
  if (needs_ptr(d->alpha_mode) && !la) return GDR_ERR_INVALID_ARG;
  if (needs_ptr(d->b_mode) && !b) return GDR_ERR_INVALID_ARG;
  if (needs_ptr(d->w_mode) && !w) return GDR_ERR_INVALID_ARG;
  const void *ptrs[] = {q, k, v, o, needs_ptr(d->alpha_mode) ? la : nullptr,
                        needs_ptr(d->b_mode) ? b : nullptr, needs_ptr(d->w_mode) ? w : nullptr,
                        gamma, z};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_INVALID_ARG;
  return GDR_OK;
}

// nseq = 0: B sequences of T tokens; nseq > 0: a packed batch (B = 1).
gdr_status chunk_plan(const gdr_desc *d, int nseq, size_t *ws) {
  gdr_status s = check_common(d, d ? d->T : 0);
  if (s != GDR_OK) return s;
  if (d->chunk != 64 && d->chunk != 128) return GDR_ERR_INVALID_ARG;
  if (nseq < 0 || (nseq > 0 && d->B != 1)) return GDR_ERR_INVALID_ARG;
  const int ns = d->in_dtype == GDR_BF16 ? 2 : 3;
  if (!gdr::chunk_intra_fits(d->chunk, d->dk, ns)) return GDR_ERR_UNSUPPORTED;
  *ws = gdr::chunk_workspace(nullptr, nullptr, d->B, d->H, d->T, d->chunk, d->dk, ns, nseq);
  return GDR_OK;
}

// Validation and launch shared by the whole call (phases = 3), the
// intra-chunk phase (1: reads the token inputs, writes the workspace) and the
// scan phase (2: reads the workspace and S0, writes o and S_T).
// Output gate of the whole call: y = RMSNorm(o) * norm_w * sigmoid(g), token-major.
struct OutGate {
  const void *g;
  const float *norm_w;
  float eps;
  void *y;
  float *o;  // optional: o before the norm and gate (fp32)
};

// seg > 0: a whole call of a uniform batch in segments of `seg` chunks per
// stream, over a workspace laid out for that many chunks per stream.
gdr_status chunk_call(const gdr_desc *desc, int nseq, const int *cu, const void *q, const void *k,
                      const void *v, const float *log_alpha, const void *b, const void *w,
                      const float *gamma, const void *z, const float *S0, void *o, float *S_T,
                      void *workspace, size_t workspace_bytes, void *stream, int phases,
                      const OutGate *og = nullptr, int seg = 0) {
  size_t need = 0;
  gdr_status s = chunk_plan(desc, nseq, &need);
  if (s != GDR_OK) return s;
  const gdr_desc &d = *desc;
  const int ns_ = d.in_dtype == GDR_BF16 ? 2 : 3;
  const int t_layout = seg > 0 ? seg * d.chunk : d.T;  // tokens per stream the workspace is laid out for
  if (seg > 0) need = gdr::chunk_workspace(nullptr, nullptr, d.B, d.H, t_layout, d.chunk, d.dk, ns_, 0);
  const long long streams = nseq > 0 ? (long long)nseq * d.H : (long long)d.B * d.H;
  if (streams == 0) return GDR_OK;
  if (nseq > 0 && (!cu || (reinterpret_cast<uintptr_t>(cu) & 3u))) return GDR_ERR_INVALID_ARG;
  if (og) {  // gated output: y replaces o
    if (!og->g || !og->y || !aligned16(og->g) || !aligned16(og->y)) return GDR_ERR_INVALID_ARG;
    if (og->norm_w && !aligned16(og->norm_w)) return GDR_ERR_INVALID_ARG;
    if (og->o && !aligned16(og->o)) return GDR_ERR_INVALID_ARG;
    if (!(og->eps >= 0.f) || og->eps > 3.0e38f) return GDR_ERR_INVALID_ARG;
    o = og->y;
  }
  if (d.T > 0 && (phases & 1)) {
    s = check_inputs(desc, q, k, v, log_alpha, b, w, gamma, z, (phases & 2) ? o : q);
    if (s != GDR_OK) return s;
  }
  if (d.T > 0 && (phases & 2) && (!o || !aligned16(o))) return GDR_ERR_INVALID_ARG;
  if ((S0 && !aligned16(S0)) || (S_T && !aligned16(S_T))) return GDR_ERR_INVALID_ARG;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDR_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GDR_ERR_WORKSPACE;

  const int ns = d.in_dtype == GDR_BF16 ? 2 : 3;
  gdr::ChunkArgs a{};  // every field not set below is null / zero
  a.q = q; a.k = k; a.v = v; a.b = b; a.w = w; a.z = z;
  a.log_alpha = log_alpha; a.gamma = gamma; a.S0 = S0;
  a.o = o; a.S_T = S_T;
  a.Qp = a.Mm = a.Sc = nullptr; a.Ob = a.Nn = a.Sst = nullptr;
  gdr::chunk_workspace(&a, workspace, d.B, d.H, t_layout, d.chunk, d.dk, ns, nseq);
  a.B = nseq > 0 ? nseq : d.B; a.H = d.H; a.T = d.T;
  a.alpha_mode = d.alpha_mode; a.b_mode = d.b_mode; a.w_mode = d.w_mode;
  a.normalize_qk = d.normalize_qk; a.scale = d.scale;
  a.cu = nseq > 0 ? cu : nullptr;
  a.nseq = nseq;
  a.c0 = 0;  // the chunk range of each launch is set by launch_chunk
  a.ncs = 0;
  a.rev = 0;
  a.og = og ? og->g : nullptr;
  a.onw = og ? og->norm_w : nullptr;
  a.oeps = og ? og->eps : 0.f;
  a.y = og ? og->y : nullptr;
  a.oraw = og ? og->o : nullptr;
  if (nseq == 0) { a.ctab = nullptr; a.coff = nullptr; a.ctab_len = 0; }
  hipError_t e = gdr::launch_chunk(d, a, phases, static_cast<hipStream_t>(stream), seg);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

// Segment length of the allocation-free whole call: the library's regular
// choice when its workspace fits the static scratch, else the longest that
// fits; 0 when not even one chunk per stream fits.
int static_segment(const gdr_desc &d) {
  const int ns = d.in_dtype == GDR_BF16 ? 2 : 3;
  int seg = gdr::chunk_segment(d.B, d.H, d.T, d.chunk, d.dk, ns);
  while (seg > 0 &&
         gdr::chunk_workspace(nullptr, nullptr, d.B, d.H, seg * d.chunk, d.chunk, d.dk, ns, 0) > gdr::kStaticScratchBytes)
    --seg;
  return seg;
}

// The five-gate projection: validation, workspace size (the latent h).
gdr_status gate_plan(const gdr_gate_desc *d, size_t *ws, int *R) {
  if (!d) return GDR_ERR_INVALID_ARG;
  if (d->B < 0 || d->T < 0 || d->H <= 0 || d->d_model <= 0 || d->d_model % 32) return GDR_ERR_INVALID_ARG;
  if (!valid_dtype(d->out_dtype)) return GDR_ERR_INVALID_ARG;
  int r = 0;
  for (int i = 0; i < 5; ++i) {
    if (d->rank[i] <= 0 || d->rank[i] % 32) return GDR_ERR_INVALID_ARG;
    if (d->rank[i] > 128) return GDR_ERR_UNSUPPORTED;
    r += d->rank[i];
  }
  if (d->d != 64 && d->d != 128) return GDR_ERR_UNSUPPORTED;
  const long long N = (long long)d->B * d->T;
  if (N * d->H > (1LL << 31) - 1 || N * (long long)(d->d_model > r ? d->d_model : r) > (1LL << 40) ||
      N * (long long)d->H * d->d > (1LL << 40))
    return GDR_ERR_INVALID_ARG;
  *R = r;
  *ws = (size_t)N * r * sizeof(float);  // the latent h, fp32
  return GDR_OK;
}

// The backward: validation as the forward (its chunk size is its own, 64) and
// the workspace (the forward's chunk maps, the reverse chain's buffers and
// per-chunk scratch).
gdr_status bwd_plan(const gdr_desc *d, int nseq, size_t *ws) {
  if (!d) return GDR_ERR_INVALID_ARG;
  gdr_desc fd = *d;
  fd.chunk = 64;
  size_t fws = 0;
  gdr_status s = chunk_plan(&fd, nseq, &fws);  // also: nseq > 0 needs B = 1
  if (s != GDR_OK) return s;
  const int ns = d->in_dtype == GDR_BF16 ? 2 : 3;
  const long long nch = nseq > 0 ? (long long)d->H * ((d->T + 63) / 64 + nseq)
                                 : (long long)d->B * d->H * ((d->T + 63) / 64);
  if (nch > (1LL << 31) - 1) return GDR_ERR_INVALID_ARG;
  *ws = nch == 0 ? 0 : gdr::bwd_workspace(nullptr, nullptr, nullptr, d->B, d->H, d->T, d->dk, ns, nseq);
  return GDR_OK;
}

gdr_status bwd_call(const gdr_desc *desc, int nseq, const int *cu, const void *q, const void *k,
                    const void *v, const float *log_alpha, const void *b, const void *w, const float *gamma,
                    const void *z, const float *S0, const void *dO, const float *dS_T, float *dq, float *dk,
                    float *dv, float *dlog_alpha, float *db, float *dw, float *dgamma, float *dz, float *dS0,
                    void *workspace, size_t workspace_bytes, void *stream) {
  size_t need = 0;
  gdr_status s = bwd_plan(desc, nseq, &need);
  if (s != GDR_OK) return s;
  const gdr_desc &d = *desc;
  if ((long long)d.B * d.H == 0) return GDR_OK;
  if (nseq > 0 && (!cu || (reinterpret_cast<uintptr_t>(cu) & 3u))) return GDR_ERR_INVALID_ARG;
  if (d.T > 0) {
    s = check_inputs(desc, q, k, v, log_alpha, b, w, gamma, z, q);
    if (s != GDR_OK) return s;
    if (!dO || !aligned16(dO)) return GDR_ERR_INVALID_ARG;
  }
  const void *outs[] = {S0, dS_T, dq, dk, dv, dlog_alpha, db, dw, dgamma, dz, dS0};
  for (const void *p : outs)
    if (p && !aligned16(p)) return GDR_ERR_INVALID_ARG;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDR_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GDR_ERR_WORKSPACE;

  const int ns = d.in_dtype == GDR_BF16 ? 2 : 3;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  gdr_desc fd = d;
  fd.chunk = 64;
  gdr::ChunkArgs f{};  // every field not set below is null / zero
  f.q = q; f.k = k; f.v = v; f.b = b; f.w = w; f.z = z;
  f.log_alpha = log_alpha; f.gamma = gamma; f.S0 = S0;
  f.o = nullptr; f.S_T = nullptr;
  f.Qp = f.Mm = f.Sc = nullptr; f.Ob = f.Nn = f.Sst = nullptr;
  f.B = nseq > 0 ? nseq : d.B;  // chains: one per (sequence, head)
  f.H = d.H; f.T = d.T;
  f.alpha_mode = d.alpha_mode; f.b_mode = d.b_mode; f.w_mode = d.w_mode;
  f.normalize_qk = d.normalize_qk; f.scale = d.scale;
  f.cu = nseq > 0 ? cu : nullptr; f.coff = nullptr; f.ctab = nullptr; f.nseq = nseq; f.ctab_len = 0;
  f.c0 = 0; f.ncs = 0; f.rev = 0;
  f.og = nullptr; f.onw = nullptr; f.oeps = 0.f; f.y = nullptr; f.oraw = nullptr;
  gdr::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.b = b; a.w = w; a.z = z; a.dO = dO;
  a.log_alpha = log_alpha; a.gamma = gamma;
  a.B = d.B; a.H = d.H; a.T = d.T; a.NC = (d.T + 63) / 64;
  a.alpha_mode = d.alpha_mode; a.b_mode = d.b_mode; a.w_mode = d.w_mode;
  a.normalize_qk = d.normalize_qk; a.do_bf16 = d.out_dtype == GDR_BF16; a.scale = d.scale;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dla = dlog_alpha; a.db = db; a.dw = dw;
  a.dz = z ? dz : nullptr;
  a.dgamma = gamma ? dgamma : nullptr;
  a.ctab = nullptr; a.ctab_len = 0;
  // chunk slots: the token chunks of a uniform batch, or the (bounded) chunk
  // list of a packed one; none without tokens (then dS0 = dS_T, dgamma = 0)
  const bool chunks = d.T > 0 && (nseq > 0 || a.NC > 0);
  hipError_t e = hipSuccess;
  if (chunks) gdr::bwd_workspace(&a, &f, workspace, d.B, d.H, d.T, d.dk, ns, nseq);
  // the chain of chunk-end state gradients, last chunk to first (the final
  // one is dS0): the forward's chain kernel with M^T and Q'^T dO
  gdr::ChunkArgs r = f;
  r.Mm = chunks ? a.Mt : nullptr;
  r.Nn = chunks ? a.Gn : nullptr;
  r.Sc = chunks ? a.Xc : nullptr;
  r.S0 = dS_T;
  r.S_T = dS0;
  r.rev = 1;
  if (chunks) {
    a.Mm = f.Mm; a.Sc = f.Sc;
    // forward recompute: the chunk maps and M^T (a packed batch's chunk list
    // first), then Q'^T dO; then the forward chain (chunk-start states) and
    // the reverse chain side by side
    // the backward needs no O_bar (the intra kernel skips it) but the
    // per-token vectors and the chunk system's A and T^-1, which the same
    // kernel writes beside the maps
    gdr::ChunkArgs fi = f;
    fi.Ob = nullptr;
    fi.pp_kn = a.KN; fi.pp_kh = a.KH; fi.pp_qt = a.QT; fi.pp_vh = a.VH; fi.pp_lam = a.LAM;
    fi.pp_am = a.AM; fi.pp_ti = a.TI; fi.pp_mt = a.Mt;
    fi.pp_do = dO; fi.pp_do_bf16 = a.do_bf16; fi.pp_g = a.Gn;
    e = gdr::launch_chunk(fd, fi, 1, st);
    f.c0 = r.c0 = 0;
    f.ncs = r.ncs = a.NC;
    if (e == hipSuccess) e = gdr::launch_chain_pair(fd, f, r, st);
  } else if (dS0) {
    e = gdr::launch_chunk(fd, r, 4, st);
  }
  if (e == hipSuccess && (chunks || a.dgamma)) e = gdr::launch_bwd(a, d.dk, ns, st);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

// The output gate's backward: rows of the descriptor's streams; the weight's
// gradient through per-block partial sums in the workspace.
gdr_status og_bwd_plan(const gdr_desc *d, bool weight_grad, size_t *ws) {
  gdr_status s = check_common(d, d ? d->T : 0);
  if (s != GDR_OK) return s;
  const long long ntb = (d->T + 63) / 64;
  const long long blocks = (long long)d->B * d->H * ntb;
  if (blocks > (1LL << 31) - 1) return GDR_ERR_INVALID_ARG;
  *ws = weight_grad ? (size_t)((blocks * d->dv * 4 + 255) & ~255LL) : 0;
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_bwd_workspace_size(const gdr_desc *desc, size_t *bytes) {
  if (!bytes) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  gdr_status s = bwd_plan(desc, 0, &ws);
  if (s == GDR_OK) *bytes = ws;
  return s;
}

gdr_status gdr_chunk_bwd(const gdr_desc *desc, const void *q, const void *k, const void *v,
                         const float *log_alpha, const void *b, const void *w, const float *gamma,
                         const void *z, const float *S0, const void *dO, const float *dS_T, float *dq,
                         float *dk, float *dv, float *dlog_alpha, float *db, float *dw, float *dgamma,
                         float *dz, float *dS0, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_call(desc, 0, nullptr, q, k, v, log_alpha, b, w, gamma, z, S0, dO, dS_T, dq, dk, dv, dlog_alpha,
                  db, dw, dgamma, dz, dS0, workspace, workspace_bytes, stream);
}

gdr_status gdr_chunk_bwd_varlen_workspace_size(const gdr_desc *desc, int n_seqs, size_t *bytes) {
  if (!bytes || n_seqs < 1) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  gdr_status s = bwd_plan(desc, n_seqs, &ws);
  if (s == GDR_OK) *bytes = ws;
  return s;
}

gdr_status gdr_chunk_bwd_varlen(const gdr_desc *desc, int n_seqs, const int *cu_seqlens, const void *q,
                                const void *k, const void *v, const float *log_alpha, const void *b,
                                const void *w, const float *gamma, const void *z, const float *S0,
                                const void *dO, const float *dS_T, float *dq, float *dk, float *dv,
                                float *dlog_alpha, float *db, float *dw, float *dgamma, float *dz,
                                float *dS0, void *workspace, size_t workspace_bytes, void *stream) {
  if (n_seqs < 1) return GDR_ERR_INVALID_ARG;
  return bwd_call(desc, n_seqs, cu_seqlens, q, k, v, log_alpha, b, w, gamma, z, S0, dO, dS_T, dq, dk, dv,
                  dlog_alpha, db, dw, dgamma, dz, dS0, workspace, workspace_bytes, stream);
}

gdr_status gdr_output_gate_bwd_workspace_size(const gdr_desc *desc, int with_weight, size_t *bytes) {
  if (!bytes) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  gdr_status s = og_bwd_plan(desc, with_weight != 0, &ws);
  if (s == GDR_OK) *bytes = ws;
  return s;
}

gdr_status gdr_output_gate_bwd(const gdr_desc *desc, const float *o, const void *g, const float *norm_weight,
                               float eps, const void *dy, float *d_o, float *dg, float *d_norm_weight,
                               void *workspace, size_t workspace_bytes, void *stream) {
  const bool wgrad = norm_weight && d_norm_weight;
  size_t need = 0;
  gdr_status s = og_bwd_plan(desc, wgrad, &need);
  if (s != GDR_OK) return s;
  const gdr_desc &d = *desc;
  if (!(eps >= 0.f) || eps > 3.0e38f) return GDR_ERR_INVALID_ARG;
  if ((long long)d.B * d.H == 0) return GDR_OK;
  if (d.T > 0 && (!o || !g || !dy || !d_o)) return GDR_ERR_INVALID_ARG;
  const void *ptrs[] = {o, g, norm_weight, dy, d_o, dg, d_norm_weight};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_INVALID_ARG;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDR_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GDR_ERR_WORKSPACE;
  gdr::OgBwdArgs a;
  a.o = o; a.nw = norm_weight; a.g = g; a.dy = dy;
  a.dO = d_o; a.dg = dg; a.dnw = wgrad ? d_norm_weight : nullptr;
  a.part = wgrad ? static_cast<float *>(workspace) : nullptr;
  a.B = d.B; a.H = d.H; a.T = d.T; a.ntb = (d.T + 63) / 64;
  a.dy_bf16 = d.out_dtype == GDR_BF16; a.eps = eps;
  hipError_t e = gdr::launch_out_gate_bwd(a, d.dv, d.in_dtype == GDR_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

gdr_status gdr_gate_proj_workspace_size(const gdr_gate_desc *desc, size_t *bytes) {
  if (!bytes) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  int R = 0;
  gdr_status s = gate_plan(desc, &ws, &R);
  if (s == GDR_OK) *bytes = ws;
  return s;
}

gdr_status gdr_gate_proj(const gdr_gate_desc *desc, const void *x, const void *w_down,
                         const void *w_up, const float *bias, float *log_alpha, void *b,
                         void *g, void *w, void *z, void *workspace, size_t workspace_bytes,
                         void *stream) {
  size_t need = 0;
  int R = 0;
  gdr_status s = gate_plan(desc, &need, &R);
  if (s != GDR_OK) return s;
  const gdr_gate_desc &d = *desc;
  if ((long long)d.B * d.T == 0) return GDR_OK;
  if (!x || !w_down || !w_up) return GDR_ERR_INVALID_ARG;
  const void *ptrs[] = {x, w_down, w_up, bias, log_alpha, b, g, w, z};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_INVALID_ARG;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDR_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GDR_ERR_WORKSPACE;
  gdr::GateArgs a;
  a.x = static_cast<const uint16_t *>(x);
  a.wd = static_cast<const uint16_t *>(w_down);
  a.wu = static_cast<const uint16_t *>(w_up);
  a.bias = bias;
  a.hlat = static_cast<float *>(workspace);
  void *outs[5] = {log_alpha, b, g, w, z};
  a.N = d.B * d.T;
  a.T = d.T;
  a.dm = d.d_model;
  a.H = d.H;
  a.R = R;
  size_t wo = 0;
  int ro = 0;
  for (int i = 0; i < 5; ++i) {
    a.out[i] = outs[i];
    a.rank[i] = d.rank[i];
    a.roff[i] = ro;
    a.wuoff[i] = wo;
    ro += d.rank[i];
    wo += (size_t)d.H * d.d * d.rank[i];
  }
  hipError_t e = gdr::launch_gate_proj(a, d.d, d.out_dtype == GDR_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

gdr_status gdr_chunk_fwd_workspace_size(const gdr_desc *desc, size_t *bytes) {
  if (!bytes) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  gdr_status s = chunk_plan(desc, 0, &ws);
  if (s == GDR_OK) *bytes = ws;
  return s;
}

gdr_status gdr_chunk_fwd(const gdr_desc *desc, const void *q, const void *k, const void *v,
                         const float *log_alpha, const void *b, const void *w, const float *gamma,
                         const void *z, const float *S0, void *o, float *S_T, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return chunk_call(desc, 0, nullptr, q, k, v, log_alpha, b, w, gamma, z, S0, o, S_T, workspace,
                    workspace_bytes, stream, 3);
}

gdr_status gdr_chunk_fwd_static(const gdr_desc *desc, const void *q, const void *k, const void *v,
                                const float *log_alpha, const void *b, const void *w, const float *gamma,
                                const void *z, const float *S0, void *o, float *S_T, void *stream) {
  size_t ignored = 0;
  gdr_status s = chunk_plan(desc, 0, &ignored);
  if (s != GDR_OK) return s;
  if ((long long)desc->B * desc->H == 0) return GDR_OK;
  int seg = 1;
  if (desc->T > 0) {
    seg = static_segment(*desc);
    if (seg < 1) return GDR_ERR_UNSUPPORTED;  // B * H streams' segment state exceeds the static scratch
  }
  void *ws = nullptr;
  if (gdr::static_scratch(&ws) != hipSuccess) return GDR_ERR_HIP;
  return chunk_call(desc, 0, nullptr, q, k, v, log_alpha, b, w, gamma, z, S0, o, S_T, ws, gdr::kStaticScratchBytes,
                    stream, 3, nullptr, seg);
}

gdr_status gdr_chunk_fwd_gated(const gdr_desc *desc, const void *q, const void *k, const void *v,
                               const float *log_alpha, const void *b, const void *w,
                               const float *gamma, const void *z, const float *S0, const void *g,
                               const float *norm_weight, float eps, void *y, float *o, float *S_T,
                               void *workspace, size_t workspace_bytes, void *stream) {
  const OutGate og{g, norm_weight, eps, y, o};
  return chunk_call(desc, 0, nullptr, q, k, v, log_alpha, b, w, gamma, z, S0, nullptr, S_T, workspace,
                    workspace_bytes, stream, 3, &og);
}

gdr_status gdr_chunk_fwd_intra(const gdr_desc *desc, const void *q, const void *k, const void *v,
                               const float *log_alpha, const void *b, const void *w,
                               const float *gamma, const void *z, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return chunk_call(desc, 0, nullptr, q, k, v, log_alpha, b, w, gamma, z, nullptr, nullptr, nullptr,
                    workspace, workspace_bytes, stream, 1);
}

gdr_status gdr_chunk_fwd_scan(const gdr_desc *desc, const float *S0, void *o, float *S_T,
                              const void *workspace, size_t workspace_bytes, void *stream) {
  return chunk_call(desc, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, S0, o, S_T, const_cast<void *>(workspace), workspace_bytes, stream, 2);
}

gdr_status gdr_chunk_fwd_segment_chunks(const gdr_desc *desc, int *chunks) {
  if (!chunks) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  gdr_status s = chunk_plan(desc, 0, &ws);
  if (s != GDR_OK) return s;
  const int ns = desc->in_dtype == GDR_BF16 ? 2 : 3;
  *chunks = desc->T > 0 ? gdr::chunk_segment(desc->B, desc->H, desc->T, desc->chunk, desc->dk, ns) : 0;
  return GDR_OK;
}

gdr_status gdr_chunk_fwd_varlen_workspace_size(const gdr_desc *desc, int n_seqs, size_t *bytes) {
  if (!bytes || n_seqs < 1) return GDR_ERR_INVALID_ARG;
  size_t ws = 0;
  gdr_status s = chunk_plan(desc, n_seqs, &ws);
  if (s == GDR_OK) *bytes = ws;
  return s;
}

gdr_status gdr_chunk_fwd_varlen(const gdr_desc *desc, int n_seqs, const int *cu_seqlens,
                                const void *q, const void *k, const void *v,
                                const float *log_alpha, const void *b, const void *w,
                                const float *gamma, const void *z, const float *S0, void *o,
                                float *S_T, void *workspace, size_t workspace_bytes, void *stream) {
  if (n_seqs < 1) return GDR_ERR_INVALID_ARG;
  return chunk_call(desc, n_seqs, cu_seqlens, q, k, v, log_alpha, b, w, gamma, z, S0, o, S_T,
                    workspace, workspace_bytes, stream, 3);
}

gdr_status gdr_decode_step(const gdr_desc *desc, float *S, const void *q, const void *k,
                           const void *v, const float *log_alpha, const void *b, const void *w,
                           const float *gamma, const void *z, void *o, void *stream) {
  gdr_status s = check_common(desc, 1);
  if (s != GDR_OK) return s;
  const gdr_desc &d = *desc;
  if ((size_t)d.B * d.H == 0) return GDR_OK;
  if (!S || !aligned16(S)) return GDR_ERR_INVALID_ARG;
  s = check_inputs(desc, q, k, v, log_alpha, b, w, gamma, z, o);
  if (s != GDR_OK) return s;
  hipError_t e = gdr::launch_decode(d, S, q, k, v, log_alpha, b, w, gamma, z, o,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

gdr_status gdr_check_inputs(const gdr_desc *desc, const void *q, const void *k, const void *v,
                            const float *log_alpha, const void *b, const void *w, const float *gamma,
                            const void *z, unsigned long long *counts, void *stream) {
  gdr_status s = check_common(desc, desc ? desc->T : 0);
  if (s != GDR_OK) return s;
  if (!counts || reinterpret_cast<uintptr_t>(counts) % 8) return GDR_ERR_INVALID_ARG;
  const gdr_desc &d = *desc;
  const unsigned long long rows = (unsigned long long)d.B * d.H * d.T;
  if (rows > 0) {
    s = check_inputs(desc, q, k, v, log_alpha, b, w, gamma, z, q);  // no output: q stands in for o
    if (s != GDR_OK) return s;
  }
  if (gamma && !aligned16(gamma)) return GDR_ERR_INVALID_ARG;  // read even without tokens
  const int bf = d.in_dtype == GDR_BF16;
  auto gate_n = [&](gdr_gate_mode m, int dim) {
    return m == GDR_GATE_PER_CHANNEL ? rows * dim : m == GDR_GATE_PER_TOKEN ? rows : 0ull;
  };
  auto gate_p = [&](gdr_gate_mode m, const void *p) { return needs_ptr(m) && rows > 0 ? p : nullptr; };
  const gdr::CheckTensor t[gdr::kCheckCounts] = {
      {rows > 0 ? q : nullptr, rows * d.dk, bf, 0},
      {rows > 0 ? k : nullptr, rows * d.dk, bf, 0},
      {rows > 0 ? v : nullptr, rows * d.dv, bf, 0},
      {gate_p(d.alpha_mode, log_alpha), gate_n(d.alpha_mode, d.dk), 0, 1},
      {gate_p(d.b_mode, b), gate_n(d.b_mode, d.dk), bf, 0},
      {gate_p(d.w_mode, w), gate_n(d.w_mode, d.dv), bf, 0},
      {rows > 0 ? z : nullptr, rows * d.dk, bf, 0},
      {gamma, (unsigned long long)d.H * d.dk, 0, 0}};
  hipError_t e = gdr::launch_check(t, counts, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

const char *gdr_status_string(gdr_status status) {
  switch (status) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG: invalid argument";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED: configuration not supported";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case GDR_ERR_HIP: return "GDR_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown gdr_status";
  }
}

int gdr_version(void) { return 100; }

}  // extern "C"
