/*
 * gdr.h -- C ABI of libgdr.so: the channel-wise gated delta rule on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (Muir reading notes, arXiv:2611.08376, section 2.1 "GDN-2 state
 * update and Muir read-out"; pre-pass from the "Kimi3 = GPT2 x 22580" blog,
 * section 3 "DeltaNet", forward()).  For every independent stream (b, h) the
 * state S in R^{dk x dv} (fp32, rows = key channels) evolves token by token:
 *
 *   qh  = SiLU(q_t) / max(|SiLU(q_t)|_2, 1e-12)      (skipped if !normalize_qk)
 *   kn  = SiLU(k_t) / max(|SiLU(k_t)|_2, 1e-12)      (skipped if !normalize_qk)
 *   qt  = scale * gamma (.) 2 sigmoid(z_t) (.) qh     read-out gain on the query
 *   S_hat = Diag(alpha_t) S_{t-1},  alpha_t = exp(log_alpha_t) in (0, 1]
 *   u   = w_t (.) v_t - (b_t (.) kn) S_hat            erase key b (.) k, write w (.) v
 *   S_t = S_hat + kn^T u
 *   o_t = qt S_t                                       read after the write
 *
 * With b = w = beta this is Kimi Delta Attention, with a scalar alpha Gated
 * DeltaNet, with alpha = 1 DeltaNet, with b = 0 gated linear attention.  The
 * notes drop the display equation of the update; the form above is the one
 * under which their chunk system T Z = [V_hat, K_hat decayed],
 * T = I + L_strict (section 2.4, "Boundary-Pivoted Chunkwise Kernel") holds.
 *
 * Calls
 *   gdr_chunk_fwd     whole sequences [B, H, T] at once, chunkwise (prefill /
 *                     training forward); S0 -> S_T
 *   gdr_decode_step   one token per (sequence, head); state updated in place
 *
 * Conventions common to every call
 *   - Tensors are device pointers owned by the caller, contiguous, row-major,
 *     head-major:  q, k, z, log_alpha, b (per channel): [B, H, T, dk];
 *     v, w (per channel), o: [B, H, T, dv]; per-token gates: [B, H, T];
 *     gamma: [H, dk]; states: [B, H, dk, dv] fp32.  For decode T = 1.
 *   - Every pointer that is read must be 16-byte aligned.
 *   - q, k, v, b, w, z share the storage dtype desc->in_dtype; log_alpha,
 *     gamma and states are always fp32; o has desc->out_dtype.
 *   - Calls are asynchronous on `stream` (a hipStream_t; 0 = the null
 *     stream).  The library never synchronises and allocates no device
 *     memory; chunk_fwd takes its scratch from a caller workspace whose size
 *     gdr_chunk_fwd_workspace_size() reports.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed validation returns its status and has no side effect.  A launch
 *     failure returns GDR_ERR_HIP.  No C++ exception crosses this ABI.
 *   - Inputs must not alias outputs, except S_T == S0 in gdr_chunk_fwd and
 *     the in-place state of gdr_decode_step.
 *   - Preconditions not checked on the hot path: log_alpha finite and in
 *     [-30, 0]; b, w, z, gamma finite.  A NaN in one (b, h) stream stays in
 *     that stream.
 *   - fp32 inputs (in_dtype = GDR_F32) select the fp32-accurate arithmetic
 *     (three-term bf16 splits on the matrix cores, relative error ~1e-6);
 *     bf16 inputs select two-term splits (~1e-5).  State, log-decay and all
 *     accumulation are fp32 in both.
 *   - The library keeps no mutable global state, so concurrent calls from
 *     several threads or streams are safe; the one exception is
 *     gdr_chunk_fwd_static, whose scratch array is shared by every call on
 *     a GPU.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size or enum      */
  GDR_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. dk not 64/128)   */
  GDR_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
  GDR_ERR_HIP = 4          /* a HIP launch or runtime call failed              */
} gdr_status;

typedef enum gdr_dtype { GDR_BF16 = 0, GDR_F32 = 1 } gdr_dtype;

/* How a gate argument is given. */
typedef enum gdr_gate_mode {
  GDR_GATE_PER_CHANNEL = 0, /* full tensor [B, H, T, d]                          */
  GDR_GATE_PER_TOKEN = 1,   /* scalar per token [B, H, T], broadcast over d      */
  GDR_GATE_ONES = 2,        /* pointer ignored; value 1 (for alpha: log_alpha 0) */
  GDR_GATE_ZEROS = 3        /* pointer ignored; value 0 (b only: linear attention) */
} gdr_gate_mode;

typedef struct gdr_desc {
  int B;                    /* batch (decode: number of sequences)            */
  int H;                    /* heads                                           */
  int T;                    /* tokens per sequence (ignored by decode, = 1)    */
  int dk;                   /* key channels: 64 or 128                         */
  int dv;                   /* value channels: must equal dk                   */
  int chunk;                /* chunk size of gdr_chunk_fwd: 64 or 128 (any T;  */
                            /* the last chunk of a sequence may be short)      */
  gdr_dtype in_dtype;       /* storage of q, k, v, b, w, z                     */
  gdr_dtype out_dtype;      /* storage of o                                    */
  int normalize_qk;         /* 1: SiLU + L2 pre-pass on q, k; 0: used as given */
  float scale;              /* query scale (1.0: no 1/sqrt(d))                 */
  gdr_gate_mode alpha_mode; /* PER_CHANNEL, PER_TOKEN or ONES                  */
  gdr_gate_mode b_mode;     /* PER_CHANNEL, PER_TOKEN, ONES or ZEROS           */
  gdr_gate_mode w_mode;     /* PER_CHANNEL, PER_TOKEN or ONES                  */
} gdr_desc;

/*
 * Bytes of device workspace gdr_chunk_fwd needs for `desc` (validated as for
 * gdr_chunk_fwd).  Written to *bytes on success.
 */
gdr_status gdr_chunk_fwd_workspace_size(const gdr_desc *desc, size_t *bytes);

/*
 * Chunkwise forward of whole sequences (Muir notes section 2.4; the blog's
 * section 4 chunk form): per chunk of `desc->chunk` tokens, an intra-chunk
 * kernel builds the decayed key Gram matrix and read-out scores with
 * boundary pivots (every decay factor exp(Lambda_t - Lambda_s) is formed from
 * exponents <= 0), inverts the unit-lower-triangular matrix T of the chunk
 * system T Z = [V_hat, K_hat e^Lambda], and reduces the chunk to an affine map
 * of the state; a scan kernel then carries S in fp32 across chunks and writes
 * o.  A long uniform batch is processed in segments of chunks (the state
 * handed from one segment to the next in fp32, so the result is the same), so
 * that the workspace a segment's kernels pass to each other stays in the
 * GPU's last-level cache.
 *
 *   q, k      [B,H,T,dk] in_dtype        v     [B,H,T,dv] in_dtype
 *   log_alpha per alpha_mode, fp32       b, w  per b_mode / w_mode, in_dtype
 *   gamma     [H,dk] fp32 or NULL (= 1)  z     [B,H,T,dk] in_dtype or NULL (2 sigma = 1)
 *   S0        [B,H,dk,dv] fp32 or NULL (= 0)
 *   o         [B,H,T,dv] out_dtype (written)
 *   S_T       [B,H,dk,dv] fp32 or NULL (written; may alias S0)
 *   workspace >= gdr_chunk_fwd_workspace_size() bytes, 256-byte aligned,
 *             contents undefined on entry and on return.
 */
gdr_status gdr_chunk_fwd(const gdr_desc *desc, const void *q, const void *k,
                         const void *v, const float *log_alpha, const void *b,
                         const void *w, const float *gamma, const void *z,
                         const float *S0, void *o, float *S_T, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Chunks per (batch, head) stream in one segment of gdr_chunk_fwd on a
 * uniform batch: the whole call runs the intra-chunk, chain and output
 * kernels over that many chunks of every stream at a time (each launch of
 * the intra-chunk and output kernels covers B * H * chunks chunks), handing
 * the fp32 state from one segment to the next, so that the chunk maps the
 * kernels exchange stay in the GPU's last-level cache (Muir notes section 2.4
 * computes the same chunk maps; the segmenting is this library's).  Equal to
 * ceil(T / chunk) when the call runs in one pass.  Validation as
 * gdr_chunk_fwd_workspace_size; written to *chunks (0 when T = 0).
 */
gdr_status gdr_chunk_fwd_segment_chunks(const gdr_desc *desc, int *chunks);

/*
 * gdr_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, hosts that forbid allocation.  Same
 * arguments, results and validation as gdr_chunk_fwd on a uniform batch,
 * without the workspace: the scratch is a static array of the library
 * (64 MiB per GPU, held by every GPU the library runs on until the process
 * ends), and the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  The long-context path runs in segments of chunks sized
 * to fit that array; the results equal gdr_chunk_fwd's, bit for bit.
 *   Limit: B * H streams' maps for one chunk each, plus their fp32 handoff
 *   states, must fit the array (about 170 streams at dk = dv = 128 and chunk
 *   128, 230 at chunk 64); a larger problem returns GDR_ERR_UNSUPPORTED
 *   before any launch.
 *   Every call on a GPU uses that GPU's one copy of the array: calls that
 *   overlap in time on one GPU (other streams, other threads) race and give
 *   undefined results; calls ordered on one stream are safe.  No state
 *   carries over from one call to the next (nothing needs clearing).
 */
gdr_status gdr_chunk_fwd_static(const gdr_desc *desc, const void *q, const void *k,
                                const void *v, const float *log_alpha, const void *b,
                                const void *w, const float *gamma, const void *z,
                                const float *S0, void *o, float *S_T, void *stream);

/*
 * The five gates from one shared low-rank projection of the layer input
 * (Muir reading notes, section 2.3: a shared down-projection, then per gate
 * an up-projection and a channel bias give the logits of the decay f, erase
 * b, output gate g, write w and query gain q, with ranks
 * (r_f, r_b, r_g, r_w, r_q); the main model uses (64, 64, 128, 128, 128)).
 *   h        = x W_down^T                              [N, R], R = sum of ranks
 *   l_gate   = h[:, ranks of the gate] W_up_gate^T + bias_gate   [N, H*d]
 * The pages print neither the formula nor the activations; this library
 * reads them as follows (ranges from section 2.1):
 *   log_alpha = log sigmoid(l_f)  (alpha in (0,1); fp32)
 *   b = 2 sigmoid(l_b) in (0,2),  w = sigmoid(l_w) in (0,1)
 *   g = l_g  (gdr_chunk_fwd_gated applies the sigmoid)
 *   z = l_q  (the read-out applies 2 sigmoid(z))
 * Output channel j = h*d + c of token (b, t) is written at [b, h, t, c], the
 * layout gdr_chunk_fwd reads (per-channel gate modes).
 */
typedef struct gdr_gate_desc {
  int B, T;         /* tokens; x is [B, T, d_model]                            */
  int d_model;      /* input width: a positive multiple of 32                  */
  int H, d;         /* outputs [B, H, T, d]; d = 64 or 128                     */
  int rank[5];      /* (r_f, r_b, r_g, r_w, r_q): multiples of 32, 32..128     */
  gdr_dtype out_dtype; /* storage of b, w, g, z (log_alpha is always fp32)     */
} gdr_gate_desc;

/* Bytes of device workspace gdr_gate_proj needs: the latent h, fp32
 * [B*T, R]. */
gdr_status gdr_gate_proj_workspace_size(const gdr_gate_desc *desc, size_t *bytes);

/*
 *   x          [B, T, d_model] bf16
 *   w_down     [R, d_model] bf16 (rows in gate order f, b, g, w, q)
 *   w_up       the gates' [H*d, r_gate] bf16 matrices, back to back in gate order
 *   bias       [5, H*d] fp32 in gate order, or NULL (= 0)
 *   log_alpha  [B, H, T, d] fp32;  b, g, w, z [B, H, T, d] out_dtype -- each
 *              output may be NULL, and that gate is then not computed
 *   workspace  >= gdr_gate_proj_workspace_size() bytes, 256-byte aligned
 * Every pointer 16-byte aligned.  Invalid sizes (including B*T*H >= 2^31),
 * null required pointers or misalignment: GDR_ERR_INVALID_ARG; a rank above
 * 128 or d not 64 / 128: GDR_ERR_UNSUPPORTED; all checked on the host before
 * any launch.
 */
gdr_status gdr_gate_proj(const gdr_gate_desc *desc, const void *x, const void *w_down,
                         const void *w_up, const float *bias, float *log_alpha, void *b,
                         void *g, void *w, void *z, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * gdr_chunk_fwd with the layer's output gate fused into the output kernel
 * (Muir reading notes, section 2.1: after a per-head RMSNorm the output gate
 * g_t modulates every channel).  Instead of o, it writes
 *   y[b,t,h,c] = o[b,h,t,c] / sqrt(mean_c' o[b,h,t,c']^2 + eps)
 *                * norm_weight[h,c] * sigmoid(g[b,h,t,c])
 * in token-major layout, ready for the output projection; o is not
 * materialised.  The pages name neither the gate's activation nor the norm's
 * epsilon: sigmoid (a gate in (0,1), like w) and a caller-given eps are this
 * library's reading.
 *
 *   arguments as gdr_chunk_fwd, except:
 *   g            [B,H,T,dv] in_dtype: output-gate logits
 *   norm_weight  [H,dv] fp32 RMSNorm weight, or NULL (= 1)
 *   eps          >= 0, finite (added to the mean square)
 *   y            [B,T,H,dv] out_dtype (written)
 *   o            [B,H,T,dv] fp32 or NULL: when given, o itself (before the
 *                norm and the gate) is written too, for gdr_output_gate_bwd
 * Validation as gdr_chunk_fwd, plus: g and y non-null and 16-byte aligned,
 * eps finite and >= 0 (GDR_ERR_INVALID_ARG).
 */
gdr_status gdr_chunk_fwd_gated(const gdr_desc *desc, const void *q, const void *k,
                               const void *v, const float *log_alpha, const void *b,
                               const void *w, const float *gamma, const void *z,
                               const float *S0, const void *g, const float *norm_weight,
                               float eps, void *y, float *o, float *S_T, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Backward of gdr_chunk_fwd: the gradients of the loss <dO, o> + <dS_T, S_T>
 * with respect to every input (reverse mode of the recurrence of Muir reading
 * notes, section 2.1, through the chunk system of section 2.4: a chain of
 * state gradients over the chunks, last to first, X <- M^T X + Q'^T dO, then
 * per chunk the gradients of its tokens).  It recomputes what it needs of the
 * forward pass, in chunks of 64 tokens whatever desc->chunk says.
 *
 *   arguments q .. S0 and desc as gdr_chunk_fwd (uniform batches)
 *   dO          [B,H,T,dv] in desc->out_dtype: the upstream gradient of o
 *   dS_T        [B,H,dk,dv] fp32 or NULL (= 0): the upstream gradient of S_T
 *   outputs, all fp32, each may be NULL (not written):
 *     dq, dk    [B,H,T,dk];  dv [B,H,T,dv];  dz [B,H,T,dk] (only with z)
 *     dlog_alpha, db, dw  shaped as their gate: [B,H,T,d] per channel,
 *                         [B,H,T] per token; not written for ONES / ZEROS
 *     dgamma    [H,dk] (only with gamma; summed over batch and tokens)
 *     dS0       [B,H,dk,dv]
 *   workspace   >= gdr_chunk_bwd_workspace_size() bytes, 256-byte aligned
 * Validation as gdr_chunk_fwd, plus dO non-null and every pointer 16-byte
 * aligned (GDR_ERR_INVALID_ARG), before any launch.
 */
gdr_status gdr_chunk_bwd_workspace_size(const gdr_desc *desc, size_t *bytes);
gdr_status gdr_chunk_bwd(const gdr_desc *desc, const void *q, const void *k, const void *v,
                         const float *log_alpha, const void *b, const void *w, const float *gamma,
                         const void *z, const float *S0, const void *dO, const float *dS_T,
                         float *dq, float *dk, float *dv, float *dlog_alpha, float *db, float *dw,
                         float *dgamma, float *dz, float *dS0, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Backward of the output gate of gdr_chunk_fwd_gated (Muir reading notes,
 * section 2.1: per-head RMSNorm of o, then the output gate g per channel; the
 * library's reading y = o / sqrt(mean_c o^2 + eps) * norm_weight *
 * sigmoid(g)).  For the loss <dy, y> it returns the gradients of o, g and
 * norm_weight, so that a layer's backward can run this, then gdr_chunk_bwd
 * with d_o as its dO.
 *
 *   desc        B, H, T, dk = dv (64 or 128); in_dtype is g's dtype, out_dtype
 *               dy's dtype (the rest of the descriptor is not used)
 *   o           [B,H,T,dv] fp32: the recurrence's output (gdr_chunk_fwd's o)
 *   g           [B,H,T,dv] in_dtype: the gate logits
 *   norm_weight [H,dv] fp32 or NULL (= 1);  eps >= 0, finite
 *   dy          [B,T,H,dv] out_dtype (token-major, as y)
 *   d_o         [B,H,T,dv] fp32 (written)
 *   dg          [B,H,T,dv] fp32 or NULL (not written)
 *   d_norm_weight [H,dv] fp32 or NULL; written only with norm_weight (summed
 *               over batch and tokens)
 *   workspace   >= gdr_output_gate_bwd_workspace_size(desc, with_weight)
 *               bytes (with_weight: norm_weight and d_norm_weight both given),
 *               256-byte aligned; 0 bytes without the weight's gradient
 * Errors: dimensions and dtypes as gdr_chunk_fwd; null o, g, dy or d_o (with
 * T > 0), misaligned pointers or a bad eps: GDR_ERR_INVALID_ARG; workspace:
 * GDR_ERR_WORKSPACE; all on the host before any launch.
 */
gdr_status gdr_output_gate_bwd_workspace_size(const gdr_desc *desc, int with_weight, size_t *bytes);
gdr_status gdr_output_gate_bwd(const gdr_desc *desc, const float *o, const void *g,
                               const float *norm_weight, float eps, const void *dy, float *d_o,
                               float *dg, float *d_norm_weight, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Backward of gdr_chunk_fwd_varlen: the gradients of a packed batch of n_seqs
 * sequences (each with its own S0 and S_T), the reverse of the recurrence of
 * gdr_chunk_bwd run per sequence and head.  Layouts as gdr_chunk_fwd_varlen:
 * desc->B must be 1 and desc->T = cu_seqlens[n_seqs]; every per-token tensor
 * (inputs, dO and the per-token gradients) is [1,H,T,...] over the packed
 * tokens; S0, dS_T and dS0 are [n_seqs,H,dk,dv]; dgamma [H,dk] sums over all
 * sequences.  cu_seqlens (device, int32, n_seqs + 1 non-decreasing offsets from
 * 0) is read on the device; sequences of length 0 pass dS_T to dS0.
 *   workspace  >= gdr_chunk_bwd_varlen_workspace_size(desc, n_seqs) bytes,
 *              256-byte aligned
 * Validation as gdr_chunk_bwd, plus n_seqs >= 1, desc->B == 1 and cu_seqlens
 * non-null and 4-byte aligned (GDR_ERR_INVALID_ARG); the offsets themselves
 * are the caller's contract, read as gdr_chunk_fwd_varlen reads them.
 */
gdr_status gdr_chunk_bwd_varlen_workspace_size(const gdr_desc *desc, int n_seqs, size_t *bytes);
gdr_status gdr_chunk_bwd_varlen(const gdr_desc *desc, int n_seqs, const int *cu_seqlens,
                                const void *q, const void *k, const void *v,
                                const float *log_alpha, const void *b, const void *w,
                                const float *gamma, const void *z, const float *S0,
                                const void *dO, const float *dS_T, float *dq, float *dk,
                                float *dv, float *dlog_alpha, float *db, float *dw,
                                float *dgamma, float *dz, float *dS0, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * The two phases of gdr_chunk_fwd as separate calls, for callers that overlap
 * the fully parallel phase of one batch with the serial scan of another on a
 * second stream, or that time the phases.  gdr_chunk_fwd(...) gives exactly
 * the results of gdr_chunk_fwd_intra(...) followed by gdr_chunk_fwd_scan(...)
 * on the same stream with the same descriptor and workspace (these two are
 * not segmented: the workspace holds every chunk between them).
 *
 * gdr_chunk_fwd_intra: reads the token inputs (arguments as gdr_chunk_fwd)
 *   and writes, per chunk, the chunk's affine state map into the workspace:
 *   Q' = Qt e^Lambda - A Y, O_bar = A U_bar, M = Diag(e^Lambda_C) - K'^T Y,
 *   N = K'^T U_bar (Muir notes section 2.4: the chunk system solved once per
 *   chunk, outputs and next state by matrix products).
 * gdr_chunk_fwd_scan: reads that workspace and S0, carries the fp32 state
 *   through the chunks (O = Q' S + O_bar, S <- M S + N) and writes o and S_T.
 *   The workspace must hold the intra phase's results for the same inputs.
 */
gdr_status gdr_chunk_fwd_intra(const gdr_desc *desc, const void *q, const void *k,
                               const void *v, const float *log_alpha, const void *b,
                               const void *w, const float *gamma, const void *z,
                               void *workspace, size_t workspace_bytes, void *stream);

gdr_status gdr_chunk_fwd_scan(const gdr_desc *desc, const float *S0, void *o, float *S_T,
                              const void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunkwise forward of a packed batch of n_seqs sequences of different
 * lengths: every sequence and head runs the recurrence of gdr_chunk_fwd from
 * its own S0 (Muir notes section 2.4 chunk form; the blog's forward(x, cache)
 * per sequence).  The token axis of every per-token tensor is the
 * concatenation of the sequences: sequence n holds packed tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1, and its chunks start at its first token.
 *
 *   desc->B     must be 1; desc->T = total packed tokens = cu_seqlens[n_seqs]
 *   cu_seqlens  device int32 [n_seqs + 1]: cu_seqlens[0] = 0, nondecreasing,
 *               last = desc->T; a sequence may be empty.  A precondition:
 *               offsets that break it give undefined results, but the device
 *               clamps every offset to [0, T] and each sequence's end to no
 *               less than its start, and writes no chunk entry past the
 *               workspace's list, so they cause no access out of bounds
 *   q, k, v, log_alpha, b, w, z, o   as gdr_chunk_fwd with B = 1 (packed)
 *   gamma       [H,dk] fp32 or NULL
 *   S0, S_T     [n_seqs,H,dk,dv] fp32 or NULL; S_T may alias S0
 *   workspace   >= gdr_chunk_fwd_varlen_workspace_size(desc, n_seqs) bytes,
 *               256-byte aligned, contents undefined on entry and on return.
 * Errors as gdr_chunk_fwd; GDR_ERR_INVALID_ARG also for desc->B != 1,
 * n_seqs < 1, or a null or misaligned cu_seqlens.
 */
gdr_status gdr_chunk_fwd_varlen_workspace_size(const gdr_desc *desc, int n_seqs, size_t *bytes);

gdr_status gdr_chunk_fwd_varlen(const gdr_desc *desc, int n_seqs, const int *cu_seqlens,
                                const void *q, const void *k, const void *v,
                                const float *log_alpha, const void *b, const void *w,
                                const float *gamma, const void *z, const float *S0, void *o,
                                float *S_T, void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step for B sequences x H heads (the blog's section 3 forward()
 * with a one-token x and `cache` = S): reads S once, forms
 * u = v_hat - k_hat (Diag(alpha) S), writes S <- Diag(alpha) S + kn^T u in
 * place and o = qt S.  desc->T and desc->chunk are ignored.
 *
 *   S         [B,H,dk,dv] fp32, updated in place
 *   q, k, z   [B,H,dk] in_dtype (z may be NULL)    v [B,H,dv] in_dtype
 *   log_alpha [B,H,dk] or [B,H] fp32 per alpha_mode
 *   b, w      [B,H,d] or [B,H] per mode             gamma [H,dk] fp32 or NULL
 *   o         [B,H,dv] out_dtype (written)
 */
gdr_status gdr_decode_step(const gdr_desc *desc, float *S, const void *q,
                           const void *k, const void *v, const float *log_alpha,
                           const void *b, const void *w, const float *gamma,
                           const void *z, void *o, void *stream);

/*
 * Opt-in precondition check of the token inputs of a call with this
 * descriptor (gdr_chunk_fwd's layout; for decode pass T = 1).  The update
 * above decays the state by alpha_t = exp(log_alpha_t) in (0, 1] and the
 * chunk kernels' pivoted decay factors are sized for log_alpha >= -30; no
 * entry point looks for a violation on its hot path.  This call counts, on
 * the device, the elements that break the preconditions:
 *
 *   counts[GDR_CHECK_Q], [_K], [_V], [_B], [_W], [_Z], [_GAMMA]: NaN or +-inf
 *   counts[GDR_CHECK_LOG_ALPHA]: NaN, +-inf, > 0 or < -30
 *
 * Tensors follow desc (in_dtype, gate modes; a gate in mode ONES or ZEROS,
 * a NULL z or gamma is not read and counts 0).  counts: device memory, 8-byte
 * aligned, GDR_CHECK_COUNT unsigned 64-bit counters, zeroed and then written
 * on `stream` (read them once the stream's work is done).  Errors: as
 * gdr_chunk_fwd's validation (GDR_ERR_INVALID_ARG for a null desc or
 * counts, a null required input or a misaligned pointer), checked on the
 * host before any launch; GDR_ERR_HIP on a launch failure.
 */
enum {
  GDR_CHECK_Q = 0,
  GDR_CHECK_K = 1,
  GDR_CHECK_V = 2,
  GDR_CHECK_LOG_ALPHA = 3,
  GDR_CHECK_B = 4,
  GDR_CHECK_W = 5,
  GDR_CHECK_Z = 6,
  GDR_CHECK_GAMMA = 7,
  GDR_CHECK_COUNT = 8
};
gdr_status gdr_check_inputs(const gdr_desc *desc, const void *q, const void *k,
                            const void *v, const float *log_alpha, const void *b,
                            const void *w, const float *gamma, const void *z,
                            unsigned long long *counts, void *stream);

/* Static, human-readable name of a status code. */
const char *gdr_status_string(gdr_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
