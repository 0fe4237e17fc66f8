/*
 * libxattn: causal multi-head / grouped-query scaled-dot-product attention with a
 * per-head QK-RMSNorm + rotate_half RoPE prologue, forward and backward, for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes (page titles and sections):
 *   [T9]   xtrain "Phase T9: Export to xserv": conventions table (RMSNorm with no mean
 *          subtraction, per-head QK-norm with one gamma[head_dim] per tensor, rotate_half
 *          RoPE with frequency theta^(-2i/hd) and position = token index, scale
 *          1/sqrt(head_dim), causal mask) and Decision 1 (QK-norm after the head reshape,
 *          before RoPE).
 *   [MINT] Mint documentation, sections 5.3.1 (score, causal mask, stable softmax,
 *          weighted sum), 5.4.1-5.4.4 (RoPE rotation, angle, backward = rotation by the
 *          negative angle, positions restart at 0 per sequence, cached frequencies),
 *          5.5.1-5.5.2 (RMSNorm forward and backward, dgamma accumulated across rows).
 *   [T15]  xtrain "Phase T15: GQA": layouts [batch*heads, S, hd] for Q and
 *          [batch*num_kv_heads, S, hd] for K/V; query head qh reads KV head qh/group;
 *          num_heads % num_kv_heads == 0; the K/V gradient of a shared head is the
 *          deterministic sum of its group's query-head gradients, with no atomics.
 *   [MINT] (continued) 10.3 (KV cache: append in place, attention of the new token over
 *          every cached key, equal to full-sequence attention), 14.2 item 5 (fused
 *          single-token GPU decode), 8.2 (block-causal mask of a flattened batch: no
 *          attention across samples, causal inside a sample).
 *   [T12]  xtrain "Phase T12: bf16 mixed precision", precision table: bf16 activations
 *          with fp32 accumulation; softmax, norm and RoPE computed in fp32; fp32 master
 *          weights (gamma) and gradients.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers to contiguous row-major tensors owned by the caller,
 *     16-byte aligned.  Outputs are overwritten, never accumulated into, and must not
 *     alias inputs.  The library never allocates or frees device memory; scratch comes
 *     from a caller-provided workspace sized by the matching *_workspace_bytes query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work and
 *     return; results are valid once the caller synchronises the stream.
 *   - io dtype: XATTN_F32 (fp32 everywhere) or XATTN_BF16 (bf16 tensors, fp32
 *     arithmetic inside, fp32 lse / rstd / gamma / dgamma).
 *   - Errors: every argument is validated before any device work; an invalid call
 *     returns a status and has no side effects.  Kernel-launch failures are reported
 *     as XATTN_ERR_HIP (the HIP error is peeked, not cleared).  Faults inside kernels
 *     surface at the caller's next synchronisation.  No call aborts the process or lets
 *     a C++ exception escape.  xattn_last_error() gives a thread-local message.
 *   - Inputs are assumed finite; non-finite inputs propagate, results unspecified.
 *   - Supported head_dim: 16, 32, 64, 128.  seq_len >= 1.  Every tensor's element count
 *     must stay below 2^31.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { XATTN_F32 = 0, XATTN_BF16 = 1 } xattn_dtype;

typedef enum {
  XATTN_OK = 0,
  XATTN_ERR_INVALID_ARG = 1,  /* null pointer, size <= 0, H % Hkv != 0, odd head_dim,
                                 misaligned pointer, element count >= 2^31, bad dtype */
  XATTN_ERR_UNSUPPORTED = 2,  /* a valid shape this build does not run: head_dim not in
                                 {16, 32, 64, 128}, or a decode call beyond its row limit */
  XATTN_ERR_HIP = 3           /* a kernel launch reported a HIP error */
} xattn_status;

/* Shape of one attention call ([T15] layouts). */
typedef struct {
  int64_t batch;         /* B */
  int64_t seq_len;       /* S: query and key length (square causal self-attention) */
  int64_t num_heads;     /* H: query heads */
  int64_t num_kv_heads;  /* Hkv: K/V heads; H % Hkv == 0, group = H / Hkv */
  int64_t head_dim;      /* hd */
  int32_t dtype;         /* xattn_dtype of q, k, v, out, dout, dq, dk, dv */
  /* Packed documents ([MINT] 8.2, block-causal mask): NULL and NULL for plain causal
   * attention over each batch row; otherwise device int32 arrays [seq_len] giving, for
   * every row, the first (seg_lo) and last (seg_hi) row of the document it belongs to,
   * the same packing for every batch row.  Row i then attends to keys
   * seg_lo[i] <= j <= i only.  Documents are contiguous (both arrays non-decreasing,
   * seg_lo[i] <= i <= seg_hi[i]); xattn_segments builds them from document offsets.
   * Other contents give unspecified values but no access outside the tensors. */
  const int32_t* seg_lo;
  const int32_t* seg_hi;
} xattn_dims;

/* Prologue inputs that let xattn_bwd also run the QK-norm + RoPE backward, so that
 * dq / dk come out with respect to the raw (pre-norm) projections. */
typedef struct {
  const void* xq;          /* [B*H, S, hd] io dtype: raw Q before QK-norm */
  const void* xk;          /* [B*Hkv, S, hd] io dtype: raw K before QK-norm */
  const float* gamma_q;    /* [hd] fp32 */
  const float* gamma_k;    /* [hd] fp32 */
  const float* rstd_q;     /* [B*H*S] fp32, as written by xattn_qknorm_rope_fwd */
  const float* rstd_k;     /* [B*Hkv*S] fp32 */
  const float* cos_tab;    /* [S, hd/2] fp32, from xattn_rope_cache */
  const float* sin_tab;    /* [S, hd/2] fp32 */
  float* dgamma_q;         /* [hd] fp32 output (overwritten) */
  float* dgamma_k;         /* [hd] fp32 output (overwritten) */
} xattn_prologue;

/* RoPE cos/sin table ([MINT] 5.4.2 and 5.4.4, [T9] "cos/sin cache"):
 *   angle(t, i) = t * theta^(-2i/head_dim), t in [0, seq_len), i in [0, head_dim/2),
 * evaluated in fp64 on the device and rounded once to fp32.
 * cos_tab, sin_tab: [seq_len, head_dim/2] fp32 outputs. */
xattn_status xattn_rope_cache(float* cos_tab, float* sin_tab, int64_t seq_len,
                              int64_t head_dim, double theta, void* stream);

/* Packed documents ([MINT] 8.2; 5.4.4: positions restart in every sequence): from the
 * document offsets cu_seqlens[0] = 0 < cu_seqlens[1] < ... < cu_seqlens[ndocs] = seq_len
 * (device int32 [ndocs + 1]) writes, for every row r in [0, seq_len), seg_lo[r] and
 * seg_hi[r] (first and last row of r's document, as xattn_dims takes them) and, when
 * positions is not NULL, positions[r] = r - seg_lo[r] (its position in its document, for
 * xattn_rope_cache_at).  Outputs: device int32 [seq_len]. */
xattn_status xattn_segments(const int32_t* cu_seqlens, int32_t ndocs, int64_t seq_len,
                            int32_t* seg_lo, int32_t* seg_hi, int32_t* positions, void* stream);

/* RoPE table at explicit positions: row r of cos_tab / sin_tab ([rows, head_dim/2] fp32)
 * holds the angles of position positions[r] (device int32 [rows]), evaluated like
 * xattn_rope_cache.  With packed documents, positions from xattn_segments give the
 * per-row table the prologue calls take (row t of the table for row t of the sequence). */
xattn_status xattn_rope_cache_at(float* cos_tab, float* sin_tab, const int32_t* positions,
                                 int64_t rows, int64_t head_dim, double theta, void* stream);

/* Prologue forward ([T9] Decision 1, [MINT] 5.4.1 and 5.5.1), per row x in R^hd of a
 * [rows, seq_len, hd] tensor (rows = B*H for Q or B*Hkv for K), row position t = s:
 *   rstd = 1 / sqrt(mean(x^2) + eps);  n = gamma * x * rstd;
 *   y[i] = n[i] cos - n[i+hd/2] sin;  y[i+hd/2] = n[i] sin + n[i+hd/2] cos.
 * x, y: io dtype [rows, S, hd]; gamma: fp32 [hd]; cos/sin: fp32 [S, hd/2];
 * rstd: fp32 [rows*S] output (kept for the backward). */
xattn_status xattn_qknorm_rope_fwd(const void* x, const float* gamma, const float* cos_tab,
                                   const float* sin_tab, void* y, float* rstd, int64_t rows,
                                   int64_t seq_len, int64_t head_dim, float eps,
                                   int32_t dtype, void* stream);

/* Prologue forward with the RoPE table built in the same launch ([T9] "cos/sin cache",
 * [MINT] 5.4.2, 5.4.4, 5.4.1 and 5.5.1): writes cos_tab / sin_tab ([seq_len, hd/2] fp32)
 * exactly as xattn_rope_cache(seq_len, hd, theta) does (positions == NULL) or as
 * xattn_rope_cache_at(positions, seq_len rows) does (positions: device int32 [seq_len]), and
 * y, rstd exactly as xattn_qknorm_rope_fwd with that table: bitwise the results of the two
 * calls, in one launch (the table's fp64 evaluation runs under the rows' loads).  Arguments
 * as in those two calls; the table is an output here and must not overlap x, gamma, y,
 * rstd or positions. */
xattn_status xattn_qknorm_rope_fwd_table(const void* x, const float* gamma,
                                         const int32_t* positions, double theta,
                                         float* cos_tab, float* sin_tab, void* y, float* rstd,
                                         int64_t rows, int64_t seq_len, int64_t head_dim,
                                         float eps, int32_t dtype, void* stream);

/* Bytes of workspace xattn_qknorm_rope_bwd needs (per-block dgamma partials). */
size_t xattn_qknorm_rope_bwd_workspace_bytes(int64_t rows, int64_t seq_len, int64_t head_dim);

/* Prologue backward ([MINT] 5.4.4 and 5.5.2): dn = rotation of dy by the negative angle;
 *   dot = sum(gamma * dn * x);  dx = gamma * dn * rstd - x * dot * rstd^3 / hd;
 *   dgamma = sum over all rows*S rows of dn * x * rstd, reduced in a fixed order
 *   (bitwise reproducible run to run).
 * dy, x, dx: io dtype [rows, S, hd]; rstd: fp32 [rows*S]; dgamma: fp32 [hd] output. */
xattn_status xattn_qknorm_rope_bwd(const void* dy, const void* x, const float* gamma,
                                   const float* rstd, const float* cos_tab,
                                   const float* sin_tab, void* dx, float* dgamma,
                                   void* workspace, size_t workspace_bytes, int64_t rows,
                                   int64_t seq_len, int64_t head_dim, int32_t dtype,
                                   void* stream);

/* Attention forward ([MINT] 5.3.1, [T9] scale and causal mask, [T15] head mapping):
 * for batch b, query head qh (kv head kvh = qh / group), query i and key j <= i:
 *   s_ij = q_i . k_j / sqrt(hd);  p_ij = softmax_j(s_ij) (fp32, max-subtracted);
 *   out_i = sum_j p_ij v_j;  lse_i = ln(sum_{j<=i} exp(s_ij)).
 * q, out: [B*H, S, hd] io dtype; k, v: [B*Hkv, S, hd] io dtype; lse: [B*H*S] fp32 output.
 * For bf16 the probabilities are rounded to bf16 before the P.V product. */
xattn_status xattn_fwd(const xattn_dims* dims, const void* q, const void* k, const void* v,
                       void* out, float* lse, void* stream);

/* Q side of the prologue, for xattn_fwd_qnorm. */
typedef struct {
  const void* xq;          /* [B*H, S, hd] io dtype: raw Q before QK-norm */
  const float* gamma_q;    /* [hd] fp32 */
  const float* cos_tab;    /* [S, hd/2] fp32, from xattn_rope_cache */
  const float* sin_tab;    /* [S, hd/2] fp32 */
  float eps;               /* finite, >= 0 */
  void* yq;                /* [B*H, S, hd] io dtype output: normalised, rotated Q */
  float* rstd_q;           /* [B*H*S] fp32 output */
} xattn_fwd_prologue;

/* Attention forward with the Q side of the prologue fused ([T9] Decision 1, [MINT] 5.4.1,
 * 5.4.4, 5.5.1 and 5.3.1): the same results as xattn_qknorm_rope_fwd(pro->xq) into
 * pro->yq / pro->rstd_q followed by xattn_fwd(pro->yq, k, v), in one pass: the attention
 * reads the raw Q rows it keeps resident and normalises and rotates them itself (yq and
 * rstd_q are still written, as xattn_bwd needs them; bitwise the rows xattn_qknorm_rope_fwd
 * gives, except bf16 at hd 64 / 128: within one rounding of them, the mean square being
 * summed in another order).  k must already be normalised and rotated
 * (xattn_qknorm_rope_fwd): every query tile reads every K tile before it, so K is
 * prepared once.  out, lse as in xattn_fwd. */
xattn_status xattn_fwd_qnorm(const xattn_dims* dims, const xattn_fwd_prologue* pro,
                             const void* k, const void* v, void* out, float* lse,
                             void* stream);

/* Bytes of workspace xattn_bwd needs; with_prologue != 0 sizes it for a call with a
 * non-NULL xattn_prologue. */
size_t xattn_bwd_workspace_bytes(const xattn_dims* dims, int with_prologue);

/* Attention backward: the chain rule of xattn_fwd.  With D_i = sum_d dout_id out_id,
 *   dP_ij = dout_i . v_j;  dS_ij = p_ij (dP_ij - D_i);
 *   dq_i = sum_j dS_ij k_j / sqrt(hd);
 *   dk_j = sum_{r<group} sum_{i>=j} dS^(r)_ij q^(r)_i / sqrt(hd);
 *   dv_j = sum_{r<group} sum_{i>=j} p^(r)_ij dout^(r)_i,
 * where r runs over the query heads kvh*group + r sharing the KV head ([T15] Decision 2).
 * Each dk/dv element has a single owner that sums its group in a fixed order: no
 * atomics, bitwise reproducible run to run (dq, too).
 * pro == NULL: dq, dk are gradients w.r.t. the q, k that xattn_fwd consumed.
 * pro != NULL: the prologue backward runs too; dq, dk are then gradients w.r.t. the raw
 * pro->xq, pro->xk and pro->dgamma_q / dgamma_k are written (the arithmetic of
 * xattn_qknorm_rope_bwd; dgamma summed in a fixed order, bitwise reproducible).  For bf16
 * io it is applied inside the dq and dk stores (the gradients w.r.t. the rotated q, k never
 * reach memory), except at hd 16 / 32 for shapes so small that the dk/dv pass spreads a
 * group's query heads over several workgroups; there, and for fp32, it is a separate pass
 * over fp32 gradients.
 * q, out, dout, dq: [B*H, S, hd]; k, v, dk, dv: [B*Hkv, S, hd]; lse: [B*H*S] fp32 from
 * xattn_fwd.  workspace: device memory of at least xattn_bwd_workspace_bytes bytes. */
xattn_status xattn_bwd(const xattn_dims* dims, const void* q, const void* k, const void* v,
                       const void* out, const float* lse, const void* dout, void* dq,
                       void* dk, void* dv, const xattn_prologue* pro, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Attention backward with no allocation and no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as xattn_bwd (bitwise: the same kernels),
 * but the scratch is a static device array of XATTN_BWD_NOALLOC_SCRATCH_BYTES that each GPU
 * holds until the process ends; its address is looked up on the first call with that GPU
 * current.  A shape whose xattn_bwd_workspace_bytes exceeds that size is rejected with
 * XATTN_ERR_UNSUPPORTED: 16 MiB holds, with the prologue, about 900 thousand query rows
 * (B*H*S) of bf16 MHA at head_dim 64 (6.4 MiB for B=32, S=1024, 12 heads) and about 60
 * thousand of fp32.  Every call on one GPU shares its array, and the array keeps the
 * last call's contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU (different streams or threads) race and must be serialised by the caller. */
#define XATTN_BWD_NOALLOC_SCRATCH_BYTES (16u << 20)
xattn_status xattn_bwd_noalloc(const xattn_dims* dims, const void* q, const void* k,
                               const void* v, const void* out, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv,
                               const xattn_prologue* pro, void* stream);

/* ---- Projections around attention --------------------------------------------------------
 * [MINT] 5.3.1-5.3.2: Q = X Wq + bq, K = X Wk + bk, V = X Wv + bv, output
 * Concat(heads) Wo + bo, with weights [d_in, d_out] applied as x @ W; [T5] layout pipeline:
 * the projections' token rows are split into heads ([B*H, S, hd], [B*Hkv, S, hd], what the
 * prologue and attention take) and the attention output is merged back into token rows
 * before Wo; [T12]: GEMMs take the io dtype with fp32 accumulation, the weight and bias
 * gradients are fp32.  Token rows: x, y, dx [B*S, d], row b*S + s.  The GEMMs are the
 * library's own kernels (bf16: MFMA), with the head split, bias and rounding in their
 * epilogues, and (bf16, hd and S multiples of 64) the head-major tensors read in place
 * instead of merged into a copy; weight gradients are summed in a fixed order (bitwise
 * reproducible).
 * Requires d % 8 == 0 and every operand below 2^31 bytes.  The segment fields of dims are
 * ignored. */
typedef struct {
  int64_t model_dim;  /* d */
  const void* wq;     /* [d, H*hd] io dtype */
  const void* wk;     /* [d, Hkv*hd] io dtype */
  const void* wv;     /* [d, Hkv*hd] io dtype */
  const void* wo;     /* [H*hd, d] io dtype */
  const float* bq;    /* NULL (no bias) or fp32 [H*hd] */
  const float* bk;    /* NULL or fp32 [Hkv*hd] */
  const float* bv;    /* NULL or fp32 [Hkv*hd] */
  const float* bo;    /* NULL or fp32 [d] */
} xattn_proj;

/* Bytes of workspace each projection call below needs (one size serves all four). */
size_t xattn_proj_workspace_bytes(const xattn_dims* dims, int64_t model_dim);

/* xq, xk, v (head layouts, io dtype) = split_heads(x Wq + bq), ... (only wq, wk, wv and
 * their biases are read). */
xattn_status xattn_qkv_proj_fwd(const xattn_dims* dims, const xattn_proj* p, const void* x,
                                void* xq, void* xk, void* v, void* workspace,
                                size_t workspace_bytes, void* stream);

/* y [B*S, d] = merge_heads(out) Wo + bo; out: [B*H, S, hd]. */
xattn_status xattn_out_proj_fwd(const xattn_dims* dims, const xattn_proj* p, const void* out,
                                void* y, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Chain rule of xattn_out_proj_fwd for the upstream gradient dy [B*S, d]:
 *   dout = split_heads(dy Wo^T) [B*H, S, hd] (io dtype); dwo = merge_heads(out)^T dy
 *   [H*hd, d] fp32; dbo = column sums of dy [d] fp32 (NULL: not computed). */
xattn_status xattn_out_proj_bwd(const xattn_dims* dims, const xattn_proj* p, const void* out,
                                const void* dy, void* dout, float* dwo, float* dbo,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Chain rule of xattn_qkv_proj_fwd for the gradients dxq, dxk, dv (head layouts):
 *   dx = merge(dxq) Wq^T + merge(dxk) Wk^T + merge(dv) Wv^T [B*S, d] (io dtype, summed in
 *   fp32 before one rounding); dwq = x^T merge(dxq) [d, H*hd] fp32, dwk, dwv likewise;
 *   dbq, dbk, dbv = column sums of the merged gradients (fp32, each NULL: not computed).
 *   Column sums are taken in a fixed order (bitwise reproducible). */
xattn_status xattn_qkv_proj_bwd(const xattn_dims* dims, const xattn_proj* p, const void* x,
                                const void* dxq, const void* dxk, const void* dv, void* dx,
                                float* dwq, float* dwk, float* dwv, float* dbq, float* dbk,
                                float* dbv, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- KV-cache decode ---------------------------------------------------------------------
 * Shape of a decode call: each of `batch` sequences has cache_len tokens cached and adds
 * q_len new ones at positions cache_len .. cache_len + q_len - 1. */
typedef struct {
  int32_t batch;
  int32_t num_heads;     /* query heads H */
  int32_t num_kv_heads;  /* Hkv; H % Hkv == 0 */
  int32_t head_dim;      /* 16, 32, 64 or 128 */
  int32_t dtype;         /* xattn_dtype of xq, xk, v, the caches and out */
  int32_t q_len;         /* new tokens per sequence, >= 1 */
  int32_t cache_len;     /* tokens already in the cache per sequence, >= 0 */
  int32_t capacity;      /* cache rows per (sequence, KV head); cache_len + q_len <= capacity */
} xattn_decode_dims;

/* Bytes of workspace xattn_decode needs.  It depends on capacity, not on cache_len, so one
 * workspace serves every step of a cache; 0 for invalid dims. */
size_t xattn_decode_workspace_bytes(const xattn_decode_dims* dims);

/* KV-cache decode step ([MINT] 10.3 "KV cache": the new tokens' K/V are appended to the
 * cache in place and their queries attend to every cached key; equal to full-sequence
 * attention; [MINT] 14.2 item 5: RoPE, append and attention fused instead of per-head
 * launches).  For new token i of sequence b at position t = cache_len + i:
 *   q_t, k_t = QK-norm + RoPE of xq, xk at position t (as xattn_qknorm_rope_fwd);
 *   k_cache, v_cache row t of KV head (b, kvh) <- k_t, v;
 *   out_t = sum_{j <= t} softmax_j(q_t . k_j / sqrt(hd)) v_j over that KV head's cache rows,
 *   lse_t = ln sum_{j <= t} exp(q_t . k_j / sqrt(hd)),
 * for every query head qh of the group kvh = qh / (H / Hkv).
 * xq: [B*H, q_len, hd]; xk, v: [B*Hkv, q_len, hd] (raw, io dtype); gamma_q, gamma_k: [hd];
 * cos_tab, sin_tab: [capacity, hd/2] from xattn_rope_cache(capacity); k_cache, v_cache:
 * [B*Hkv, capacity, hd] io dtype, rows [0, cache_len) hold the previous tokens' rotated keys
 * and values (read), rows [cache_len, cache_len + q_len) are written, the rest untouched;
 * out: [B*H, q_len, hd]; lse: [B*H*q_len] fp32.  Any (H / Hkv) * q_len: the query rows of
 * a KV head are handled in chunks (16 rows for fp32 io and for bf16 with hd 64 / 128, 8 for
 * bf16 with hd 16 / 32) that each stream the cache.  bf16 io rounds the rotated queries and
 * the softmax probabilities to bf16 before the products (fp32 accumulation), as the training
 * forward does.  The key ranges are summed in a fixed order: bitwise reproducible run to
 * run. */
xattn_status xattn_decode(const xattn_decode_dims* dims, const void* xq, const void* xk,
                          const void* v, const float* gamma_q, const float* gamma_k,
                          const float* cos_tab, const float* sin_tab, float eps, void* k_cache,
                          void* v_cache, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/* KV-cache decode with one cache length per sequence ([MINT] 10.3 for each sequence): as
 * xattn_decode, except that sequence b has cache_lens[b] tokens cached (device int32
 * [batch]) and its new tokens sit at positions cache_lens[b] + i (RoPE angle, cache rows
 * written, causal limit).  dims->cache_len must be the largest cache_lens[b] (it sizes the
 * key ranges, and the workspace query does not depend on it).  Each cache_lens[b] is clamped
 * into [0, capacity - q_len] on the device: a length outside it, or above dims->cache_len,
 * gives wrong results but no access outside the tensors.  cache_lens is read-only and must
 * not overlap the outputs. */
xattn_status xattn_decode_varlen(const xattn_decode_dims* dims, const int32_t* cache_lens,
                                 const void* xq, const void* xk, const void* v,
                                 const float* gamma_q, const float* gamma_k,
                                 const float* cos_tab, const float* sin_tab, float eps,
                                 void* k_cache, void* v_cache, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ---- Instrumentation (no effect on results) ---------------------------------------------
 * Per-kernel timing with HIP events: between xattn_profile_start and xattn_profile_stop,
 * every kernel the library launches is bracketed by two events recorded on its launch
 * stream (process-wide, all threads).  xattn_profile_stop waits for those events, turns
 * timing off and writes, in first-launch order, one entry per kernel name: the number of
 * launches and their summed elapsed milliseconds.  Up to max_entries entries are written;
 * *n_entries receives the number of distinct kernels.  Timing adds a few microseconds per
 * launch while on and costs nothing measurable while off. */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} xattn_kernel_time;

xattn_status xattn_profile_start(void);
xattn_status xattn_profile_stop(xattn_kernel_time* entries, int32_t max_entries,
                                int32_t* n_entries);

/* Static description of a status code; any integer is accepted (values that are not an
 * xattn_status give "unknown xattn_status"). */
const char* xattn_status_string(int32_t status);

/* Thread-local message describing the last failing call on this thread ("" if none). */
const char* xattn_last_error(void);

/* Library version string. */
const char* xattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
