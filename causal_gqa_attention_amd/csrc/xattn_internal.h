// Internal launcher interface between the C-ABI layer (xattn_api.cpp) and the HIP
// kernels.  All arguments have been validated by the caller: sizes are positive,
// element counts fit in int32, pointers are non-null and 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xattn {

enum IoType { IO_F32 = 0, IO_BF16 = 1 };

// Sets the calling thread's message returned by xattn_last_error().
void set_last_error(const char* msg);

// ---- prologue ------------------------------------------------------------------------
hipError_t launch_rope_cache(float* cos_tab, float* sin_tab, int seq_len, int head_dim,
                             double theta, hipStream_t stream);
// Table rows at explicit positions: row r holds the angles of position positions[r].
hipError_t launch_rope_cache_at(float* cos_tab, float* sin_tab, const int* positions, int rows,
                                int head_dim, double theta, hipStream_t stream);
// Per-row document bounds and positions from cu_seqlens ([ndocs + 1] document offsets).
hipError_t launch_segments(const int* cu_seqlens, int ndocs, int seq_len, int* seg_lo,
                           int* seg_hi, int* positions, hipStream_t stream);

hipError_t launch_qknorm_rope_fwd(IoType io, int head_dim, const void* x, const float* gamma,
                                  const float* cos_tab, const float* sin_tab, void* y,
                                  float* rstd, int nrows, int seq_len, float eps,
                                  hipStream_t stream);
// The same rows with the RoPE table built in the launch (written to cos_tab / sin_tab as
// launch_rope_cache, or launch_rope_cache_at when positions is not null); heads = rows of
// the [heads, seq_len, head_dim] tensor.
hipError_t launch_qknorm_rope_fwd_table(IoType io, int head_dim, const void* x,
                                        const float* gamma, const int* positions, double theta,
                                        float* cos_tab, float* sin_tab, void* y, float* rstd,
                                        int heads, int seq_len, float eps, hipStream_t stream);

// Number of per-block dgamma partial rows the backward writes for `nrows` rows.
int qknorm_rope_bwd_blocks(int64_t nrows);

// dy_io is the dtype of dy (may be fp32 while x / dx are bf16).  partials: workspace of
// qknorm_rope_bwd_blocks(nrows) * head_dim floats.
hipError_t launch_qknorm_rope_bwd(IoType dy_io, IoType x_io, int head_dim, const void* dy,
                                  const void* x, const float* gamma, const float* rstd,
                                  const float* cos_tab, const float* sin_tab, void* dx,
                                  float* dgamma, float* partials, int nrows, int seq_len,
                                  hipStream_t stream);

// Q and K in one launch (and one dgamma reduction launch); same arithmetic and orders
// as two launch_qknorm_rope_bwd calls.
hipError_t launch_qknorm_rope_bwd_qk(IoType dy_io, IoType x_io, int head_dim, const void* dyq,
                                     const void* xq, const float* gamma_q, const float* rstd_q,
                                     void* dxq, float* dgamma_q, float* partials_q, int nrows_q,
                                     const void* dyk, const void* xk, const float* gamma_k,
                                     const float* rstd_k, void* dxk, float* dgamma_k,
                                     float* partials_k, int nrows_k, const float* cos_tab,
                                     const float* sin_tab, int seq_len, hipStream_t stream);

// dgamma of one or two tensors from per-slot partials ([head_dim][nparts], column-major),
// summed in a fixed order.  nparts_k == 0 reduces the first tensor only.
hipError_t launch_dgamma_reduce_qk(int head_dim, const float* partials_q, int nparts_q,
                                   float* dgamma_q, const float* partials_k, int nparts_k,
                                   float* dgamma_k, hipStream_t stream);

// ---- attention -----------------------------------------------------------------------
struct AttnShape {
  int batch, seq_len, num_heads, num_kv_heads, head_dim;
  // block-causal mask of packed documents: [seq_len] first / last row of each row's
  // document (both null: plain causal attention)
  const int* seg_lo = nullptr;
  const int* seg_hi = nullptr;
};


// gfx950 fast path (bf16 io, head_dim 64 or 128), attn_bf16.hip.  The backward also
// writes -lse * log2(e) and -D (D = dO . out) per query row (workspace) for its dk/dv kernel.
bool fast_bf16_supported(int head_dim);
// With `pro` non-null the forward reads the raw pro->xq instead of q and applies the
// QK-norm + RoPE forward to its resident Q rows itself, writing the rotated rows to
// pro->yq and their rstd to pro->rstd_q (what xattn_bwd takes as q and rstd_q).
struct QProFuse {
  const void* xq;
  const float *gamma_q, *cos_tab, *sin_tab;
  void* yq;
  float* rstd_q;
  float eps;
};
hipError_t launch_attn_fwd_bf16_fast(const AttnShape& s, const void* q, const void* k,
                                     const void* v, void* out, float* lse,
                                     const QProFuse* pro, hipStream_t stream);
// Any io / head_dim.  `pro` (q unused) as for launch_attn_fwd_bf16_fast: the Q side of the
// prologue runs inside the forward, for every io dtype and head_dim.
hipError_t launch_attn_fwd(IoType io, const AttnShape& s, const void* q, const void* k,
                           const void* v, void* out, float* lse, const QProFuse* pro,
                           hipStream_t stream);
//
// With `pro` non-null the prologue backward is applied in the dq and dk stores: dq, dk
// receive the gradients w.r.t. the raw xq, xk (io dtype) and dgamma_q, dgamma_k are
// written from partials_q / partials_k (workspace of fused_pro_parts_q(B*H, S) and
// fused_pro_parts_k(B*Hkv, S) slots of head_dim floats each).
struct ProFuse {
  const void* xq;
  const void* xk;
  const float *gamma_q, *gamma_k, *rstd_q, *rstd_k, *cos_tab, *sin_tab;
  float *partials_q, *partials_k, *dgamma_q, *dgamma_k;
};
int fused_pro_parts_q(int64_t q_heads, int seq_len);
int fused_pro_parts_k(int64_t kv_heads, int seq_len);
hipError_t launch_attn_bwd_bf16_fast(const AttnShape& s, const void* q, const void* k,
                                     const void* v, const void* out, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv,
                                     float* delta, float* lse2, const ProFuse* pro,
                                     hipStream_t stream);

// grads_f32: when true, dq and dk are written as fp32 (used when the standalone prologue
// backward follows inside xattn_bwd); otherwise in the io dtype.  dv is always in the io
// dtype.  dkdv_part: fp32 scratch of dkdv_partial_floats(io, s) floats (the generic dk/dv
// kernel splits the group's query heads over workgroups for shapes with few key blocks; NULL
// when that is 0).  pro (only where generic_pro_parts(io, s) holds; grads_f32 false): the
// prologue backward is applied in the dq and dk stores as in launch_attn_bwd_bf16_fast, with
// generic_pro_parts' nq / nk partial slots of head_dim floats in partials_q / partials_k.
hipError_t launch_attn_bwd(IoType io, const AttnShape& s, const void* q, const void* k,
                           const void* v, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* delta,
                           float* lse2, bool grads_f32, float* dkdv_part, const ProFuse* pro,
                           hipStream_t stream);
size_t dkdv_partial_floats(IoType io, const AttnShape& s);
// Whether the generic kernels (bf16, head_dim 16 / 32) apply the prologue backward in their
// stores for this shape (not where the dk/dv launch splits the group's query heads), and
// their dgamma partial slot counts.
bool generic_pro_parts(IoType io, const AttnShape& s, int* nq, int* nk);

// ---- KV-cache decode (decode.hip) ---------------------------------------------------
struct DecodeShape {
  int batch, num_heads, num_kv_heads, head_dim, q_len, cache_len, capacity;
  float eps;
};
struct DecodeBufs {
  const void *xq, *xk, *v;
  const float *gamma_q, *gamma_k, *cos_tab, *sin_tab;
  void *k_cache, *v_cache, *out;
  float* lse;
  float* part_o;   // workspace: [B*Hkv][splits][group*Sq][hd]
  float* part_ml;  // workspace: [B*Hkv][splits][group*Sq][2]
  const int* cache_lens = nullptr;  // [B] cached rows per sequence (null: cache_len for all)
};
struct DecodePlan {
  int nsplit, ks;  // key ranges per KV head and keys per range
};
int decode_max_splits(int batch, int num_kv_heads, int cache_rows);
DecodePlan decode_plan(const DecodeShape& d, int cache_rows);
hipError_t launch_decode(IoType io, const DecodeShape& d, const DecodeBufs& bufs,
                         hipStream_t stream);

// ---- projections (proj.hip: layouts and bias sums; gemm.hip: the GEMMs) ----------------
// Head merge of a head-major io-dtype tensor into token rows [rows, cols].
struct MergeJob {
  const void* src;
  void* dst;
  int rows, cols;
};
struct MergeJobs {
  MergeJob job[3];
  int n;
};
// Column sums of an io-dtype [rows, cols] matrix (bias gradients), in a fixed order.
constexpr int kColsumRows = 128;  // rows per partial sum
inline int colsum_parts(int rows) { return (rows + kColsumRows - 1) / kColsumRows; }
struct ColsumJob {
  const void* src;
  float* partial;  // [colsum_parts(rows)][cols] scratch
  float* out;      // [cols]
  int rows, cols;
  int heads;       // 0: src is [rows, cols] row-major; else head-major [B*heads, S, hd]
  int S;           // sequence length of a head-major src (rows = B*S, cols = heads*hd)
};
struct ColsumJobs {
  ColsumJob job[3];
  int n;
};
hipError_t launch_merge_heads(IoType io, const MergeJobs& jobs, int S, int hd,
                              hipStream_t stream);
hipError_t launch_colsum(IoType io, const ColsumJobs& jobs, hipStream_t stream);

// Row-major GEMMs in the io dtype with fp32 accumulation (gemm.hip).  Forms: GEMM_NN
// C = A B (A [m, k], B [k, n]); GEMM_NT C = A B^T (B stored [n, k]); GEMM_TN C = A^T B (A
// stored [k, m]).  A job sums its K segments (each with its own A, B and k) in one fp32
// accumulator.  Outputs: GEMM_OUT_IO_ROWS (io dtype [m, ldc] + bias), GEMM_OUT_IO_HEADS
// (io dtype, row r = b*S + s and column c = h*hd + e stored at [(b*c_heads + h)*S + s][e]
// + bias), GEMM_OUT_F32 (fp32 [m, ldc], ldc == n; with `part` set, K may be split over
// workgroups whose partial products, gemm_partial_floats floats of workspace, are added in
// split order).  Every operand buffer must stay below 2^31 bytes; the callers guarantee
// it and that n, every k and every ld are multiples of 8.
enum { GEMM_NN = 0, GEMM_NT = 1, GEMM_TN = 2 };
enum { GEMM_OUT_IO_ROWS = 0, GEMM_OUT_IO_HEADS = 1, GEMM_OUT_F32 = 2 };
constexpr int kGemmMaxJobs = 3, kGemmMaxSegs = 3;
struct GemmMat {
  const void* p;
  int ld;          // elements per stored row
  uint32_t bytes;  // size of the stored matrix
  // 0: row-major with ld.  Else the matrix is the token-row view [B*S, heads*hd] of a
  // head-major tensor [B*heads, S, hd] (element (b*S + s, h*hd + e) at ((b*heads + h)*S +
  // s)*hd + e; S and hd from the launch), read in place (bf16 only; hd % 64 == 0, and
  // S % 64 == 0 when tokens run along K)
  int heads;
};
struct GemmSeg {
  GemmMat a, b;
  int k;
};
struct GemmJob {
  GemmSeg seg[kGemmMaxSegs];
  int nseg;
  int m, n;
  void* c;
  int ldc;
  int c_heads;
  const float* bias;  // [n] or null (io outputs)
  float* part;        // split-K workspace (fp32 outputs) or null
};
size_t gemm_partial_floats(IoType io, const GemmJob& job);
hipError_t launch_gemm(IoType io, int form, int out, const GemmJob* jobs, int njobs, int S,
                       int hd, hipStream_t stream);

// ---- opt-in per-kernel event timing (see xattn_profile_start) ------------------------
// Construct around each kernel launch: records a start event now and a stop event at
// scope exit on `stream`, when timing is enabled.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  hipStream_t stream_;
  const char* name_ = nullptr;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

void profile_start();
// Waits for the recorded events, aggregates elapsed time per kernel name (in first-launch
// order), disables timing.  Returns the number of distinct kernels (may exceed max_entries).
int profile_stop(char (*names)[48], long long* launches, double* total_ms, int max_entries,
                 hipError_t* err);

}  // namespace xattn
