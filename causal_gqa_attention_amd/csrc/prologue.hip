// QK-norm + rotate_half RoPE prologue: cos/sin cache, fused forward, fused backward
// with a fixed-order dgamma reduction.
//
// What is computed (xtrain "Phase T9: Export to xserv", conventions table and
// Decision 1; Mint documentation 5.4.1-5.4.4 and 5.5.1-5.5.2):
//   forward, per head vector x in R^hd at position t:
//     rstd = 1/sqrt(mean(x^2) + eps), n = gamma * x * rstd,
//     y[i] = n[i] cos(a) - n[i+hd/2] sin(a), y[i+hd/2] = n[i] sin(a) + n[i+hd/2] cos(a),
//     a = t * theta^(-2i/hd);
//   backward: dn = dy rotated by -a; dot = sum(gamma dn x);
//     dx = gamma dn rstd - x dot rstd^3 / hd; dgamma = sum over rows of dn x rstd.
// Arithmetic is fp32 whatever the io dtype ("Phase T12: bf16 mixed precision": norm and
// RoPE run in fp32); the angle is evaluated in fp64 once, in the cache.
//
// Layout on MI355X: the prologue is HBM-bound (one read and one write of each element),
// so each lane moves whole 16-byte vectors; LPR lanes share a row (the first-half chunk
// and the matching second-half chunk, so each lane owns complete rotation pairs) and the
// row reduction is a short xor-shuffle within those lanes.
#include <algorithm>

#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {

// One block covers 4 * (256 / half) consecutive positions: thread f = tid % half owns one
// frequency, evaluates theta^(-2f/hd) once and the angle's cos and sin at 4 positions.
__global__ __launch_bounds__(256) void rope_cache_kernel(float* __restrict__ cos_tab,
                                                         float* __restrict__ sin_tab,
                                                         int seq_len, int head_dim,
                                                         double theta) {
  const int half = head_dim / 2;
  const int f = threadIdx.x % half, lanes = 256 / half;
  const double inv_freq = pow(theta, -2.0 * (double)f / (double)head_dim);
  const int t0 = blockIdx.x * 4 * lanes + (int)threadIdx.x / half;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = t0 + k * lanes;
    if (t < seq_len) {
      double sv, cv;
      sincos((double)t * inv_freq, &sv, &cv);
      cos_tab[(size_t)t * half + f] = (float)cv;
      sin_tab[(size_t)t * half + f] = (float)sv;
    }
  }
}

hipError_t launch_rope_cache(float* cos_tab, float* sin_tab, int seq_len, int head_dim,
                             double theta, hipStream_t stream) {
  const int per_block = 4 * (256 / (head_dim / 2));
  ProfScope prof("rope_cache", stream);
  hipLaunchKernelGGL(rope_cache_kernel, dim3((seq_len + per_block - 1) / per_block), dim3(256),
                     0, stream, cos_tab, sin_tab, seq_len, head_dim, theta);
  return hipPeekAtLastError();
}

// The same table for explicit per-row positions (tokens of packed documents, whose
// positions restart in every document): thread f of a row group owns one frequency.
__global__ __launch_bounds__(256) void rope_cache_at_kernel(float* __restrict__ cos_tab,
                                                            float* __restrict__ sin_tab,
                                                            const int* __restrict__ positions,
                                                            int rows, int head_dim,
                                                            double theta) {
  const int half = head_dim / 2;
  const int f = threadIdx.x % half, lanes = 256 / half;
  const double inv_freq = pow(theta, -2.0 * (double)f / (double)head_dim);
  const int r0 = blockIdx.x * 4 * lanes + (int)threadIdx.x / half;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + k * lanes;
    if (r < rows) {
      double sv, cv;
      sincos((double)positions[r] * inv_freq, &sv, &cv);
      cos_tab[(size_t)r * half + f] = (float)cv;
      sin_tab[(size_t)r * half + f] = (float)sv;
    }
  }
}

hipError_t launch_rope_cache_at(float* cos_tab, float* sin_tab, const int* positions, int rows,
                                int head_dim, double theta, hipStream_t stream) {
  const int per_block = 4 * (256 / (head_dim / 2));
  ProfScope prof("rope_cache", stream);
  hipLaunchKernelGGL(rope_cache_at_kernel, dim3((rows + per_block - 1) / per_block), dim3(256),
                     0, stream, cos_tab, sin_tab, positions, rows, head_dim, theta);
  return hipPeekAtLastError();
}

// Row r of a sequence of packed documents (offsets cu_seqlens[0] = 0 < ... <
// cu_seqlens[ndocs] = seq_len): its document d is the last one with cu_seqlens[d] <= r
// (binary search); seg_lo = cu_seqlens[d], seg_hi = cu_seqlens[d + 1] - 1, position =
// r - seg_lo.  Results are clamped into [0, seq_len) whatever the offsets hold.
__global__ __launch_bounds__(256) void segments_kernel(const int* __restrict__ cu, int ndocs,
                                                       int seq_len, int* __restrict__ seg_lo,
                                                       int* __restrict__ seg_hi,
                                                       int* __restrict__ positions) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= seq_len) return;
  int lo = 0, hi = ndocs - 1;  // invariant: cu[lo] <= r (cu[0] = 0), answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cu[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int a = min(max(cu[lo], 0), r);
  const int b = min(max(cu[lo + 1] - 1, r), seq_len - 1);
  seg_lo[r] = a;
  seg_hi[r] = b;
  if (positions != nullptr) positions[r] = r - a;
}

hipError_t launch_segments(const int* cu_seqlens, int ndocs, int seq_len, int* seg_lo,
                           int* seg_hi, int* positions, hipStream_t stream) {
  ProfScope prof("segments", stream);
  hipLaunchKernelGGL(segments_kernel, dim3((seq_len + 255) / 256), dim3(256), 0, stream,
                     cu_seqlens, ndocs, seq_len, seg_lo, seg_hi, positions);
  return hipPeekAtLastError();
}

// Load N contiguous elements (N * sizeof(T) a multiple of 16 bytes) as floats.
template <typename T, int N>
__device__ __forceinline__ void load_f32(const T* __restrict__ p, float (&out)[N]) {
  constexpr int per = V16<T>::n;
  static_assert(N % per == 0, "whole 16-byte vectors only");
#pragma unroll
  for (int k = 0; k < N / per; ++k) {
    const vec16_t<T> v = load16(p + k * per);
#pragma unroll
    for (int j = 0; j < per; ++j) out[k * per + j] = to_f32(v[j]);
  }
}

template <typename T, int N>
__device__ __forceinline__ void store_from_f32(T* __restrict__ p, const float (&in)[N]) {
  constexpr int per = V16<T>::n;
  static_assert(N % per == 0, "whole 16-byte vectors only");
#pragma unroll
  for (int k = 0; k < N / per; ++k) {
    vec16_t<T> v;
#pragma unroll
    for (int j = 0; j < per; ++j) v[j] = from_f32<T>(in[k * per + j]);
    store16(p + k * per, v);
  }
}

// --------------------------------------------------------------------------------------
// forward
// --------------------------------------------------------------------------------------
// The arithmetic of one row for the lane owning columns [c0, c0 + VEC) and the matching
// second-half columns (a: first-half values, b: second-half values): the row's mean square
// over its LPR lanes, rstd, then y = rotate(gamma * x * rstd).  Shared by both forward
// kernels, so they give bitwise the same rows: every product and sum is rounded on its own
// (no multiply-add contraction, whose choice could differ with the inlining context).
template <int HD, int VEC>
__device__ __forceinline__ float qknorm_rope_row(const float (&a)[VEC], const float (&b)[VEC],
                                                 const float (&g1)[VEC], const float (&g2)[VEC],
                                                 const float (&cs)[VEC], const float (&sn)[VEC],
                                                 float eps, float (&o1)[VEC], float (&o2)[VEC]) {
#pragma clang fp contract(off)
  constexpr int LPR = (HD / 2) / VEC;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) ss += a[e] * a[e] + b[e] * b[e];
  ss = xor_sum_up<LPR>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / (float)HD) + eps);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float n1 = a[e] * r * g1[e];
    const float n2 = b[e] * r * g2[e];
    o1[e] = n1 * cs[e] - n2 * sn[e];
    o2[e] = n1 * sn[e] + n2 * cs[e];
  }
  return r;
}

// Rows are taken in groups of R heads at one position t (rows h*S + t, h in the group):
// the lanes of a row group load the position's cos / sin and gamma once and issue the R
// rows' loads together.  Row groups are numbered with t fastest, so neighbouring groups
// read neighbouring rows.
template <typename T, int HD, int R>
__global__ __launch_bounds__(256) void qknorm_rope_fwd_kernel(
    const T* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, T* __restrict__ y, float* __restrict__ rstd, int ngroups,
    int seq_len, float eps) {
  constexpr int VEC = V16<T>::n;
  constexpr int HALF = HD / 2;
  constexpr int LPR = HALF / VEC;  // lanes per row
  static_assert(LPR >= 1 && 64 % LPR == 0, "row must split over a power-of-two lane count");
  const int g = blockIdx.x * 256 + threadIdx.x;
  const int rg = g / LPR, part = g % LPR;
  const bool valid = rg < ngroups;
  const int rgv = valid ? rg : 0;  // lanes past the end redo group 0 and store nothing
  const int t = rgv % seq_len, h0 = (rgv / seq_len) * R;
  const int c0 = part * VEC;

  float a[R][VEC], b[R][VEC];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const size_t row = (size_t)(h0 + j) * seq_len + t;
    load_f32<T, VEC>(x + row * HD + c0, a[j]);
    load_f32<T, VEC>(x + row * HD + HALF + c0, b[j]);
  }
  float cs[VEC], sn[VEC], g1[VEC], g2[VEC];
  load_f32<float, VEC>(cos_tab + (size_t)t * HALF + c0, cs);
  load_f32<float, VEC>(sin_tab + (size_t)t * HALF + c0, sn);
  load_f32<float, VEC>(gamma + c0, g1);
  load_f32<float, VEC>(gamma + HALF + c0, g2);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float o1[VEC], o2[VEC];
    const float r = qknorm_rope_row<HD, VEC>(a[j], b[j], g1, g2, cs, sn, eps, o1, o2);
    if (valid) {
      const size_t row = (size_t)(h0 + j) * seq_len + t;
      store_from_f32<T, VEC>(y + row * HD + c0, o1);
      store_from_f32<T, VEC>(y + row * HD + HALF + c0, o2);
      if (part == 0) rstd[row] = r;
    }
  }
}

// heads per row group: 4 when the head count allows it
static int fwd_group(int heads) { return heads % 4 == 0 ? 4 : (heads % 2 == 0 ? 2 : 1); }

template <typename T, int HD>
static hipError_t fwd_dispatch(const void* x, const float* gamma, const float* cos_tab,
                               const float* sin_tab, void* y, float* rstd, int nrows,
                               int seq_len, float eps, hipStream_t stream) {
  constexpr int LPR = (HD / 2) / V16<T>::n;
  const int heads = nrows / seq_len, R = fwd_group(heads);
  const int ngroups = (heads / R) * seq_len;
  const long long threads = (long long)ngroups * LPR;
  const int blocks = (int)((threads + 255) / 256);
  ProfScope prof("qknorm_rope_fwd", stream);
#define XATTN_FWD_R(RV)                                                                    \
  hipLaunchKernelGGL((qknorm_rope_fwd_kernel<T, HD, RV>), dim3(blocks), dim3(256), 0, stream, \
                     (const T*)x, gamma, cos_tab, sin_tab, (T*)y, rstd, ngroups, seq_len, eps)
  if (R == 4) XATTN_FWD_R(4);
  else if (R == 2) XATTN_FWD_R(2);
  else XATTN_FWD_R(1);
#undef XATTN_FWD_R
  return hipPeekAtLastError();
}

hipError_t launch_qknorm_rope_fwd(IoType io, int head_dim, const void* x, const float* gamma,
                                  const float* cos_tab, const float* sin_tab, void* y,
                                  float* rstd, int nrows, int seq_len, float eps,
                                  hipStream_t stream) {
#define XATTN_FWD_CASE(T, HD)                                                            \
  if (head_dim == HD)                                                                    \
    return fwd_dispatch<T, HD>(x, gamma, cos_tab, sin_tab, y, rstd, nrows, seq_len, eps, \
                               stream);
  if (io == IO_F32) {
    XATTN_FWD_CASE(float, 16) XATTN_FWD_CASE(float, 32) XATTN_FWD_CASE(float, 64)
    XATTN_FWD_CASE(float, 128)
  } else {
    XATTN_FWD_CASE(bf16, 16) XATTN_FWD_CASE(bf16, 32) XATTN_FWD_CASE(bf16, 64)
    XATTN_FWD_CASE(bf16, 128)
  }
#undef XATTN_FWD_CASE
  return hipErrorInvalidValue;
}

// Prologue forward with the RoPE table built in the same launch.  Block (bx, by) owns
// positions [bx*P, bx*P + P) of head rows [by*HB, by*HB + HB): at most 256 / LPR rows, one
// pass, its loads issued first.  Under them it evaluates the table entries of its positions
// (P * HD/2 <= 256, one per thread, as the table kernels do: one pow and one sincos in fp64,
// rounded once to fp32) into LDS; blocks with by == 0 also write them to the table.  Then it
// normalises and rotates its rows.  Every row and table entry is bitwise what
// xattn_rope_cache(_at) followed by xattn_qknorm_rope_fwd give.
template <typename T, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_fwd_table_kernel(
    const T* __restrict__ x, const float* __restrict__ gamma, const int* __restrict__ positions,
    double theta, float* __restrict__ cos_tab, float* __restrict__ sin_tab, T* __restrict__ y,
    float* __restrict__ rstd, int heads, int seq_len, int P, int HB, float eps) {
  constexpr int VEC = V16<T>::n;
  constexpr int HALF = HD / 2;
  constexpr int LPR = HALF / VEC;
  __shared__ float tcs[256], tsn[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * P, h0 = blockIdx.y * HB;
  const int np = min(P, seq_len - t0);  // positions of this block
  const int nh = min(HB, heads - h0);   // head rows of this block
  const int nrows = nh * np;            // (h0 + k / np, t0 + k % np) for k < nrows
  const int g = tid / LPR, part = tid % LPR, c0 = part * VEC;
  const int k = g < nrows ? g : 0;      // lanes past the rows redo row 0 and store nothing
  const int i = k % np;
  const size_t row = (size_t)(h0 + k / np) * seq_len + t0 + i;
  float a[VEC], b[VEC], g1[VEC], g2[VEC];
  load_f32<T, VEC>(x + row * HD + c0, a);
  load_f32<T, VEC>(x + row * HD + HALF + c0, b);
  load_f32<float, VEC>(gamma + c0, g1);
  load_f32<float, VEC>(gamma + HALF + c0, g2);
  // table entries of the block's positions: thread tid -> (position tid / HALF, frequency
  // tid % HALF)
  if (tid < np * HALF) {
    const int p = tid / HALF, f = tid % HALF, t = t0 + p;
    const double inv_freq = pow(theta, -2.0 * (double)f / (double)HD);
    const int pos = positions != nullptr ? positions[t] : t;
    double sv, cv;
    sincos((double)pos * inv_freq, &sv, &cv);
    tcs[tid] = (float)cv;
    tsn[tid] = (float)sv;
    if (blockIdx.y == 0) {
      cos_tab[(size_t)t * HALF + f] = (float)cv;
      sin_tab[(size_t)t * HALF + f] = (float)sv;
    }
  }
  __syncthreads();
  float cs[VEC], sn[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    cs[e] = tcs[i * HALF + c0 + e];
    sn[e] = tsn[i * HALF + c0 + e];
  }
  float o1[VEC], o2[VEC];
  const float r = qknorm_rope_row<HD, VEC>(a, b, g1, g2, cs, sn, eps, o1, o2);
  if (g < nrows) {
    store_from_f32<T, VEC>(y + row * HD + c0, o1);
    store_from_f32<T, VEC>(y + row * HD + HALF + c0, o2);
    if (part == 0) rstd[row] = r;
  }
}

template <typename T, int HD>
static hipError_t fwd_table_dispatch(const void* x, const float* gamma, const int* positions,
                                     double theta, float* cos_tab, float* sin_tab, void* y,
                                     float* rstd, int heads, int seq_len, float eps,
                                     hipStream_t stream) {
  constexpr int HALF = HD / 2;
  constexpr int NG = 256 / (HALF / V16<T>::n);  // rows per block
  // positions per block: as many as leave one row group per head row (at most one table
  // entry per thread), and at head_dim <= 32 (rows of 64 bytes or less) at least enough
  // for 8 heads' rows to form contiguous runs; head rows per block: the rest of the block
  const int P = std::max(1, std::min(256 / HALF, NG / (HD <= 32 ? std::min(heads, 8) : heads)));
  const int HB = std::max(1, NG / P);
  const dim3 grid((seq_len + P - 1) / P, (heads + HB - 1) / HB);
  ProfScope prof("qknorm_rope_fwd", stream);
  hipLaunchKernelGGL((qknorm_rope_fwd_table_kernel<T, HD>), grid, dim3(256), 0, stream,
                     (const T*)x, gamma, positions, theta, cos_tab, sin_tab, (T*)y, rstd, heads,
                     seq_len, P, HB, eps);
  return hipPeekAtLastError();
}

hipError_t launch_qknorm_rope_fwd_table(IoType io, int head_dim, const void* x,
                                        const float* gamma, const int* positions, double theta,
                                        float* cos_tab, float* sin_tab, void* y, float* rstd,
                                        int heads, int seq_len, float eps, hipStream_t stream) {
#define XATTN_FWD_CASE(T, HD)                                                                \
  if (head_dim == HD)                                                                        \
    return fwd_table_dispatch<T, HD>(x, gamma, positions, theta, cos_tab, sin_tab, y, rstd, \
                                     heads, seq_len, eps, stream);
  if (io == IO_F32) {
    XATTN_FWD_CASE(float, 16) XATTN_FWD_CASE(float, 32) XATTN_FWD_CASE(float, 64)
    XATTN_FWD_CASE(float, 128)
  } else {
    XATTN_FWD_CASE(bf16, 16) XATTN_FWD_CASE(bf16, 32) XATTN_FWD_CASE(bf16, 64)
    XATTN_FWD_CASE(bf16, 128)
  }
#undef XATTN_FWD_CASE
  return hipErrorInvalidValue;
}

// --------------------------------------------------------------------------------------
// backward
// --------------------------------------------------------------------------------------
// Row groups (R heads at one position, as in the forward) are split into equal contiguous
// chunks, one per block; a block's 256 / LPR group slots take the chunk's groups in turn.
// Each lane accumulates its dgamma terms in a fixed order, the block sums its lanes in a
// fixed order into one partial per column, stored column-major ([HD][nblocks]) so that the
// reduction reads each column contiguously; a reduction wave then sums a column's partials
// in a fixed order.  Every order depends only on the shape, so dgamma is bitwise
// reproducible run to run.  One launch serves one or two tensors (Q and K).
constexpr int kBwdMaxBlocks = 1024;
constexpr int kBwdRowsPerBlock = 128;
constexpr int kBwdHeadsPerGroup = 2;  // rows handled together by a lane (1, 2 or 4)

int qknorm_rope_bwd_blocks(int64_t nrows) {
  int64_t nb = (nrows + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock;
  if (nb > kBwdMaxBlocks) nb = kBwdMaxBlocks;
  if (nb < 1) nb = 1;
  return (int)nb;
}

struct BwdJob {
  const void* dy;
  const void* x;
  const float* gamma;
  const float* rstd;
  void* dx;
  float* partials;  // [HD][nblocks]
  float* dgamma;
  int ngroups, groups_per_block, nblocks, heads_per_group;
};

template <typename TDy, typename TX, int HD, int R>
__device__ __forceinline__ void qknorm_rope_bwd_block(const BwdJob& jb, int blk,
                                                      const float* __restrict__ cos_tab,
                                                      const float* __restrict__ sin_tab,
                                                      int seq_len, float (*red)[2 * V16<TX>::n]) {
  constexpr int VEC = V16<TX>::n;
  constexpr int HALF = HD / 2;
  constexpr int LPR = HALF / VEC;
  constexpr int GPB = 256 / LPR;  // group slots per block
  const TDy* __restrict__ dy = static_cast<const TDy*>(jb.dy);
  const TX* __restrict__ x = static_cast<const TX*>(jb.x);
  TX* __restrict__ dx = static_cast<TX*>(jb.dx);
  const float* __restrict__ rstd = jb.rstd;

  const int tid = threadIdx.x;
  const int slot = tid / LPR, part = tid % LPR;
  const int c0 = part * VEC;
  const int gs = blk * jb.groups_per_block;
  const int ge = min(jb.ngroups, gs + jb.groups_per_block);

  float g1[VEC], g2[VEC];
  load_f32<float, VEC>(jb.gamma + c0, g1);
  load_f32<float, VEC>(jb.gamma + HALF + c0, g2);
  float acc1[VEC], acc2[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc1[e] = acc2[e] = 0.f;

  for (int rg = gs + slot; rg < ge; rg += GPB) {
    const int t = rg % seq_len, h0 = (rg / seq_len) * R;
    float d1[R][VEC], d2[R][VEC], x1[R][VEC], x2[R][VEC], rr[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const size_t row = (size_t)(h0 + j) * seq_len + t;
      load_f32<TDy, VEC>(dy + row * HD + c0, d1[j]);
      load_f32<TDy, VEC>(dy + row * HD + HALF + c0, d2[j]);
      load_f32<TX, VEC>(x + row * HD + c0, x1[j]);
      load_f32<TX, VEC>(x + row * HD + HALF + c0, x2[j]);
      rr[j] = rstd[row];
    }
    float cs[VEC], sn[VEC];
    load_f32<float, VEC>(cos_tab + (size_t)t * HALF + c0, cs);
    load_f32<float, VEC>(sin_tab + (size_t)t * HALF + c0, sn);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float r = rr[j];
      float n1[VEC], n2[VEC];
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        n1[e] = d1[j][e] * cs[e] + d2[j][e] * sn[e];  // rotation by the negative angle
        n2[e] = -d1[j][e] * sn[e] + d2[j][e] * cs[e];
        dot += g1[e] * n1[e] * x1[j][e] + g2[e] * n2[e] * x2[j][e];
      }
      dot = xor_sum_up<LPR>(dot);
      const float coef = dot * r * r * r * (1.0f / (float)HD);
      float o1[VEC], o2[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        o1[e] = g1[e] * n1[e] * r - x1[j][e] * coef;
        o2[e] = g2[e] * n2[e] * r - x2[j][e] * coef;
        acc1[e] += n1[e] * x1[j][e] * r;
        acc2[e] += n2[e] * x2[j][e] * r;
      }
      const size_t row = (size_t)(h0 + j) * seq_len + t;
      store_from_f32<TX, VEC>(dx + row * HD + c0, o1);
      store_from_f32<TX, VEC>(dx + row * HD + HALF + c0, o2);
    }
  }

#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    red[tid][e] = acc1[e];
    red[tid][VEC + e] = acc2[e];
  }
  __syncthreads();
  if (tid < HD) {
    const int col = tid;
    const int hsel = col / HALF, cc = col % HALF;
    const int p = cc / VEC, e = cc % VEC;
    float sum = 0.f;
    for (int sb = 0; sb < GPB; ++sb) sum += red[sb * LPR + p][hsel * VEC + e];
    jb.partials[(size_t)col * jb.nblocks + blk] = sum;
  }
}

template <typename TDy, typename TX, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(BwdJob j0, BwdJob j1,
                                                              const float* __restrict__ cos_tab,
                                                              const float* __restrict__ sin_tab,
                                                              int seq_len) {
  __shared__ float red[256][2 * V16<TX>::n];
  const bool second = (int)blockIdx.x >= j0.nblocks;
  const BwdJob& jb = second ? j1 : j0;
  const int blk = second ? (int)blockIdx.x - j0.nblocks : (int)blockIdx.x;
  if (jb.heads_per_group == 4)
    qknorm_rope_bwd_block<TDy, TX, HD, 4>(jb, blk, cos_tab, sin_tab, seq_len, red);
  else if (jb.heads_per_group == 2)
    qknorm_rope_bwd_block<TDy, TX, HD, 2>(jb, blk, cos_tab, sin_tab, seq_len, red);
  else
    qknorm_rope_bwd_block<TDy, TX, HD, 1>(jb, blk, cos_tab, sin_tab, seq_len, red);
}

// One wave per dgamma column of one or two tensors: lane k sums partials k, k + 64, ... of
// the column (contiguous) in ascending order, then a fixed xor butterfly combines the lanes.
__global__ __launch_bounds__(256) void dgamma_reduce_kernel(BwdJob j0, BwdJob j1, int head_dim) {
  const int w = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const bool second = w >= head_dim;
  const BwdJob& jb = second ? j1 : j0;
  const int col = second ? w - head_dim : w;
  if (col >= head_dim) return;
  const float* p = jb.partials + (size_t)col * jb.nblocks;
  float s = 0.f;
  for (int b = lane; b < jb.nblocks; b += 64) s += p[b];
  s = xor_sum_down<64>(s);
  if (lane == 0) jb.dgamma[col] = s;
}

static BwdJob make_job(const void* dy, const void* x, const float* gamma, const float* rstd,
                       void* dx, float* dgamma, float* partials, int nrows, int seq_len) {
  const int heads = nrows / seq_len;
  int R = 1;
  if (kBwdHeadsPerGroup >= 4 && heads % 4 == 0) R = 4;
  else if (kBwdHeadsPerGroup >= 2 && heads % 2 == 0) R = 2;
  BwdJob j;
  j.heads_per_group = R;
  j.dy = dy, j.x = x, j.gamma = gamma, j.rstd = rstd, j.dx = dx, j.partials = partials;
  j.dgamma = dgamma;
  j.nblocks = qknorm_rope_bwd_blocks(nrows);
  j.ngroups = (nrows / seq_len / R) * seq_len;
  j.groups_per_block = (j.ngroups + j.nblocks - 1) / j.nblocks;
  return j;
}

template <typename TDy, typename TX, int HD>
static hipError_t bwd_dispatch(const BwdJob& j0, const BwdJob& j1, const float* cos_tab,
                               const float* sin_tab, int seq_len, hipStream_t stream) {
  const int nb = j0.nblocks + j1.nblocks;
  const int njobs = j1.nblocks > 0 ? 2 : 1;
  {
    ProfScope prof("qknorm_rope_bwd", stream);
    hipLaunchKernelGGL((qknorm_rope_bwd_kernel<TDy, TX, HD>), dim3(nb), dim3(256), 0, stream,
                       j0, j1, cos_tab, sin_tab, seq_len);
  }
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope prof("dgamma_reduce", stream);
    hipLaunchKernelGGL(dgamma_reduce_kernel, dim3((njobs * HD + 3) / 4), dim3(256), 0, stream,
                       j0, j1, HD);
  }
  return hipPeekAtLastError();
}

template <typename TDy, typename TX>
static hipError_t bwd_hd(int head_dim, const BwdJob& j0, const BwdJob& j1,
                         const float* cos_tab, const float* sin_tab, int seq_len,
                         hipStream_t stream) {
  switch (head_dim) {
    case 16: return bwd_dispatch<TDy, TX, 16>(j0, j1, cos_tab, sin_tab, seq_len, stream);
    case 32: return bwd_dispatch<TDy, TX, 32>(j0, j1, cos_tab, sin_tab, seq_len, stream);
    case 64: return bwd_dispatch<TDy, TX, 64>(j0, j1, cos_tab, sin_tab, seq_len, stream);
    case 128: return bwd_dispatch<TDy, TX, 128>(j0, j1, cos_tab, sin_tab, seq_len, stream);
  }
  return hipErrorInvalidValue;
}

static hipError_t bwd_types(IoType dy_io, IoType x_io, int head_dim, const BwdJob& j0,
                            const BwdJob& j1, const float* cos_tab, const float* sin_tab,
                            int seq_len, hipStream_t stream) {
  if (x_io == IO_F32 && dy_io == IO_F32)
    return bwd_hd<float, float>(head_dim, j0, j1, cos_tab, sin_tab, seq_len, stream);
  if (x_io == IO_BF16 && dy_io == IO_BF16)
    return bwd_hd<bf16, bf16>(head_dim, j0, j1, cos_tab, sin_tab, seq_len, stream);
  if (x_io == IO_BF16 && dy_io == IO_F32)
    return bwd_hd<float, bf16>(head_dim, j0, j1, cos_tab, sin_tab, seq_len, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_qknorm_rope_bwd(IoType dy_io, IoType x_io, int head_dim, const void* dy,
                                  const void* x, const float* gamma, const float* rstd,
                                  const float* cos_tab, const float* sin_tab, void* dx,
                                  float* dgamma, float* partials, int nrows, int seq_len,
                                  hipStream_t stream) {
  const BwdJob j0 = make_job(dy, x, gamma, rstd, dx, dgamma, partials, nrows, seq_len);
  BwdJob j1{};
  return bwd_types(dy_io, x_io, head_dim, j0, j1, cos_tab, sin_tab, seq_len, stream);
}

hipError_t launch_qknorm_rope_bwd_qk(IoType dy_io, IoType x_io, int head_dim, const void* dyq,
                                     const void* xq, const float* gamma_q, const float* rstd_q,
                                     void* dxq, float* dgamma_q, float* partials_q, int nrows_q,
                                     const void* dyk, const void* xk, const float* gamma_k,
                                     const float* rstd_k, void* dxk, float* dgamma_k,
                                     float* partials_k, int nrows_k, const float* cos_tab,
                                     const float* sin_tab, int seq_len, hipStream_t stream) {
  const BwdJob jq = make_job(dyq, xq, gamma_q, rstd_q, dxq, dgamma_q, partials_q, nrows_q,
                             seq_len);
  const BwdJob jk = make_job(dyk, xk, gamma_k, rstd_k, dxk, dgamma_k, partials_k, nrows_k,
                             seq_len);
  return bwd_types(dy_io, x_io, head_dim, jq, jk, cos_tab, sin_tab, seq_len, stream);
}

// One block per dgamma column of one or two tensors, for many partials per column:
// thread t sums partials t, t + 256, ... in ascending order, a fixed xor butterfly
// combines each wave and thread 0 adds the four wave sums in wave order.
__global__ __launch_bounds__(256) void dgamma_reduce_wide_kernel(const float* __restrict__ pq,
                                                                 int nq, float* __restrict__ gq,
                                                                 const float* __restrict__ pk,
                                                                 int nk, float* __restrict__ gk,
                                                                 int head_dim) {
  __shared__ float wsum[4];
  const bool second = (int)blockIdx.x >= head_dim;
  const int col = second ? blockIdx.x - head_dim : blockIdx.x;
  const int n = second ? nk : nq;
  const float* p = (second ? pk : pq) + (size_t)col * n;
  const int tid = threadIdx.x;
  float s = 0.f;
#pragma unroll 8
  for (int b = tid; b < n; b += 256) s += p[b];
  s = xor_sum_down<64>(s);
  if ((tid & 63) == 0) wsum[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) (second ? gk : gq)[col] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

hipError_t launch_dgamma_reduce_qk(int head_dim, const float* partials_q, int nparts_q,
                                   float* dgamma_q, const float* partials_k, int nparts_k,
                                   float* dgamma_k, hipStream_t stream) {
  const int njobs = nparts_k > 0 ? 2 : 1;
  ProfScope prof("dgamma_reduce", stream);
  hipLaunchKernelGGL(dgamma_reduce_wide_kernel, dim3(njobs * head_dim), dim3(256), 0, stream,
                     partials_q, nparts_q, dgamma_q, partials_k, nparts_k, dgamma_k, head_dim);
  return hipPeekAtLastError();
}

}  // namespace xattn
