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
#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {

__global__ void rope_cache_kernel(float* __restrict__ cos_tab, float* __restrict__ sin_tab,
                                  int seq_len, int head_dim, double theta) {
  const int half = head_dim / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= seq_len * half) return;
  const int t = idx / half, i = idx % half;
  const double inv_freq = pow(theta, -2.0 * (double)i / (double)head_dim);
  const double a = (double)t * inv_freq;
  cos_tab[idx] = (float)cos(a);
  sin_tab[idx] = (float)sin(a);
}

hipError_t launch_rope_cache(float* cos_tab, float* sin_tab, int seq_len, int head_dim,
                             double theta, hipStream_t stream) {
  const int n = seq_len * (head_dim / 2);
  ProfScope prof("rope_cache", stream);
  hipLaunchKernelGGL(rope_cache_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cos_tab,
                     sin_tab, seq_len, head_dim, theta);
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
template <typename T, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_fwd_kernel(
    const T* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, T* __restrict__ y, float* __restrict__ rstd, int nrows,
    int seq_len, float eps) {
  constexpr int VEC = V16<T>::n;
  constexpr int HALF = HD / 2;
  constexpr int LPR = HALF / VEC;  // lanes per row
  static_assert(LPR >= 1 && 64 % LPR == 0, "row must split over a power-of-two lane count");
  const int g = blockIdx.x * 256 + threadIdx.x;
  const int row = g / LPR, part = g % LPR;
  const bool valid = row < nrows;
  const int rr = valid ? row : 0;  // rows past the end read row 0 and store nothing
  const int c0 = part * VEC;

  float a[VEC], b[VEC];
  load_f32<T, VEC>(x + (size_t)rr * HD + c0, a);
  load_f32<T, VEC>(x + (size_t)rr * HD + HALF + c0, b);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VEC; ++j) ss += a[j] * a[j] + b[j] * b[j];
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) ss += shfl_xor(ss, m);
  const float r = 1.0f / sqrtf(ss * (1.0f / (float)HD) + eps);

  const int t = rr % seq_len;
  float cs[VEC], sn[VEC], g1[VEC], g2[VEC];
  load_f32<float, VEC>(cos_tab + (size_t)t * HALF + c0, cs);
  load_f32<float, VEC>(sin_tab + (size_t)t * HALF + c0, sn);
  load_f32<float, VEC>(gamma + c0, g1);
  load_f32<float, VEC>(gamma + HALF + c0, g2);
  float o1[VEC], o2[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const float n1 = a[j] * r * g1[j];
    const float n2 = b[j] * r * g2[j];
    o1[j] = n1 * cs[j] - n2 * sn[j];
    o2[j] = n1 * sn[j] + n2 * cs[j];
  }
  if (valid) {
    store_from_f32<T, VEC>(y + (size_t)row * HD + c0, o1);
    store_from_f32<T, VEC>(y + (size_t)row * HD + HALF + c0, o2);
    if (part == 0) rstd[row] = r;
  }
}

template <typename T, int HD>
static hipError_t fwd_dispatch(const void* x, const float* gamma, const float* cos_tab,
                               const float* sin_tab, void* y, float* rstd, int nrows,
                               int seq_len, float eps, hipStream_t stream) {
  constexpr int LPR = (HD / 2) / V16<T>::n;
  const long long threads = (long long)nrows * LPR;
  const int blocks = (int)((threads + 255) / 256);
  ProfScope prof("qknorm_rope_fwd", stream);
  hipLaunchKernelGGL((qknorm_rope_fwd_kernel<T, HD>), dim3(blocks), dim3(256), 0, stream,
                     (const T*)x, gamma, cos_tab, sin_tab, (T*)y, rstd, nrows, seq_len, eps);
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

// --------------------------------------------------------------------------------------
// backward
// --------------------------------------------------------------------------------------
// Rows are split into fixed contiguous chunks, one per block; each block writes one
// [HD] row of dgamma partials, summed over its rows in ascending row order.  The
// partials are then summed over blocks in a fixed order.  Both orders depend only on
// the shape, so dgamma is bitwise reproducible run to run.
constexpr int kBwdMaxBlocks = 1024;
constexpr int kBwdMinRowsPerBlock = 64;

int qknorm_rope_bwd_blocks(int64_t nrows) {
  int64_t nb = (nrows + kBwdMinRowsPerBlock - 1) / kBwdMinRowsPerBlock;
  if (nb > kBwdMaxBlocks) nb = kBwdMaxBlocks;
  if (nb < 1) nb = 1;
  return (int)nb;
}

template <typename TDy, typename TX, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(
    const TDy* __restrict__ dy, const TX* __restrict__ x, const float* __restrict__ gamma,
    const float* __restrict__ rstd, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, TX* __restrict__ dx, float* __restrict__ partials,
    int nrows, int seq_len, int rows_per_block) {
  constexpr int VEC = V16<TX>::n;
  constexpr int HALF = HD / 2;
  constexpr int LPR = HALF / VEC;
  constexpr int RPP = 256 / LPR;  // rows per pass of the block
  __shared__ float red[256][2 * VEC];

  const int tid = threadIdx.x;
  const int sub = tid / LPR, part = tid % LPR;
  const int c0 = part * VEC;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(nrows, r0 + rows_per_block);

  float g1[VEC], g2[VEC];
  load_f32<float, VEC>(gamma + c0, g1);
  load_f32<float, VEC>(gamma + HALF + c0, g2);
  float acc1[VEC], acc2[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc1[j] = acc2[j] = 0.f;

  for (int row = r0 + sub; row < r1; row += RPP) {
    float d1[VEC], d2[VEC], x1[VEC], x2[VEC], cs[VEC], sn[VEC];
    load_f32<TDy, VEC>(dy + (size_t)row * HD + c0, d1);
    load_f32<TDy, VEC>(dy + (size_t)row * HD + HALF + c0, d2);
    load_f32<TX, VEC>(x + (size_t)row * HD + c0, x1);
    load_f32<TX, VEC>(x + (size_t)row * HD + HALF + c0, x2);
    const int t = row % seq_len;
    load_f32<float, VEC>(cos_tab + (size_t)t * HALF + c0, cs);
    load_f32<float, VEC>(sin_tab + (size_t)t * HALF + c0, sn);
    const float r = rstd[row];
    float n1[VEC], n2[VEC];
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      n1[j] = d1[j] * cs[j] + d2[j] * sn[j];   // rotation by the negative angle
      n2[j] = -d1[j] * sn[j] + d2[j] * cs[j];
      dot += g1[j] * n1[j] * x1[j] + g2[j] * n2[j] * x2[j];
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) dot += shfl_xor(dot, m);
    const float coef = dot * r * r * r * (1.0f / (float)HD);
    float o1[VEC], o2[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      o1[j] = g1[j] * n1[j] * r - x1[j] * coef;
      o2[j] = g2[j] * n2[j] * r - x2[j] * coef;
      acc1[j] += n1[j] * x1[j] * r;
      acc2[j] += n2[j] * x2[j] * r;
    }
    store_from_f32<TX, VEC>(dx + (size_t)row * HD + c0, o1);
    store_from_f32<TX, VEC>(dx + (size_t)row * HD + HALF + c0, o2);
  }

#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    red[tid][j] = acc1[j];
    red[tid][VEC + j] = acc2[j];
  }
  __syncthreads();
  if (tid < HD) {
    const int col = tid;
    const int hsel = col / HALF, cc = col % HALF;
    const int p = cc / VEC, j = cc % VEC;
    float s = 0.f;
    for (int sb = 0; sb < RPP; ++sb) s += red[sb * LPR + p][hsel * VEC + j];
    partials[(size_t)blockIdx.x * HD + col] = s;
  }
}

// One wave per dgamma column: lane k sums partial rows k, k+64, ... in ascending order,
// then a fixed xor butterfly combines the 64 lane sums.
__global__ __launch_bounds__(256) void dgamma_reduce_kernel(const float* __restrict__ partials,
                                                            float* __restrict__ dgamma,
                                                            int nblocks, int head_dim) {
  const int col = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (col >= head_dim) return;
  float s = 0.f;
  for (int b = lane; b < nblocks; b += 64) s += partials[(size_t)b * head_dim + col];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += shfl_xor(s, m);
  if (lane == 0) dgamma[col] = s;
}

template <typename TDy, typename TX, int HD>
static hipError_t bwd_dispatch(const void* dy, const void* x, const float* gamma,
                               const float* rstd, const float* cos_tab, const float* sin_tab,
                               void* dx, float* dgamma, float* partials, int nrows,
                               int seq_len, hipStream_t stream) {
  const int nb = qknorm_rope_bwd_blocks(nrows);
  const int rpb = (nrows + nb - 1) / nb;
  {
    ProfScope prof("qknorm_rope_bwd", stream);
    hipLaunchKernelGGL((qknorm_rope_bwd_kernel<TDy, TX, HD>), dim3(nb), dim3(256), 0, stream,
                       (const TDy*)dy, (const TX*)x, gamma, rstd, cos_tab, sin_tab, (TX*)dx,
                       partials, nrows, seq_len, rpb);
  }
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope prof("dgamma_reduce", stream);
    hipLaunchKernelGGL(dgamma_reduce_kernel, dim3((HD + 3) / 4), dim3(256), 0, stream,
                       (const float*)partials, dgamma, nb, HD);
  }
  return hipPeekAtLastError();
}

hipError_t launch_qknorm_rope_bwd(IoType dy_io, IoType x_io, int head_dim, const void* dy,
                                  const void* x, const float* gamma, const float* rstd,
                                  const float* cos_tab, const float* sin_tab, void* dx,
                                  float* dgamma, float* partials, int nrows, int seq_len,
                                  hipStream_t stream) {
#define XATTN_BWD_CASE(TDY, TX, HD)                                                        \
  if (head_dim == HD)                                                                      \
    return bwd_dispatch<TDY, TX, HD>(dy, x, gamma, rstd, cos_tab, sin_tab, dx, dgamma,     \
                                     partials, nrows, seq_len, stream);
#define XATTN_BWD_HDS(TDY, TX)                                                     \
  XATTN_BWD_CASE(TDY, TX, 16) XATTN_BWD_CASE(TDY, TX, 32) XATTN_BWD_CASE(TDY, TX, 64) \
  XATTN_BWD_CASE(TDY, TX, 128)
  if (x_io == IO_F32) {
    if (dy_io == IO_F32) { XATTN_BWD_HDS(float, float) }
  } else {
    if (dy_io == IO_BF16) { XATTN_BWD_HDS(bf16, bf16) }
    if (dy_io == IO_F32) { XATTN_BWD_HDS(float, bf16) }
  }
#undef XATTN_BWD_HDS
#undef XATTN_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
