// Layout and reduction kernels around the projection GEMMs (Mint documentation 5.3.1-5.3.2:
// Q = X Wq + bq, ..., output Concat(heads) Wo + bo; "Phase T5: Tiny Transformer" layout
// pipeline: the projection's [tokens, heads*hd] rows are reshaped to [tokens, heads, hd] and
// transposed so that each head's [seq, hd] block is contiguous, and merged back before Wo).
//
// The GEMMs (gemm.hip) split their outputs into heads themselves; what remains here are
// HBM-bound passes: the head merge of an attention-layout tensor into token rows (each lane
// moves 16-byte vectors) and the bias gradients as fixed-order column sums.
#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {
namespace {

// Element (m, c) of a token-row matrix [B*S, heads*hd] <-> element (b*heads + h, s, e) of
// the head-major tensor, m = b*S + s, c = h*hd + e.
__device__ __forceinline__ size_t head_index(size_t m, int c, int S, int heads, int hd) {
  const size_t b = m / S, s = m - b * S;
  const int h = c / hd, e = c - h * hd;
  return ((b * heads + h) * S + s) * hd + e;
}

// Merge: dst (token rows, io dtype) = src (head-major, io dtype); up to three tensors.
template <typename T>
__global__ __launch_bounds__(256) void merge_heads_kernel(MergeJobs jobs, int S, int hd) {
  size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  constexpr int VEC = V16<T>::n;
  for (int j = 0; j < jobs.n; ++j) {
    const MergeJob& jb = jobs.job[j];
    const size_t nvec = (size_t)jb.rows * jb.cols / VEC;
    if (g < nvec) {
      const size_t m = g / (jb.cols / VEC);
      const int c = (int)(g - m * (jb.cols / VEC)) * VEC;
      const T* s = static_cast<const T*>(jb.src) + head_index(m, c, S, jb.cols / hd, hd);
      store16(static_cast<T*>(jb.dst) + m * jb.cols + c, load16(s));
      return;
    }
    g -= nvec;
  }
}

// Column sums of [rows, cols] in a fixed order: partial[p][c] sums rows p*chunk ..
// (ascending) for column c; then out[c] = sum over p ascending.  Bitwise reproducible.
template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(ColsumJobs jobs, int chunk) {
  const int c = blockIdx.x * 256 + threadIdx.x, p = blockIdx.y;
  const ColsumJob& jb = jobs.job[blockIdx.z];
  if (c >= jb.cols) return;
  const T* src = static_cast<const T*>(jb.src);
  const size_t r0 = (size_t)p * chunk, r1 = min((size_t)jb.rows, r0 + chunk);
  float s = 0.f;
  if (jb.heads == 0) {
#pragma unroll 8
    for (size_t r = r0; r < r1; ++r) s += to_f32(src[r * jb.cols + c]);
  } else {  // head-major source: column c = (h, e), row r = (b, t), walked t by t
    const int hd = jb.cols / jb.heads, h = c / hd, e = c - h * hd;
    size_t b = r0 / jb.S, t = r0 - b * jb.S;
    for (size_t r = r0; r < r1;) {
      const size_t n = min(r1 - r, (size_t)jb.S - t);  // rows left in this sequence
      const T* q = src + ((b * jb.heads + h) * jb.S + t) * hd + e;
#pragma unroll 8
      for (size_t i = 0; i < n; ++i) s += to_f32(q[i * hd]);
      r += n;
      ++b;
      t = 0;
    }
  }
  jb.partial[(size_t)p * jb.cols + c] = s;
}

__global__ __launch_bounds__(256) void colsum_final_kernel(ColsumJobs jobs, int nparts) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const ColsumJob& jb = jobs.job[blockIdx.z];
  if (c >= jb.cols) return;
  float s = 0.f;
#pragma unroll 8
  for (int p = 0; p < nparts; ++p) s += jb.partial[(size_t)p * jb.cols + c];
  jb.out[c] = s;
}

}  // namespace

hipError_t launch_merge_heads(IoType io, const MergeJobs& jobs, int S, int hd,
                              hipStream_t stream) {
  const int vec = io == IO_F32 ? 4 : 8;
  size_t total = 0;
  for (int j = 0; j < jobs.n; ++j) total += (size_t)jobs.job[j].rows * jobs.job[j].cols / vec;
  ProfScope prof("merge_heads", stream);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (io == IO_F32)
    hipLaunchKernelGGL(merge_heads_kernel<float>, grid, dim3(256), 0, stream, jobs, S, hd);
  else
    hipLaunchKernelGGL(merge_heads_kernel<bf16>, grid, dim3(256), 0, stream, jobs, S, hd);
  return hipPeekAtLastError();
}

hipError_t launch_colsum(IoType io, const ColsumJobs& jobs, hipStream_t stream) {
  int maxc = 0;
  size_t rows = 0;
  for (int j = 0; j < jobs.n; ++j) {
    maxc = jobs.job[j].cols > maxc ? jobs.job[j].cols : maxc;
    rows = jobs.job[j].rows > rows ? jobs.job[j].rows : rows;
  }
  const int nparts = colsum_parts((int)rows);
  const dim3 g1((maxc + 255) / 256, nparts, jobs.n), g2((maxc + 255) / 256, 1, jobs.n);
  ProfScope prof("bias_grad", stream);
  if (io == IO_F32)
    hipLaunchKernelGGL(colsum_partial_kernel<float>, g1, dim3(256), 0, stream, jobs,
                       kColsumRows);
  else
    hipLaunchKernelGGL(colsum_partial_kernel<bf16>, g1, dim3(256), 0, stream, jobs,
                       kColsumRows);
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_final_kernel, g2, dim3(256), 0, stream, jobs, nparts);
  return hipPeekAtLastError();
}

}  // namespace xattn
