// Device-side helpers shared by the libxattn kernels (gfx950 / CDNA4 only).
//
// MFMA operand conventions used throughout (checked on the device):
//   v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32, wave64, lane l, c32 = l % 32,
//   h = l / 32.  A operand: row c32; B operand: column c32; both carry the lane's
//   k-slots (8h..8h+7 for bf16, slot h for f32).  Accumulator register i of lane l
//   holds C[row = 8*(i/4) + 4*h + (i%4)][col = c32].
//   The contraction is invariant to any permutation of k applied identically to A
//   and B, which is what lets the kernels place whole 16-byte chunks per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte vector of an io dtype.
template <typename T> struct V16;
template <> struct V16<float> { typedef f32x4 type; static constexpr int n = 4; };
template <> struct V16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };

template <typename T> using vec16_t = typename V16<T>::type;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ vec16_t<T> vzero() {
  vec16_t<T> z;
#pragma unroll
  for (int j = 0; j < V16<T>::n; ++j) z[j] = from_f32<T>(0.f);
  return z;
}

template <typename T> __device__ __forceinline__ vec16_t<T> load16(const T* p) {
  return *reinterpret_cast<const vec16_t<T>*>(p);
}
template <typename T> __device__ __forceinline__ void store16(T* p, const vec16_t<T>& v) {
  *reinterpret_cast<vec16_t<T>*>(p) = v;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// One 16-byte chunk of the contraction: A and B each carry the same k-slots.
__device__ __forceinline__ f32x16 mfma_chunk(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_chunk(const f32x4& a, const f32x4& b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives element (i % 4) of the four 16-bit values at the address given by lane
// 4*j + i/4, as its element j.  With lane a pointing at row (r0 + a/4), column
// (c0 + 4*(a%4)) of a row-major tile, lane i receives column c0 + i of rows r0..r0+3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// v moved across lanes by the DPP control CTRL (lanes outside the pattern read 0).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// The value of lane l ^ M (M a power of two up to 32) without an LDS round trip: DPP within
// a 16-lane row (quad permutations; quad reversal then the half-row mirror for 4; a rotation
// by 8), v_permlane16_swap / v_permlane32_swap across rows.
template <int M>
__device__ __forceinline__ float xor_lanes(float v) {
  if constexpr (M == 1) {
    return dpp_mov<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (M == 2) {
    return dpp_mov<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (M == 4) {
    return dpp_mov<0x141>(dpp_mov<0x1B>(v));  // quad_perm [3, 2, 1, 0], then row_half_mirror
  } else if constexpr (M == 8) {
    return dpp_mov<0x128>(v);  // row_ror:8
  } else {
    static_assert(M == 16 || M == 32, "xor of a power of two up to 32");
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const int lane = __lane_id();
    if constexpr (M == 16) {
      // result 0: lane l holds lane (l & ~16); result 1: lane (l | 16)
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      return __builtin_bit_cast(float, (unsigned)((lane & 16) ? r[0] : r[1]));
    } else {
      // result 0: lane l holds lane (l & 31); result 1: lane (l | 32)
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      return __builtin_bit_cast(float, (unsigned)((lane & 32) ? r[0] : r[1]));
    }
  }
}

// Sum over groups of N consecutive lanes (N a power of two up to 64) by xor exchanges of
// increasing distance: 1, 2, ..., N/2 (the same order as a shuffle loop over those masks).
template <int N, int M = 1>
__device__ __forceinline__ float xor_sum_up(float v) {
  if constexpr (M < N) return xor_sum_up<N, 2 * M>(v + xor_lanes<M>(v));
  else return v;
}
// The same with decreasing distances N/2, ..., 1.
template <int N>
__device__ __forceinline__ float xor_sum_down(float v) {
  if constexpr (N > 1) return xor_sum_down<N / 2>(v + xor_lanes<N / 2>(v));
  else return v;
}

// Sums v[0..N) over the lanes that differ in lane bits M, M/2, .., MLAST by recursive
// halving: at the step for bit m the lane keeps one half of its remaining values (the upper
// one if its bit m is set), sends the other half to lane ^ m and adds what that lane sends.
// Fixed order, so bitwise reproducible.
template <int NV, int N, int M, int MLAST>
__device__ __forceinline__ void halving_sum(float (&v)[NV], int lane) {
  constexpr int H = N / 2;
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float keep = up ? v[k + H] : v[k];
    const float send = up ? v[k] : v[k + H];
    v[k] = keep + xor_lanes<M>(send);
  }
  if constexpr (M > MLAST) halving_sum<NV, H, M / 2, MLAST>(v, lane);
}

// Inputs and dgamma output of a prologue backward applied in an attention kernel's dq / dk
// stores (bf16 io): the gradient w.r.t. the rotated rows stays in the kernel, and the
// dgamma terms of each workgroup (or wave) go to one partial slot, reduced by a later launch.
struct ProBwd {
  const bf16* x;         // pre-norm rows, indexed like the gradient ([rows, S, HD])
  const float* gamma;    // [HD]
  const float* rstd;     // [rows * S], from the prologue forward
  const float* cos_tab;  // [S, HD / 2]
  const float* sin_tab;  // [S, HD / 2]
  float* partials;       // [HD][nparts] column-major, one slot per workgroup or wave
  int nparts;
};

}  // namespace xattn
