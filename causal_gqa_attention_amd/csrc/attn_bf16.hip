// Causal GQA attention for bf16 io at head_dim 64 and 128 (the dim768 and long-context
// shapes), forward and backward, tuned for gfx950.  Same mathematics as attn.hip
// (Mint documentation 5.3.1; xtrain "Phase T9: Export to xserv" conventions table;
// xtrain "Phase T15: GQA" head mapping and deterministic group sum), restructured for
// throughput:
//
//   * HBM -> LDS staging with direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): no
//     register round trip, issued a stage or two ahead so the loads overlap the MFMA work.
//     A wave-level load writes 64 x 16 contiguous bytes, so tile rows are unpadded and bank
//     conflicts are avoided by XOR-swizzling the 16-byte chunks of each row.  Each tile gets
//     a buffer descriptor that covers only its rows before the sequence end: the hardware
//     range check fills the rest with zeros, so ragged tiles need no per-lane clamping.
//   * The copies are inline assembly, invisible to the compiler's wait-count insertion
//     (which would otherwise make every transposing LDS read wait for all loads in flight);
//     the kernels order them against LDS reads with explicit vmcnt waits and barriers.
//   * The swizzle depends on the row modulo 16 only and satisfies swz(r + 8) = swz(r) ^ 2,
//     so every LDS operand address is (a lane-constant value) XOR (a compile-time constant)
//     plus a base.  Load addresses are per-lane 32-bit offsets, fixed for the whole kernel.
//   * One barrier per stage: the wait for this stage's loads (vmcnt), the barrier and an
//     LDS-only acquire fence; no release fence (it would drain the prefetches).
//   * Causal / sequence-end masking runs only on the few stages that straddle the diagonal
//     or the sequence end: the stage loop is split into segments that call a masked or an
//     unmasked instantiation of the step (no per-element selects in the steady state, and
//     no branch merge inside a loop, which would make the register allocator copy every
//     live accumulator).
//   * Forward softmax rescales the output accumulator only when the running max grows by
//     more than 2^8 (exact: numerator and denominator use the same reference max).
//   * dk/dv keep the lane's K and V rows in registers and read the step's LDS operands in
//     groups ahead of their MFMAs.  When the KV tiles are too few to fill the machine, each
//     wave of a workgroup streams its own interleaved query tiles through private LDS
//     buffers (no barriers in the main loop); the four partial dK/dV are added in wave
//     order at the end.
//   * Blocks of one KV head are mapped to one XCD (its L2), heaviest causal tiles first.
//   * With the QK-norm + RoPE prologue, its backward runs in the dq and dk stores: the
//     gradient tiles pass through LDS once more as fp32 rows and leave as the gradient
//     w.r.t. the raw rows, with one dgamma partial per workgroup.
#include <algorithm>
#include <type_traits>

#include "lds_copy.h"
#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {
namespace {

// Swizzled bf16 tile rows of HD elements (ROWB bytes): physical 16-byte chunk =
// logical chunk ^ swz(row).  For HD = 128 the 16 rows read together by one LDS phase of
// row reads land on 16 distinct chunk positions and the four rows of one transposing
// read phase on disjoint 64-byte windows; HD = 64 (two rows per 256-byte bank window) is
// arranged the same way.
template <int HD>
struct Lay {
  static constexpr int ROWB = 2 * HD;
  static constexpr int CPR = HD / 8;
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (HD == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  // Row reads: row R0 + lane%32 (R0 a multiple of 32), logical chunk 2c + lane/32 sits at
  // byte R0*ROWB + (a_lane ^ (c << 5)).
  __device__ static __forceinline__ uint32_t a_lane(int lane) {
    const int r = lane & 31, h = lane >> 5;
    return (uint32_t)(r * ROWB) | (uint32_t)((h ^ swz(r)) << 4);
  }
  // Transposing reads for the 8 k-slots (rows R0 + 16*c2 + 4h + {0..3} and +8 + {0..3})
  // of column 32*dt + lane%32: the two reads sit at R0*ROWB + 16*c2*ROWB + (t_lane ^
  // ((4*dt) << 4)) and R0*ROWB + (16*c2 + 8)*ROWB + (t_lane ^ ((4*dt ^ 2) << 4)).
  __device__ static __forceinline__ uint32_t t_lane(int lane) {
    const int g = lane >> 4, li = lane & 15, h = lane >> 5;
    const int r = 4 * h + (li >> 2);
    return (uint32_t)(r * ROWB) |
           (uint32_t)(((2 * (g & 1) + ((li & 3) >> 1)) ^ swz(r)) << 4) |
           (uint32_t)((li & 1) << 3);
  }
};

template <int HD>
__device__ __forceinline__ bf16x8 lds_a(lptr base, uint32_t al, int c) {
  return *(lds_cbf16x8_t*)(base + (al ^ (uint32_t)(c << 5)));
}

template <int HD>
__device__ __forceinline__ bf16x8 lds_t(lptr base, uint32_t tl, int c2, int dt) {
  constexpr int ROWB = Lay<HD>::ROWB;
  lptr p0 = base + 16 * c2 * ROWB + (tl ^ (uint32_t)((4 * dt) << 4));
  lptr p1 = base + (16 * c2 + 8) * ROWB + (tl ^ (uint32_t)(((4 * dt) ^ 2) << 4));
  const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// init + sum over hd of tile rows (base = row R0) with the lane's register fragment.  The
// softmax offsets (a running max, lse, D) enter as the accumulator's initial value, so the
// score tiles leave the matrix unit already shifted and no vector op per score is spent on
// them.
template <int HD>
__device__ __forceinline__ f32x16 contract_rows(lptr base, uint32_t al,
                                                const bf16x8 (&frag)[HD / 16],
                                                const f32x16& init) {
  f32x16 acc = init;
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) acc = mfma_bf16(lds_a<HD>(base, al, c), frag[c], acc);
  return acc;
}

__device__ __forceinline__ f32x16 splat16(float v) {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = v;
  return z;
}

// The register-resident side of the score product (Q in the forward and dq, K in dk/dv) is
// held pre-multiplied by log2(e)/sqrt(hd), rounded to bf16 once more: the score tiles then
// come out in the exponent's units (base 2) and need no scaling before exp2.
template <int HD>
__device__ __forceinline__ void scale_frag(bf16x8 (&frag)[HD / 16], float c) {
#pragma unroll
  for (int k = 0; k < HD / 16; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) frag[k][j] = (bf16)((float)frag[k][j] * c);
}

// The lane's row operands (rows R0 + lane%32, all hd) and transposed operands (the 8 k-slots
// of every 32-column block) of a 32-row tile, read into registers ahead of their MFMAs.
template <int HD>
__device__ __forceinline__ void rows_of(bf16x8 (&x)[HD / 16], lptr base, uint32_t al) {
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) x[c] = lds_a<HD>(base, al, c);
}
template <int HD>
__device__ __forceinline__ void tr_of(bf16x8 (&x)[2][HD / 32], lptr base, uint32_t tl) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) x[c2][dt] = lds_t<HD>(base, tl, c2, dt);
}

// acc[dt] += (tile rows R0..R0+31, transposed) x (two packed 8-slot operands)
template <int HD>
__device__ __forceinline__ void acc_tr(f32x16 (&acc)[HD / 32], lptr base, uint32_t tl,
                                       const bf16x8 (&pb)[2]) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
      acc[dt] = mfma_bf16(lds_t<HD>(base, tl, c2, dt), pb[c2], acc[dt]);
}

__device__ __forceinline__ void pack16(bf16x8 (&pb)[2], const float (&v)[16]) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[c2][j] = (bf16)v[8 * c2 + j];
}

// Max / sum of a value over lanes l and l ^ 32, the same in both lanes: one
// v_permlane32_swap (lanes 32..63 of the first operand trade places with lanes 0..31 of the
// second) instead of an LDS permute, so no LDS round trip and no lgkmcnt wait.  The sum adds
// the lower lane's value first in both halves.
__device__ __forceinline__ void swap_halves(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  lo = __builtin_bit_cast(float, (unsigned)r[0]);  // lane l: value of lane l & 31
  hi = __builtin_bit_cast(float, (unsigned)r[1]);  // lane l: value of lane l | 32
}
__device__ __forceinline__ float halves_max(float v) {
  float lo, hi;
  swap_halves(v, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float halves_sum(float v) {
  float lo, hi;
  swap_halves(v, lo, hi);
  return lo + hi;
}

template <int N>
__device__ __forceinline__ void stage_barrier() {
  wait_vm<N>();
  __builtin_amdgcn_s_barrier();
  lds_acquire();
}
template <int N>
__device__ __forceinline__ void stage_wait_private() {
  wait_vm<N>();
  lds_acquire();
}
// vmcnt wait that leaves the copies of `after` (0..MAXA) later tiles in flight, NL loads each
template <int MAXA, int NL>
__device__ __forceinline__ void wait_tiles_after(int after) {
  if constexpr (MAXA <= 0) {
    wait_vm<0>();
  } else {
    if (after >= MAXA) wait_vm<MAXA * NL>();
    else wait_tiles_after<MAXA - 1, NL>(after);
  }
}
// f(integral_constant<int, k>) for k = 0 .. N-1, in order
template <typename F, int... K>
__device__ __forceinline__ void for_each_buf(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}

__device__ __forceinline__ void dma4(void* dst, const float* gaddr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);  // uniform
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(gaddr)
      : "memory");
}

// Direct HBM -> LDS copy of ROWS rows of a [S, HD] bf16 matrix into a swizzled tile,
// shared by NW waves.  Each lane's byte offsets within the source rows are fixed; a tile
// that runs past the sequence end re-reads its last valid row (callers mask those rows).
template <int HD, int ROWS, int NW>
struct Dma {
  static constexpr int ROWB = 2 * HD;
  static constexpr int PER = ROWS * (HD / 8) / (64 * NW);
  static_assert(ROWS * (HD / 8) % (64 * NW) == 0, "tile must split into whole wave loads");
  uint32_t off[PER];
  __device__ __forceinline__ void init(int wv, int lane) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int p = (wv * PER + j) * 64 + lane;
      const int row = p / (HD / 8);
      const int c = (p % (HD / 8)) ^ Lay<HD>::swz(row);
      off[j] = (uint32_t)(row * ROWB + c * 16);
    }
  }
  // src: first row of the tile in global memory; nvalid: rows of it before the sequence
  // end (rows at or past it are filled with zeros)
  __device__ __forceinline__ void issue(char* tile, const char* src, int wv, int nvalid) const {
    dma16_rows<PER>(tile + wv * PER * 1024, src, (uint32_t)(min(nvalid, ROWS) * ROWB), off);
  }
};

// Row statistics of 32 query rows q0.. into LDS: -lse*log2(e) at [0,32), -D at [32,64) (as
// the dq kernel stores them); NW waves share the copy.
template <int NW>
__device__ __forceinline__ void dma_rowstats(float* dst, const float* lse2,
                                             const float* delta, int q0, int S, int wv,
                                             int lane) {
  constexpr int PER = 64 / NW;
  if (lane < PER) {
    const int e = wv * PER + lane;
    const int r = min(q0 + (e & 31), S - 1);
    dma4(dst + wv * PER, (e < 32 ? lse2 : delta) + r);
  }
}

template <int HD>
__device__ __forceinline__ void load_frag(bf16x8 (&frag)[HD / 16], const bf16* base, int row,
                                          int S, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) {
    bf16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (bf16)0.f;
    frag[c] = row < S ? *reinterpret_cast<const bf16x8*>(base + (size_t)row * HD + 16 * c + 8 * h)
                      : z;
  }
}

template <typename TO, int HD>
__device__ __forceinline__ void store_col(TO* dst, const f32x16 (&acc)[HD / 32], float mul,
                                          int h) {
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      if constexpr (sizeof(TO) == 4) {
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = acc[dt][4 * g + j] * mul;
        *reinterpret_cast<f32x4*>(dst + d) = o;
      } else {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (bf16)(acc[dt][4 * g + j] * mul);
        *reinterpret_cast<bf16x4*>(dst + d) = o;
      }
    }
}

// ---------------------------------------------------------------------------------------
// Prologue backward fused into the dq / dk stores (Mint documentation 5.4.4 and 5.5.2; the
// arithmetic of the standalone prologue backward).  The gradient w.r.t. the rotated,
// normalised rows never goes to HBM: the accumulator tiles (scaled) are written to LDS as
// fp32 rows, and each wave then walks rows in row-major order the way the standalone
// kernel does: HD/16 lanes per row, lane part p owning columns [8p, 8p+8) and the matching
// second-half columns (complete rotation pairs), 16-byte loads of x and stores of dx, and
// the row sum over the HD/16 lanes.  The dgamma terms of a workgroup's rows are summed in
// a fixed order into one partial slot per workgroup, reduced by a separate launch.
// ---------------------------------------------------------------------------------------
// LDS tile of fp32 rows of HD: row r, 16-byte chunk c at chunk position c ^ (r & 15)
// (the rows a b128 access phase touches fall on distinct bank groups).
template <int HD>
__device__ __forceinline__ f32x4* epi_chunk(float* tile, int r, int c) {
  return reinterpret_cast<f32x4*>(tile + r * HD + 4 * (c ^ (r & 15)));
}

// acc * mul (accumulator layout: row lane%32, column 32 dt + 8 g + 4 h + j) into tile rows
// 0..31.
template <int HD>
__device__ __forceinline__ void acc_to_tile(float* tile, const f32x16 (&acc)[HD / 32],
                                            float mul, int lane) {
  const int c32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = acc[dt][4 * g + j] * mul;
      *epi_chunk<HD>(tile, c32, 8 * dt + 2 * g + h) = o;
    }
}

// s_waitcnt lgkmcnt(0) + workgroup barrier + LDS acquire; outstanding global stores are
// not waited for.
__device__ __forceinline__ void lds_barrier() {
  wait_vm<63>();
  __builtin_amdgcn_s_barrier();
  lds_acquire();
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each group of LPR (4 or 8) consecutive lanes, the same value in every lane of the
// group: DPP xor-1 and xor-2 quad permutations, then (LPR = 8) the mirrored lane of the
// half-row, which lies in the other quad.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f32<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  if constexpr (LPR == 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  static_assert(LPR == 4 || LPR == 8, "row group of 4 or 8 lanes");
  return v;
}

// Global inputs of the prologue backward of rows r0 .. r0 + NROWS - 1 (positions t0 + r of
// the head whose rows start at head_row0): gamma, rstd, the raw rows x and their cos / sin
// entries.  Nothing in the attention kernels writes these arrays, so the loads may be
// issued before the epilogue's barriers and reductions and stay in flight across them.
template <int HD, int NROWS>
struct ProRowsIn {
  static constexpr int HALF = HD / 2, LPR = HD / 16, RPI = 64 / LPR, NIT = NROWS / RPI;
  static_assert(NROWS % RPI == 0, "whole row passes");
  float g[16];
  float rr[NIT];
  bf16x8 x1[NIT], x2[NIT];
  f32x4 cs[NIT][2], sn[NIT][2];

  __device__ __forceinline__ void load(const ProBwd& pb, size_t head_row0, int r0, int t0,
                                       int S, int lane) {
    const int c1 = 8 * (lane % LPR), slot = lane / LPR;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g[e] = pb.gamma[c1 + e];
      g[8 + e] = pb.gamma[HALF + c1 + e];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int t = t0 + r0 + it * RPI + slot;
      const int tc = t < S ? t : S - 1;
      const size_t row = head_row0 + tc;
      rr[it] = pb.rstd[row];
      x1[it] = *reinterpret_cast<const bf16x8*>(pb.x + row * HD + c1);
      x2[it] = *reinterpret_cast<const bf16x8*>(pb.x + row * HD + HALF + c1);
      const float* cr = pb.cos_tab + (size_t)tc * HALF + c1;
      const float* sr = pb.sin_tab + (size_t)tc * HALF + c1;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        cs[it][u] = *reinterpret_cast<const f32x4*>(cr + 4 * u);
        sn[it][u] = *reinterpret_cast<const f32x4*>(sr + 4 * u);
      }
    }
  }
};

// Prologue backward of tile rows r0 .. r0 + NROWS - 1, the gradient w.r.t. y at positions
// t0 + r, with the rows' global inputs already loaded (`in`, same r0 and t0); writes dx
// rows into dx_head + t * HD and adds the lane's dgamma terms (its 16 columns) into dg.
// Rows t >= S store and contribute nothing.
template <int HD, int NROWS>
__device__ __forceinline__ void pro_rows(const ProRowsIn<HD, NROWS>& in, float* tile, int r0,
                                         bf16* __restrict__ dx_head, int t0, int S, int lane,
                                         float (&dg)[16]) {
  using In = ProRowsIn<HD, NROWS>;
  constexpr int HALF = In::HALF, LPR = In::LPR, RPI = In::RPI, NIT = In::NIT;
  const int c1 = 8 * (lane % LPR), slot = lane / LPR;
  f32x4 d1[NIT][2], d2[NIT][2];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + it * RPI + slot;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      d1[it][u] = *epi_chunk<HD>(tile, r, c1 / 4 + u);
      d2[it][u] = *epi_chunk<HD>(tile, r, (HALF + c1) / 4 + u);
    }
  }
  bf16x8 o1[NIT], o2[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const bool valid = t0 + r0 + it * RPI + slot < S;
    float n[16], xf[16];
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = d1[it][e / 4][e % 4], b = d2[it][e / 4][e % 4];
      const float c = in.cs[it][e / 4][e % 4], sv = in.sn[it][e / 4][e % 4];
      n[e] = a * c + b * sv;  // rotation by the negative angle
      n[8 + e] = b * c - a * sv;
      xf[e] = (float)in.x1[it][e];
      xf[8 + e] = (float)in.x2[it][e];
      dot += in.g[e] * n[e] * xf[e] + in.g[8 + e] * n[8 + e] * xf[8 + e];
    }
    dot = group_sum<LPR>(dot);
    const float r = in.rr[it];
    const float coef = dot * r * r * r * (1.0f / (float)HD);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o1[it][e] = (bf16)(in.g[e] * n[e] * r - xf[e] * coef);
      o2[it][e] = (bf16)(in.g[8 + e] * n[8 + e] * r - xf[8 + e] * coef);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) dg[e] += valid ? n[e] * xf[e] * r : 0.f;
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int t = t0 + r0 + it * RPI + slot;
    if (t < S) {
      *reinterpret_cast<bf16x8*>(dx_head + (size_t)t * HD + c1) = o1[it];
      *reinterpret_cast<bf16x8*>(dx_head + (size_t)t * HD + HALF + c1) = o2[it];
    }
  }
}

// Workgroup dgamma partial from the NW waves' dg: each wave sums its lanes' terms per
// column (halving over the row-slot lane bits) into red_w (HD floats of LDS only this wave
// uses until the barrier; wave w's at red0 + w * red_stride), then threads 0..HD-1 add the
// NW waves in wave order into partial slot `slot`.  Every thread of the workgroup calls.
template <int HD, int NW = 4>
__device__ __forceinline__ void pro_partial(float (&dg)[16], float* red0, int red_stride,
                                            const ProBwd& pb, int slot, int wv, int lane,
                                            int tid) {
  constexpr int HALF = HD / 2, LPR = HD / 16, PER = LPR / 4;  // columns per lane after sum
  halving_sum<16, 16, 32, LPR>(dg, lane);
  float* red = red0 + wv * red_stride;
  const int part = lane % LPR, slot_bits = lane / LPR;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int k = PER * slot_bits + e;  // index into the lane's 16 columns
    const int col = (k < 8 ? 0 : HALF - 8) + 8 * part + k;
    red[col] = dg[e];
  }
  lds_barrier();
  if (tid < HD) {
    float s = red0[tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red0[w * red_stride + tid];
    pb.partials[(size_t)tid * pb.nparts + slot] = s;
  }
}

// Block -> (query head, query tile) with the query tiles walked heaviest first and, when
// the KV rows split evenly over the 8 XCDs, the query heads of KV row kv placed on XCD
// kv % 8 (blocks are dispatched to XCDs round robin).
struct QMap {
  int bh, qt;
};
__device__ __forceinline__ QMap map_qblock(int lin, int BH, int H, int Hkv, int nqt, bool xcd) {
  const int group = H / Hkv;
  QMap m;
  if (xcd) {
    const int x = lin & 7, slot = lin >> 3;
    const int nh = BH / 8;  // query heads per XCD
    const int rank = slot / nh, hi = slot % nh;
    const int kv = x + 8 * (hi / group);
    m.bh = (kv / Hkv) * H + (kv % Hkv) * group + hi % group;
    m.qt = nqt - 1 - rank;
  } else {
    m.bh = lin % BH;
    m.qt = nqt - 1 - lin / BH;
  }
  return m;
}

__device__ __forceinline__ void map_kvblock(int lin, int BKV, bool xcd, int& kvbh, int& kt) {
  if (xcd) {
    const int x = lin & 7, slot = lin >> 3, per = BKV / 8;
    kt = slot / per;
    kvbh = x + 8 * (slot % per);
  } else {
    kvbh = lin % BKV;
    kt = lin / BKV;
  }
}

// Forward / dq workgroup: kQW waves of 32 queries.  Eight waves (256 queries) halve the
// K/V tile copies per query against four (each staged tile feeds twice the queries) at the
// same occupancy (two waves per SIMD, one workgroup per CU).
constexpr int kQW = 8;
constexpr int kBM = 32 * kQW;  // queries per forward / dq block
constexpr int kBN = 128;  // keys per stage

// ---------------------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------------------
// Index range test on a 32x32 score tile: accumulator i of a lane sits at tile index
// base + c(i), c(i) = 8 (i / 4) + i % 4, where base is the tile origin plus 4 for the upper
// half-wave.  keep(i) is lo <= base + c(i) <= hi, evaluated as the one unsigned compare
// c(i) - a <= span with a = lo - base, span = hi - lo; an empty range takes a = 64, which
// every c(i) < 32 wraps below.
struct TileRange {
  uint32_t a, span;
  __device__ __forceinline__ TileRange(int base, int lo, int hi) {
    const int a0 = lo - base, b0 = hi - base;
    a = b0 >= a0 ? (uint32_t)a0 : 64u;
    span = b0 >= a0 ? (uint32_t)(b0 - a0) : 0u;
  }
  __device__ __forceinline__ bool keep(int i) const {
    return (uint32_t)(8 * (i >> 2) + (i & 3)) - a <= span;
  }
};

// Stage kinds of the stage loops: plain (every score visible), diag (no documents, inside the
// sequence: only the causal diagonal sub-tile of a wave is masked, in place on the scores)
// and masked (document bounds, the ragged sequence end: every element is tested).
using PlainStage = std::integral_constant<int, 0>;
using MaskedStage = std::integral_constant<int, 1>;
using DiagStage = std::integral_constant<int, 2>;

// Causal mask of a 32x32 score tile on the diagonal (tile rows and lane columns start at
// the same index): with keys on the rows (query-major kernels) row r is hidden from lane
// column c when r > c; with queries on the rows (key-major kernels) when r < c.
template <bool KEYS_ON_ROWS>
__device__ __forceinline__ void diag_mask(f32x16& st, int lane) {
  const int c = lane & 31, h4 = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + h4 + (i & 3);
    if (KEYS_ON_ROWS ? r > c : r < c) st[i] = -INFINITY;
  }
}

// Online softmax of one 32-key sub-tile.  st holds the scores in base-2 units minus the
// lane's reference mref (the matrix unit started from -mref, held in nref); mref is the
// running max m, or 0 before the row has met a visible key (m = -inf).  The reference is
// raised only when a tile's max exceeds it by more than 2^8 (exact: numerator and
// denominator share the reference): then the output accumulator and the sum are rescaled,
// the tile's scores are shifted to the new reference and nref is rebuilt.  Gives the packed
// P^T operand of the P.V product.
// Masked sub-tiles also exclude keys before lo (the first row of the lane's document); a
// row can then meet a sub-tile with no visible key before its first one, so the masked
// instantiation keeps such a row empty (reference 0, max -inf).
struct SoftmaxState {
  float m, l, mref;
};

template <int HD, bool MASK>
__device__ __forceinline__ void fwd_softmax(f32x16 (&o)[HD / 32], SoftmaxState& sm,
                                            f32x16& nref, const f32x16& st, bf16x8 (&pb)[2],
                                            int kb, int qrow, int lo, int S, int h) {
  float sv[16];
  float tmax = -INFINITY;
  // keys lo .. min(qrow, S - 1) are visible
  const TileRange rg(kb + 4 * h, lo, min(qrow, S - 1));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = st[i];
    if (MASK && !rg.keep(i)) x = -INFINITY;
    sv[i] = x;
    tmax = fmaxf(tmax, x);
  }
  tmax = halves_max(tmax) + sm.mref;  // the tile's max in base-2 units
  if (__any(tmax > sm.m + 8.f)) {
    const float m_new = fmaxf(sm.m, tmax);
    const float alpha = (MASK && m_new == -INFINITY) ? 1.f : fast_exp2(sm.m - m_new);
    sm.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) o[dt] *= alpha;
    sm.m = m_new;
    const float mref = (MASK && m_new == -INFINITY) ? 0.f : m_new;
    const float shift = mref - sm.mref;
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] -= shift;
    sm.mref = mref;
    nref = splat16(-mref);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) sv[i] = fast_exp2(sv[i]);
  // pairwise sum (a short dependency chain)
  float ps[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ps[i] = sv[2 * i] + sv[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) ps[i] += ps[i + 4];
  sm.l += (ps[0] + ps[2]) + (ps[1] + ps[3]);
  pack16(pb, sv);
}

// One 32-key sub-tile: softmax, then O^T += V^T P^T.
template <int HD, bool MASK>
__device__ __forceinline__ void fwd_subtile(f32x16 (&o)[HD / 32], SoftmaxState& sm,
                                            f32x16& nref, const f32x16& st, lptr vsub,
                                            uint32_t tl, int kb, int qrow, int lo, int S,
                                            int h) {
  bf16x8 pb[2];
  fwd_softmax<HD, MASK>(o, sm, nref, st, pb, kb, qrow, lo, S, h);
  acc_tr<HD>(o, vsub, tl, pb);
}

// Document bounds of a query-major workgroup (Mint documentation 8.2, block-causal mask
// of packed documents: row i sees keys seg_lo[i] <= j <= i).  seg_lo is non-decreasing;
// without documents every bound is 0.  Values are clamped into the sequence, so a bad
// array gives wrong results but no access outside the tensors.
struct QDoc {
  int lo_row;   // first key of the lane's row
  int lo_wave;  // first key of the wave's first row (the wave's smallest)
  int t_first;  // first key stage any row of the workgroup sees
  int t_plain;  // first stage whose keys every row of the workgroup sees (below the diagonal)
};
__device__ __forceinline__ QDoc q_doc(const int* __restrict__ seg_lo, int q0, int qw0,
                                      int qrow, int S) {
  QDoc d{0, 0, 0, 0};
  if (seg_lo != nullptr) {
    auto at = [&](int i) { return min(max(seg_lo[min(i, S - 1)], 0), S - 1); };
    d.lo_row = at(qrow);
    d.lo_wave = __builtin_amdgcn_readfirstlane(at(qw0));
    d.t_first = __builtin_amdgcn_readfirstlane(at(q0)) / kBN;
    d.t_plain = (__builtin_amdgcn_readfirstlane(at(q0 + kBM - 1)) + kBN - 1) / kBN;
  }
  return d;
}

// Stage loop of a query-major workgroup over key stages [t_first, ntiles): stages that every
// row sees in full run `plain`, the rest (document starts, the diagonal, the ragged end)
// `masked`, except that without documents the diagonal stages that end inside the sequence
// run `diag`.
template <typename F>
__device__ __forceinline__ void q_stage_loop(const QDoc& doc, bool docs, int nplain, int ntiles,
                                             int S, F&& stage) {
  const int a = min(doc.t_plain, ntiles);
  for (int t = doc.t_first; t < a; ++t) stage(MaskedStage{}, t);
  for (int t = max(doc.t_plain, doc.t_first); t < nplain; ++t) stage(PlainStage{}, t);
  const int t3 = max(max(nplain, doc.t_plain), doc.t_first);
  const int d_end = docs ? t3 : max(t3, min(ntiles, S / kBN));
  for (int t = t3; t < d_end; ++t) stage(DiagStage{}, t);
  for (int t = d_end; t < ntiles; ++t) stage(MaskedStage{}, t);
}

// QK-norm + RoPE forward on the forward's resident Q rows (Mint documentation 5.4.1,
// 5.4.4 and 5.5.1; the arithmetic of the standalone prologue forward).  The lane's fragment
// (load_frag layout: chunk c holds columns 16 c + 8 h .. + 7) keeps both members of every
// rotation pair (chunks c and c + HD/32) and half of the row, so the mean square needs one
// exchange between the lane's halves.
struct ProFwd {
  const bf16* x;         // raw rows [rows, S, HD]
  const float* gamma;    // [HD]
  const float* cos_tab;  // [S, HD / 2]
  const float* sin_tab;  // [S, HD / 2]
  bf16* y;               // rotated rows [rows, S, HD] (output)
  float* rstd;           // [rows * S] (output)
  float eps;
};

// Loads the raw row at position t of the head whose rows start at row0 into the lane's
// fragment and replaces it with y = rotate(gamma * x * rstd) rounded to bf16; y and rstd are
// also stored when t < S (the fragment is zero past the sequence end).  Every load (x, cos,
// sin, gamma) is issued before the first use, so they share one memory round trip.
template <int HD>
__device__ __forceinline__ void qknorm_rope_frag(bf16x8 (&frag)[HD / 16], const ProFwd& pf,
                                                 size_t row0, int t, int S, int lane) {
  constexpr int NC = HD / 16, HC = NC / 2, HALF = HD / 2;
  const int h = lane >> 5;
  const bool valid = t < S;
  const int tc = valid ? t : S - 1;
  const bf16* xr = pf.x + (row0 + tc) * HD + 8 * h;
  const float* cr = pf.cos_tab + (size_t)tc * HALF;
  const float* sr = pf.sin_tab + (size_t)tc * HALF;
  f32x4 cs[HC][2], sn[HC][2], g1[HC][2], g2[HC][2];
#pragma unroll
  for (int c = 0; c < NC; ++c) frag[c] = *reinterpret_cast<const bf16x8*>(xr + 16 * c);
#pragma unroll
  for (int c = 0; c < HC; ++c)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = 16 * c + 8 * h + 4 * u;
      cs[c][u] = *reinterpret_cast<const f32x4*>(cr + f);
      sn[c][u] = *reinterpret_cast<const f32x4*>(sr + f);
      g1[c][u] = *reinterpret_cast<const f32x4*>(pf.gamma + f);
      g2[c][u] = *reinterpret_cast<const f32x4*>(pf.gamma + HALF + f);
    }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xv = (float)frag[c][j];
      ss += xv * xv;
    }
  ss = halves_sum(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / (float)HD) + pf.eps);
#pragma unroll
  for (int c = 0; c < HC; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = j / 4, e = j % 4;
      const float n1 = (float)frag[c][j] * r * g1[c][u][e];
      const float n2 = (float)frag[c + HC][j] * r * g2[c][u][e];
      const float y1 = n1 * cs[c][u][e] - n2 * sn[c][u][e];
      const float y2 = n1 * sn[c][u][e] + n2 * cs[c][u][e];
      frag[c][j] = (bf16)(valid ? y1 : 0.f);
      frag[c + HC][j] = (bf16)(valid ? y2 : 0.f);
    }
  if (valid) {
    bf16* yr = pf.y + (row0 + t) * HD + 8 * h;
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<bf16x8*>(yr + 16 * c) = frag[c];
    if (h == 0) pf.rstd[row0 + t] = r;
  }
}

template <int HD, int NBUF, bool PROQ>
__global__ __launch_bounds__(64 * kQW, 1) void fwd_kernel(const bf16* __restrict__ q,
                                                     const bf16* __restrict__ k,
                                                     const bf16* __restrict__ v,
                                                     bf16* __restrict__ out,
                                                     float* __restrict__ lse, int S, int H,
                                                     int Hkv, float scale_log2, int nqt,
                                                     int xcd, ProFwd pro,
                                                     const int* __restrict__ seg_lo) {
  constexpr int ROWB = 2 * HD;
  constexpr int TILEB = kBN * ROWB;
  using D = Dma<HD, kBN, kQW>;
  constexpr int NL = 2 * D::PER;  // loads per wave per stage
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * 2 * TILEB];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = gridDim.x / nqt;
  const QMap mp = map_qblock(blockIdx.x, BH, H, Hkv, nqt, xcd != 0);
  const int bh = mp.bh, b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const char* kp = reinterpret_cast<const char*>(k + (size_t)kvbh * S * HD);
  const char* vp = reinterpret_cast<const char*>(v + (size_t)kvbh * S * HD);
  const int q0 = mp.qt * kBM, qw0 = q0 + 32 * wv, qrow = qw0 + c32;
  const uint32_t al = Lay<HD>::a_lane(lane), tl = Lay<HD>::t_lane(lane);
  D dma;
  dma.init(wv, lane);

  const QDoc doc = q_doc(seg_lo, q0, qw0, qrow, S);
  const int t0 = doc.t_first;  // stages run from t0; buffers are numbered from it
  const int ntiles = (min(S, q0 + kBM) + kBN - 1) / kBN;
  auto issue = [&](int t, int buf) {
    const int g0 = t * kBN, nv = S - g0;
    dma.issue(lds + (2 * buf) * TILEB, kp + (size_t)g0 * ROWB, wv, nv);
    dma.issue(lds + (2 * buf + 1) * TILEB, vp + (size_t)g0 * ROWB, wv, nv);
  };
  bf16x8 qf[HD / 16];
  if constexpr (PROQ) {
    // the first tiles' copies are in flight while the Q rows are normalised and rotated
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u)
      if (t0 + u < ntiles) issue(t0 + u, u);
    qknorm_rope_frag<HD>(qf, pro, (size_t)bh * S, qrow, S, lane);
  } else {
    load_frag<HD>(qf, q + (size_t)bh * S * HD, qrow, S, lane);
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u)
      if (t0 + u < ntiles) issue(t0 + u, u);
  }
  scale_frag<HD>(qf, scale_log2);
  f32x16 o[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) o[dt] = zero16();
  SoftmaxState sm{-INFINITY, 0.f, 0.f};
  f32x16 nref = zero16();  // -mref in every accumulator slot
  // Stage t: wait for its tile, prefetch stage t + NBUF - 1, then compute.  Stages below
  // nplain lie strictly before the block's first query and inside the sequence, and (with
  // documents) at or after every row's document start, so no wave needs masking there; the
  // few remaining stages run the masked instantiation.
  auto stage = [&](auto kind, int t) {
    constexpr int KIND = decltype(kind)::value;
    constexpr bool MASK = KIND == MaskedStage::value, DIAG = KIND == DiagStage::value;
    if (NBUF > 2 && t + 1 < ntiles) stage_barrier<(NBUF > 2 ? NL : 0)>();
    else stage_barrier<0>();
    if (t + NBUF - 1 < ntiles) issue(t + NBUF - 1, (t - t0 + NBUF - 1) % NBUF);
    const int bb = (t - t0) % NBUF;
    const lptr ks = to_lds(lds) + (2 * bb) * TILEB;
    const lptr vs = ks + TILEB;
#pragma unroll
    for (int s = 0; s < kBN / 32; ++s) {
      const int kb = t * kBN + 32 * s;
      if ((MASK || DIAG) && (kb > qw0 + 31 || kb >= S)) break;  // wave-uniform
      if (MASK && kb + 31 < doc.lo_wave) continue;              // before every row's document
      f32x16 st = contract_rows<HD>(ks + 32 * s * ROWB, al, qf, nref);
      if (DIAG && kb == qw0) diag_mask<true>(st, lane);
      fwd_subtile<HD, MASK>(o, sm, nref, st, vs + 32 * s * ROWB, tl, kb, qrow, doc.lo_row, S,
                            h);
    }
  };
  q_stage_loop(doc, seg_lo != nullptr, min(q0 / kBN, S / kBN), ntiles, S, stage);
  const float l = halves_sum(sm.l);
  if (qrow < S) {
    store_col<bf16, HD>(out + ((size_t)bh * S + qrow) * HD, o, 1.0f / l, h);
    if (h == 0) lse[(size_t)bh * S + qrow] = (sm.m + log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------------
// backward, dq (+ per-query -D = -dO . out and -lse * log2(e) for the dk/dv kernel)
// ---------------------------------------------------------------------------------------
// At hd 128, st = S - lse (base-2 units) and dpt = dP - D come out of the matrix unit (the
// offsets are the accumulators' initial values, two 16-register tuples): P = exp2(st),
// dS = P * dpt.  At hd 64 the kernel runs four waves per SIMD and has no registers for the
// tuples: the offsets lse2 and D are subtracted here.
constexpr bool dq_offset_tuples(int hd) { return hd == 128; }

template <int HD, bool MASK>
__device__ __forceinline__ void dq_subtile(f32x16 (&acc)[HD / 32], const f32x16& st,
                                           const f32x16& dpt, lptr ksub, uint32_t tl,
                                           int kb, int qrow, int lo, int S, int h, float lse2,
                                           float D) {
  constexpr bool TUP = dq_offset_tuples(HD);
  float dsv[16];
  const TileRange rg(kb + 4 * h, lo, min(qrow, S - 1));  // visible keys
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float p = fast_exp2(TUP ? st[i] : st[i] - lse2);
    if (MASK && !rg.keep(i)) p = 0.f;
    dsv[i] = p * (TUP ? dpt[i] : dpt[i] - D);
  }
  bf16x8 db[2];
  pack16(db, dsv);
  acc_tr<HD>(acc, ksub, tl, db);  // dQ^T += K^T dS^T
}

template <int HD, int NBUF, bool PRO>
__global__ __launch_bounds__(64 * kQW, HD == 64 ? 4 : 1) void dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ out, const bf16* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ lse2_out, float* __restrict__ delta, bf16* __restrict__ dq, int S, int H,
    int Hkv, float scale_log2, float scale, int nqt, int xcd, ProBwd pro,
    const int* __restrict__ seg_lo) {
  constexpr int ROWB = 2 * HD;
  constexpr int TILEB = kBN * ROWB;
  using D = Dma<HD, kBN, kQW>;
  constexpr int NL = 2 * D::PER;
  // staged K/V tiles; with the prologue also each wave's fp32 dq tile in the epilogue
  constexpr int EPIB = PRO ? kQW * 32 * HD * (int)sizeof(float) : 0;
  __shared__ __attribute__((aligned(1024))) char lds[std::max(NBUF * 2 * TILEB, EPIB)];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = gridDim.x / nqt;
  const QMap mp = map_qblock(blockIdx.x, BH, H, Hkv, nqt, xcd != 0);
  const int bh = mp.bh, b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const char* kp = reinterpret_cast<const char*>(k + (size_t)kvbh * S * HD);
  const char* vp = reinterpret_cast<const char*>(v + (size_t)kvbh * S * HD);
  const int q0 = mp.qt * kBM, qw0 = q0 + 32 * wv, qrow = qw0 + c32;
  const size_t hoff = (size_t)bh * S * HD;
  uint32_t al = Lay<HD>::a_lane(lane), tl = Lay<HD>::t_lane(lane);
  D dma;
  dma.init(wv, lane);

  const QDoc doc = q_doc(seg_lo, q0, qw0, qrow, S);
  const int t0 = doc.t_first;  // stages run from t0; buffers are numbered from it
  const int ntiles = (min(S, q0 + kBM) + kBN - 1) / kBN;
  auto issue = [&](int t, int buf) {
    const int g0 = t * kBN, nv = S - g0;
    dma.issue(lds + (2 * buf) * TILEB, kp + (size_t)g0 * ROWB, wv, nv);
    dma.issue(lds + (2 * buf + 1) * TILEB, vp + (size_t)g0 * ROWB, wv, nv);
  };
  // the first tiles' copies are in flight while the row operands load and delta is formed
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u)
    if (t0 + u < ntiles) issue(t0 + u, u);
  bf16x8 qf[HD / 16], df[HD / 16];
  load_frag<HD>(qf, q + hoff, qrow, S, lane);
  load_frag<HD>(df, dout + hoff, qrow, S, lane);
  float dsum = 0.f;
  {
    bf16x8 of[HD / 16];
    load_frag<HD>(of, out + hoff, qrow, S, lane);
#pragma unroll
    for (int c = 0; c < HD / 16; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += (float)df[c][j] * (float)of[c][j];
  }
  const float Dq = halves_sum(dsum);
  const float lse2 = qrow < S ? lse[(size_t)bh * S + qrow] * kLog2e : 0.f;
  // the dk/dv kernel takes -D and -lse*log2(e) as accumulator initial values
  if (qrow < S && h == 0) {
    delta[(size_t)bh * S + qrow] = -Dq;
    lse2_out[(size_t)bh * S + qrow] = -lse2;
  }
  scale_frag<HD>(qf, scale_log2);
  constexpr bool TUP = dq_offset_tuples(HD);
  const f32x16 nl2 = TUP ? splat16(-lse2) : zero16(), nd = TUP ? splat16(-Dq) : zero16();
  f32x16 acc[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) acc[dt] = zero16();

  auto stage = [&](auto kind, int t) {
    constexpr int KIND = decltype(kind)::value;
    constexpr bool MASK = KIND == MaskedStage::value, DIAG = KIND == DiagStage::value;
    if (NBUF > 2 && t + 1 < ntiles) stage_barrier<(NBUF > 2 ? NL : 0)>();
    else stage_barrier<0>();
    if (t + NBUF - 1 < ntiles) issue(t + NBUF - 1, (t - t0 + NBUF - 1) % NBUF);
    const int bb = (t - t0) % NBUF;
    const lptr ks = to_lds(lds) + (2 * bb) * TILEB;
    const lptr vs = ks + TILEB;
#pragma unroll
    for (int s = 0; s < kBN / 32; ++s) {
      const int kb = t * kBN + 32 * s;
      if ((MASK || DIAG) && (kb > qw0 + 31 || kb >= S)) break;
      if (MASK && kb + 31 < doc.lo_wave) continue;  // before every row's document
      f32x16 st = contract_rows<HD>(ks + 32 * s * ROWB, al, qf, nl2);  // S^T (- lse)
      const f32x16 dpt = contract_rows<HD>(vs + 32 * s * ROWB, al, df, nd);  // dP^T (- D)
      if (DIAG && kb == qw0) diag_mask<true>(st, lane);
      dq_subtile<HD, MASK>(acc, st, dpt, ks + 32 * s * ROWB, tl, kb, qrow, doc.lo_row, S, h,
                           lse2, Dq);
    }
  };
  q_stage_loop(doc, seg_lo != nullptr, min(q0 / kBN, S / kBN), ntiles, S, stage);
  if constexpr (PRO) {
    static_assert(sizeof(lds) >= kQW * 32 * HD * sizeof(float), "epilogue tiles fit");
    ProRowsIn<HD, 32> pin;  // in flight across the barrier and the tile write
    pin.load(pro, (size_t)bh * S, 0, qw0, S, lane);
    lds_barrier();  // every wave is done with the staged tiles
    float* tile = reinterpret_cast<float*>(lds) + wv * 32 * HD;
    acc_to_tile<HD>(tile, acc, scale, lane);
    float dg[16] = {};
    pro_rows<HD, 32>(pin, tile, 0, dq + hoff, qw0, S, lane, dg);
    asm volatile("" ::: "memory");
    pro_partial<HD, kQW>(dg, reinterpret_cast<float*>(lds), 32 * HD, pro, bh * nqt + mp.qt, wv,
                         lane, tid);
  } else if (qrow < S) {
    store_col<bf16, HD>(dq + ((size_t)bh * S + qrow) * HD, acc, scale, h);
  }
}

// ---------------------------------------------------------------------------------------
// backward, dk/dv
// ---------------------------------------------------------------------------------------
constexpr int kBQ = 32;  // queries per dk/dv stage
constexpr int kDkdvPF = 1;  // operand read-ahead of the dk/dv step (see dkdv_step_reg)

// One 32x32 (queries x keys) step of the dk/dv recurrence on a staged Q / dO tile, with the
// lane's K and V rows in registers.  LDS operand reads are issued in groups ahead
// of the MFMAs that consume them, each group fenced off from the scheduler (which would
// otherwise sink every read next to its MFMA and expose the LDS latency each time).
// PF = 0: every read up front; 1: row operands up front, transposed ones after the S / dP
// chains are issued; 2: each group one phase ahead.
template <int HD, bool MASK, int PF>
__device__ __forceinline__ void dkdv_step_reg(f32x16 (&dkt)[HD / 32], f32x16 (&dvt)[HD / 32],
                                              lptr qs, lptr dos,
                                              const float* stats, const bf16x8 (&kf)[HD / 16],
                                              const bf16x8 (&vf)[HD / 16], uint32_t al,
                                              uint32_t tl, int q0, int key, int khi, int S,
                                              float scale_log2, int h, bool diag = false) {
  bf16x8 qa[HD / 16], da[HD / 16], ta[2][HD / 32], tq[2][HD / 32];
  auto read_rows = [&](bf16x8 (&x)[HD / 16], lptr base) {
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) x[c] = lds_a<HD>(base, al, c);
  };
  auto read_tr = [&](bf16x8 (&x)[2][HD / 32], lptr base) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) x[c2][dt] = lds_t<HD>(base, tl, c2, dt);
  };
  // -lse (base 2) and -D of the tile's queries, in accumulator layout: the initial values of
  // the S and dP products
  f32x16 st, dpt;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(stats + 8 * g + 4 * h);
    const f32x4 dd = *reinterpret_cast<const f32x4*>(stats + 32 + 8 * g + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st[4 * g + j] = l2[j];
      dpt[4 * g + j] = dd[j];
    }
  }
  read_rows(qa, qs);
  if constexpr (PF <= 1) read_rows(da, dos);
  if constexpr (PF == 0) {
    read_tr(ta, dos);
    read_tr(tq, qs);
  }
  __builtin_amdgcn_sched_barrier(0);
  // S - lse: queries x keys (the K rows are pre-scaled to base-2 units)
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) st = mfma_bf16(qa[c], kf[c], st);
  if constexpr (PF == 2) {
    read_rows(da, dos);
    __builtin_amdgcn_sched_barrier(0);
  }
  // dP - D
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) dpt = mfma_bf16(da[c], vf[c], dpt);
  if constexpr (PF >= 1) {
    read_tr(ta, dos);
    if constexpr (PF == 1) read_tr(tq, qs);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the query tile starts at the wave's first key (wave-uniform): the causal diagonal
  if (diag) diag_mask<false>(st, (int)(threadIdx.x & 63));
  float pv[16];
  const TileRange rg(q0 + 4 * h, key, min(khi, S - 1));  // queries that see the key
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float p = fast_exp2(st[i]);
    if (MASK && !rg.keep(i)) p = 0.f;
    pv[i] = p;
  }
  bf16x8 pb[2];
  pack16(pb, pv);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) dvt[dt] = mfma_bf16(ta[c2][dt], pb[c2], dvt[dt]);
  if constexpr (PF == 2) {
    read_tr(tq, qs);
    __builtin_amdgcn_sched_barrier(0);
  }
  float dsv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dsv[i] = pv[i] * dpt[i];
  bf16x8 db[2];
  pack16(db, dsv);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) dkt[dt] = mfma_bf16(tq[c2][dt], db[c2], dkt[dt]);
}

// Shared variant: 4 waves own 128 consecutive keys of one KV head and share each staged
// 32-query tile of every query head of the group.
// Document bounds of a key-major workgroup (block-causal mask of packed documents: key j
// is seen by queries j <= i <= seg_hi[j]).  seg_hi is non-decreasing; without documents
// every bound is S - 1.  Clamped into the sequence like QDoc.
struct KDoc {
  int hi_key;    // last query of the lane's key
  int hi_first;  // last query of the workgroup's (or wave's) first key: the smallest
  int hi_last;   // last query of its last key: the largest
};
__device__ __forceinline__ KDoc k_doc(const int* __restrict__ seg_hi, int k_first, int k_last,
                                      int key, int S) {
  KDoc d{S - 1, S - 1, S - 1};
  if (seg_hi != nullptr) {
    auto at = [&](int i) { return min(max(seg_hi[min(i, S - 1)], 0), S - 1); };
    d.hi_key = at(key);
    d.hi_first = __builtin_amdgcn_readfirstlane(at(k_first));
    d.hi_last = __builtin_amdgcn_readfirstlane(at(k_last));
  }
  return d;
}

template <int HD, int NBUF, bool PRO>
__global__ __launch_bounds__(256, HD == 64 ? 2 : 1) void dkdv_shared_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ dk, bf16* __restrict__ dv, int S, int H,
    int Hkv, float scale_log2, float scale, int nkt, int xcd, ProBwd pro,
    const int* __restrict__ seg_hi) {
  constexpr int ROWB = 2 * HD;
  constexpr int TILEB = kBQ * ROWB;
  using D = Dma<HD, kBQ, 4>;
  constexpr int NL = 2 * D::PER + 1;
  constexpr int EPIB = PRO ? 4 * 32 * HD * (int)sizeof(float) : 0;  // epilogue tiles
  __shared__ __attribute__((aligned(1024))) char lds[std::max(NBUF * 2 * TILEB, EPIB)];
  __shared__ __attribute__((aligned(16))) float stats[NBUF][64];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int kvbh, kt;
  map_kvblock(blockIdx.x, gridDim.x / nkt, xcd != 0, kvbh, kt);
  const int b = kvbh / Hkv, kvh = kvbh - b * Hkv, group = H / Hkv;
  const int k0 = kt * 128, kw0 = k0 + 32 * wv, key = kw0 + c32;
  const uint32_t al = Lay<HD>::a_lane(lane), tl = Lay<HD>::t_lane(lane);
  D dma;
  dma.init(wv, lane);
  bf16x8 kf[HD / 16], vf[HD / 16];
  load_frag<HD>(kf, k + (size_t)kvbh * S * HD, key, S, lane);
  load_frag<HD>(vf, v + (size_t)kvbh * S * HD, key, S, lane);
  scale_frag<HD>(kf, scale_log2);
  f32x16 dkt[HD / 32], dvt[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) dkt[dt] = dvt[dt] = zero16();

  const KDoc doc = k_doc(seg_hi, k0, k0 + 127, key, S);
  const int hi_wave = __builtin_amdgcn_readfirstlane(
      seg_hi != nullptr ? min(max(seg_hi[min(kw0 + 31, S - 1)], 0), S - 1) : S - 1);
  const int qt_first = k0 / kBQ, nqt = (S + kBQ - 1) / kBQ;
  // query tiles up to the last query of the workgroup's last key
  const int per_r = max(0, min(nqt, doc.hi_last / kBQ + 1) - qt_first);
  const int nst = group * per_r;
  // tiles are issued in stage order (query head r, tile i of it); the cursor avoids a
  // division per stage
  int next_r = 0, next_i = 0;
  auto issue_next = [&](int buf) {
    const size_t bh = (size_t)(b * H + kvh * group + next_r);
    const int g0 = (qt_first + next_i) * kBQ, nv = S - g0;
    dma.issue(lds + (2 * buf) * TILEB, reinterpret_cast<const char*>(q + (bh * S + g0) * HD),
              wv, nv);
    dma.issue(lds + (2 * buf + 1) * TILEB,
              reinterpret_cast<const char*>(dout + (bh * S + g0) * HD), wv, nv);
    dma_rowstats<4>(stats[buf], lse2 + bh * S, delta + bh * S, g0, S, wv, lane);
    if (++next_i == per_r) {
      next_i = 0;
      ++next_r;
    }
  };
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < nst) issue_next(t);
  const bool live = kw0 < S;
  // Stage t = (query head, tile i of it) in buffer t % NBUF; BUF >= 0 gives that buffer as a
  // constant (the plain stages are unrolled by NBUF), so every LDS address of the stage is a
  // lane constant plus an immediate offset.
  auto stage = [&](auto kind, int t, int i, auto buf) {
    constexpr int KIND = decltype(kind)::value, BUF = decltype(buf)::value;
    constexpr bool MASK = KIND == MaskedStage::value, DIAG = KIND == DiagStage::value;
    // tile t has landed once at most the copies of the tiles after it are in flight
    wait_tiles_after<NBUF - 2, NL>(min(NBUF - 2, nst - 1 - t));
    __builtin_amdgcn_s_barrier();
    lds_acquire();
    const int bb = BUF >= 0 ? BUF : t % NBUF;
    if (t + NBUF - 1 < nst) issue_next(BUF >= 0 ? (BUF + NBUF - 1) % NBUF : (t + NBUF - 1) % NBUF);
    const int q0 = (qt_first + i) * kBQ;
    if (live && q0 + kBQ - 1 >= kw0 && q0 <= hi_wave) {
      dkdv_step_reg<HD, MASK, kDkdvPF>(dkt, dvt, to_lds(lds) + (2 * bb) * TILEB,
                                       to_lds(lds) + (2 * bb + 1) * TILEB, stats[bb], kf, vf, al,
                                       tl, q0, key, doc.hi_key, S, scale_log2, h,
                                       DIAG && q0 == kw0);
    }
  };
  // Per query head: the first four query tiles straddle the diagonal of some wave's keys
  // (without documents and inside the sequence, only each wave's diagonal tile is masked:
  // diag stages); tiles reaching past the first key's last query (a document end, or the
  // ragged end of the sequence) need masking too; the rest need none.
  const int nmask_head = min(4, per_r);
  const int ndiag_head = seg_hi != nullptr ? 0 : min(nmask_head, (S - k0) / kBQ);
  const int plain_end = max(nmask_head, min(per_r, (doc.hi_first + 1) / kBQ - qt_first));
  using Any = std::integral_constant<int, -1>;
  for (int r = 0; r < group; ++r) {
    const int t0 = r * per_r;
    for (int i = 0; i < ndiag_head; ++i) stage(DiagStage{}, t0 + i, i, Any{});
    for (int i = ndiag_head; i < nmask_head; ++i) stage(MaskedStage{}, t0 + i, i, Any{});
    int i = nmask_head;
    for (; i < plain_end && (t0 + i) % NBUF != 0; ++i) stage(PlainStage{}, t0 + i, i, Any{});
    for (; i + NBUF <= plain_end; i += NBUF)
      for_each_buf([&](auto buf) {
        constexpr int k = decltype(buf)::value;
        stage(PlainStage{}, t0 + i + k, i + k, buf);
      }, std::make_integer_sequence<int, NBUF>{});
    for (; i < plain_end; ++i) stage(PlainStage{}, t0 + i, i, Any{});
    for (i = plain_end; i < per_r; ++i) stage(MaskedStage{}, t0 + i, i, Any{});
  }
  if (key < S) store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
  if constexpr (PRO) {
    lds_barrier();  // every wave is done with the staged tiles
    float* tile = reinterpret_cast<float*>(lds) + wv * 32 * HD;
    float dg[16] = {};
    if (kw0 < S) {
      acc_to_tile<HD>(tile, dkt, scale, lane);
      ProRowsIn<HD, 32> pin;
      pin.load(pro, (size_t)kvbh * S, 0, kw0, S, lane);
      pro_rows<HD, 32>(pin, tile, 0, dk + (size_t)kvbh * S * HD, kw0, S, lane, dg);
    }
    asm volatile("" ::: "memory");
    pro_partial<HD>(dg, reinterpret_cast<float*>(lds), 32 * HD, pro, kvbh * nkt + kt, wv, lane,
                    tid);
  } else if (key < S) {
    store_col<bf16, HD>(dk + ((size_t)kvbh * S + key) * HD, dkt, scale, h);
  }
}

// Private variant: 4 waves own the same 32 keys of one KV head; wave w walks query tiles
// w, w+4, w+8, ... (of every query head of the group, r ascending) through its own LDS
// buffers, so the main loop needs no barrier.  Partials are added in wave order.
template <int HD, int NBUF, bool PRO>
__global__ __launch_bounds__(256, HD == 64 ? 2 : 1) void dkdv_private_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ dk, bf16* __restrict__ dv, int S, int H,
    int Hkv, float scale_log2, float scale, int nkt, int xcd, ProBwd pro,
    const int* __restrict__ seg_hi) {
  constexpr int ROWB = 2 * HD;
  constexpr int TILEB = kBQ * ROWB;
  constexpr int WAVEB = NBUF * 2 * TILEB;  // one wave's staging bytes
  using D = Dma<HD, kBQ, 1>;
  constexpr int NL = 2 * D::PER + 1;
  __shared__ __attribute__((aligned(1024))) char lds[4 * WAVEB];
  __shared__ __attribute__((aligned(16))) float stats[4][NBUF][64];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int kvbh, kt;
  map_kvblock(blockIdx.x, gridDim.x / nkt, xcd != 0, kvbh, kt);
  const int b = kvbh / Hkv, kvh = kvbh - b * Hkv, group = H / Hkv;
  const int kw0 = kt * 32, key = kw0 + c32;
  const uint32_t al = Lay<HD>::a_lane(lane), tl = Lay<HD>::t_lane(lane);
  D dma;
  dma.init(0, lane);
  char* mine = lds + wv * WAVEB;
  const lptr lmine = to_lds(mine);
  bf16x8 kf[HD / 16], vf[HD / 16];  // K and V rows of the lane's key
  load_frag<HD>(kf, k + (size_t)kvbh * S * HD, key, S, lane);
  load_frag<HD>(vf, v + (size_t)kvbh * S * HD, key, S, lane);
  scale_frag<HD>(kf, scale_log2);
  f32x16 dkt[HD / 32], dvt[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) dkt[dt] = dvt[dt] = zero16();

  const KDoc doc = k_doc(seg_hi, kw0, kw0 + 31, key, S);
  const int qt_first = kw0 / kBQ;
  // query tiles up to the last query of the workgroup's last key
  const int qt_end = min((S + kBQ - 1) / kBQ, doc.hi_last / kBQ + 1);
  const int per_r = max(0, (qt_end - qt_first - wv + 3) / 4);  // this wave's tiles per head
  const int nst = group * per_r;
  // tiles are issued in order: (query head r, this wave's i-th tile of it); the cursor
  // avoids a division per stage
  int next_r = 0, next_i = 0, issued = 0;
  const size_t bh0 = (size_t)(b * H + kvh * group);
  auto issue_next = [&](int buf) {
    const size_t bh = bh0 + next_r;
    const int g0 = (qt_first + wv + 4 * next_i) * kBQ, nv = S - g0;
    dma.issue(mine + (2 * buf) * TILEB, reinterpret_cast<const char*>(q + (bh * S + g0) * HD),
                  0, nv);
    dma.issue(mine + (2 * buf + 1) * TILEB,
                  reinterpret_cast<const char*>(dout + (bh * S + g0) * HD), 0, nv);
    dma_rowstats<1>(stats[wv][buf], lse2 + bh * S, delta + bh * S, g0, S, 0, lane);
    if (++next_i == per_r) {
      next_i = 0;
      ++next_r;
    }
    ++issued;
  };
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (issued < nst) issue_next(t);
  wait_vm<0>();  // the first stage has landed
  __builtin_amdgcn_s_barrier();
  lds_acquire();
  // stage t = (head r, tile i of this wave in it)
  auto stage = [&](auto mask_tag, int t, int i) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (NBUF > 2 && t + 1 < nst) stage_wait_private<(NBUF > 2 ? NL : 0)>();
    else stage_wait_private<0>();
    if (issued < nst) issue_next((t + NBUF - 1) % NBUF);
    const int bb = t % NBUF;
    const int q0 = (qt_first + wv + 4 * i) * kBQ;
    dkdv_step_reg<HD, MASK, kDkdvPF>(dkt, dvt, lmine + (2 * bb) * TILEB,
                                     lmine + (2 * bb + 1) * TILEB, stats[wv][bb], kf, vf, al, tl,
                                     q0, key, doc.hi_key, S, scale_log2, h);
  };
  // Per query head: only wave 0's first tile meets the diagonal (its keys start at its
  // first query); tiles reaching past the first key's last query (a document end, or the
  // ragged end of the sequence) need masking too: a suffix of the wave's tiles.
  if (per_r > 0) {
    const int first_mask = (wv == 0) ? 1 : 0;
    const int qt_plain_end = (doc.hi_first + 1) / kBQ;  // tiles below it end by hi_first
    const int i_mask = max(first_mask, min(per_r, (qt_plain_end - qt_first - wv + 3) / 4));
    for (int r = 0; r < group; ++r) {
      const int t0 = r * per_r;
      if (first_mask) stage(std::true_type{}, t0, 0);
      for (int i = first_mask; i < i_mask; ++i) stage(std::false_type{}, t0 + i, i);
      for (int i = i_mask; i < per_r; ++i) stage(std::true_type{}, t0 + i, i);
    }
  }

  // wave-ordered combination of the four partials, one 32-row tile of one tensor at a time
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) {
      __syncthreads();
      if (wv > 0) {
        float* slot = red + ((wv - 1) * 64 + lane) * 16;
        const f32x16& src = which == 0 ? dkt[dt] : dvt[dt];
#pragma unroll
        for (int i = 0; i < 16; ++i) slot[i] = src[i];
      }
      __syncthreads();
      if (wv == 0) {
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) {
          const float* slot = red + ((w2 - 1) * 64 + lane) * 16;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (which == 0) dkt[dt][i] += slot[i];
            else dvt[dt][i] += slot[i];
          }
        }
      }
    }
  }
  if constexpr (PRO) {
    // wave 0 holds the sums; the prologue backward of the 32 rows is shared by the waves
    constexpr int TILE_AT = 16384, RED_AT = 32768;  // clear of the combination slots
    static_assert(sizeof(lds) >= RED_AT + 4 * HD * sizeof(float), "epilogue fits");
    float* tile = reinterpret_cast<float*>(lds + TILE_AT);
    if (wv == 0) {
      acc_to_tile<HD>(tile, dkt, scale, lane);
      if (key < S) store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
    }
    lds_barrier();
    constexpr int RPW = 64 / (HD / 16);  // rows per wave: one row-major pass
    float dg[16] = {};
    if (wv * RPW < 32) {
      ProRowsIn<HD, RPW> pin;
      pin.load(pro, (size_t)kvbh * S, wv * RPW, kw0, S, lane);
      pro_rows<HD, RPW>(pin, tile, wv * RPW, dk + (size_t)kvbh * S * HD, kw0, S, lane, dg);
    }
    pro_partial<HD>(dg, reinterpret_cast<float*>(lds + RED_AT), HD, pro, kvbh * nkt + kt, wv,
                    lane, tid);
    return;
  }
  if (wv != 0) return;
  if (key < S) {
    store_col<bf16, HD>(dk + ((size_t)kvbh * S + key) * HD, dkt, scale, h);
    store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
  }
}

// ---------------------------------------------------------------------------------------
// dk/dv, software-pipelined variant (head_dim 128, one wave per SIMD).  A workgroup owns
// 64 keys of one KV head: wave w holds keys k0 + 32 (w & 1) .. + 31 in registers and walks
// the query tiles of stream w >> 1 (tiles k0/32 + s, + s + 2, ..., every query head of the
// group in turn); the two waves of a stream share each staged tile, so four tiles per
// stream stay resident.  Iteration t issues the S and dP products of tile t + 1 while the
// vector unit forms P and dS of tile t, then the dV and dK products of tile t: the matrix
// pipe always has independent work queued while the softmax arithmetic runs.  The two
// streams' partial dK / dV of the same keys are added in stream order at the end.
// ---------------------------------------------------------------------------------------
constexpr int kPipeBuf = 4;  // staged tiles per stream

template <int HD, bool PRO>
__global__ __launch_bounds__(256, 1) void dkdv_pipe_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16* __restrict__ dk, bf16* __restrict__ dv, int S, int H,
    int Hkv, float scale_log2, float scale, int nkt, int xcd, ProBwd pro,
    const int* __restrict__ seg_hi) {
  constexpr int NB = kPipeBuf;
  constexpr int ROWB = 2 * HD;
  constexpr int TILEB = kBQ * ROWB;
  constexpr int STREAMB = NB * 2 * TILEB;  // one stream's staging bytes
  using D = Dma<HD, kBQ, 2>;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STREAMB];
  __shared__ __attribute__((aligned(16))) float stats[2][NB][64];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wv & 1, st = wv >> 1;  // key half, query stream
  int kvbh, kt;
  map_kvblock(blockIdx.x, gridDim.x / nkt, xcd != 0, kvbh, kt);
  const int b = kvbh / Hkv, kvh = kvbh - b * Hkv, group = H / Hkv;
  const int k0 = kt * 64, kw0 = k0 + 32 * kb, key = kw0 + c32;
  const uint32_t al = Lay<HD>::a_lane(lane), tl = Lay<HD>::t_lane(lane);
  D dma;
  dma.init(kb, lane);
  char* mine = lds + st * STREAMB;
  const lptr lmine = to_lds(mine);
  float(*sst)[64] = stats[st];
  bf16x8 kf[HD / 16], vf[HD / 16];  // K and V rows of the lane's key
  load_frag<HD>(kf, k + (size_t)kvbh * S * HD, key, S, lane);
  load_frag<HD>(vf, v + (size_t)kvbh * S * HD, key, S, lane);
  f32x16 dkt[HD / 32], dvt[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) dkt[dt] = dvt[dt] = zero16();

  const KDoc doc = k_doc(seg_hi, k0, min(k0 + 63, S - 1), key, S);
  const int qt_first = k0 / kBQ;
  // query tiles up to the last query of the workgroup's last key, split over the streams;
  // both streams run the same count (a stream's extra tile is past every visible query)
  const int qt_end = min((S + kBQ - 1) / kBQ, doc.hi_last / kBQ + 1);
  const int per_r = max(0, (qt_end - qt_first + 1) / 2);
  const int nst = group * per_r;
  int next_r = 0, next_i = 0, issued = 0;
  const size_t bh0 = (size_t)(b * H + kvh * group);
  // Issues the next tile of the stream.  Past the last tile it issues an empty copy (no
  // bytes read; the free buffer it lands in is never read again), so the loop body needs
  // no branch.
  auto issue_next = [&]() {
    const int buf = issued % NB;
    const bool real = issued < nst;
    const size_t bh = bh0 + (real ? next_r : 0);
    // a stream's extra tile may start past the sequence: nothing is read for it either
    const int g0 = (qt_first + st + 2 * next_i) * kBQ, nv = real ? max(S - g0, 0) : 0;
    dma.issue(mine + (2 * buf) * TILEB, reinterpret_cast<const char*>(q + (bh * S + g0) * HD),
              kb, nv);
    dma.issue(mine + (2 * buf + 1) * TILEB,
              reinterpret_cast<const char*>(dout + (bh * S + g0) * HD), kb, nv);
    dma_rowstats<2>(sst[buf], lse2 + bh * S, delta + bh * S, g0, S, kb, lane);
    if (++next_i == per_r) {
      next_i = 0;
      ++next_r;
    }
    ++issued;
  };

  constexpr int NL = 2 * D::PER + 1;  // loads per wave per tile
  // The copy waits count tiles in flight: the prologue issues NB tiles and needs tiles 0
  // and 1 (NB - 2 may stay in flight); iteration t has issued tiles up to t + NB - 1 and
  // needs tile t + 2 (NB - 3 may stay in flight).  The loop reads tile t + 2 while tiles
  // t + 1 and t are still referenced, so at least three buffers are needed.
  static_assert(NB >= 3, "the pipelined dk/dv loop needs at least three staged tiles");
  constexpr int kWaitPrologue = (NB - 2) * NL, kWaitIter = (NB - 3) * NL;
  // prologue: tiles 0..NB-1 in flight; S and dP of tile 0; row operands of tile 1
  bf16x8 qa[HD / 16], da[HD / 16];
  f32x16 s_cur = zero16(), p_cur = zero16();
  if (nst > 0) {
#pragma unroll
    for (int u = 0; u < NB; ++u) issue_next();
    wait_vm<kWaitPrologue>();  // tiles 0 and 1
    __builtin_amdgcn_s_barrier();
    lds_acquire();
    rows_of<HD>(qa, lmine, al);
    rows_of<HD>(da, lmine + TILEB, al);
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      s_cur = mfma_bf16(qa[c], kf[c], s_cur);
      p_cur = mfma_bf16(da[c], vf[c], p_cur);
    }
    rows_of<HD>(qa, lmine + 2 * TILEB, al);
    rows_of<HD>(da, lmine + 3 * TILEB, al);
  }

  // Iteration t: P / dS of tile t under the S / dP products of tile t + 1, then tile t's
  // dV / dK products.  Tile t's buffer is free after the barrier (its last reads, the
  // transposed operands, are complete by then) and receives tile t + NB.
  auto iter = [&](auto mask_tag, int t, int i) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const lptr cur = lmine + (2 * (t % NB)) * TILEB;
    const float* stt = sst[t % NB];
    const int q0 = (qt_first + st + 2 * i) * kBQ;
    // -lse (base 2) and -D of tile t's queries; in this kernel the offsets are applied by
    // the vector unit (the pipelined schedule measured slower with them as the products'
    // initial values)
    f32x4 l2[4], dd[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l2[g] = *reinterpret_cast<const f32x4*>(stt + 8 * g + 4 * h);
      dd[g] = *reinterpret_cast<const f32x4*>(stt + 32 + 8 * g + 4 * h);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s_nxt = zero16(), p_nxt = zero16();
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      s_nxt = mfma_bf16(qa[c], kf[c], s_nxt);
      p_nxt = mfma_bf16(da[c], vf[c], p_nxt);
    }
    float pv[16], dsv[16];
    const TileRange rg(q0 + 4 * h, key, min(doc.hi_key, S - 1));  // queries that see the key
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = fast_exp2(s_cur[4 * g + j] * scale_log2 + l2[g][j]);
        if (MASK && !rg.keep(4 * g + j)) p = 0.f;
        pv[4 * g + j] = p;
        dsv[4 * g + j] = p * (p_cur[4 * g + j] + dd[g][j]);
      }
    bf16x8 pb[2], db[2];
    pack16(pb, pv);
    pack16(db, dsv);
    bf16x8 ta[2][HD / 32], tq[2][HD / 32];  // transposed operands of tile t
    tr_of<HD>(ta, cur + TILEB, tl);
    tr_of<HD>(tq, cur, tl);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA,
      __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);  // VALU / transcendental,
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
    }
    // P and dS are formed here, under the matrix products, not after the barrier
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(db[0]), "v"(db[1]));
    __builtin_amdgcn_sched_barrier(0);
    // tile t + 2 has landed for every wave (later tiles may still be in flight)
    wait_vm<kWaitIter>();
    __builtin_amdgcn_s_barrier();
    lds_acquire();
    issue_next();  // tile t + NB into tile t's buffer
    const lptr nx2 = lmine + (2 * ((t + 2) % NB)) * TILEB;
    rows_of<HD>(qa, nx2, al);
    rows_of<HD>(da, nx2 + TILEB, al);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) {
        dvt[dt] = mfma_bf16(ta[c2][dt], pb[c2], dvt[dt]);
        dkt[dt] = mfma_bf16(tq[c2][dt], db[c2], dkt[dt]);
      }
    s_cur = s_nxt;
    p_cur = p_nxt;
  };
  // Per query head: tile 0 of each stream meets the diagonal of one of the key halves;
  // tiles reaching past the first key's last query (a document end, the ragged end of the
  // sequence, a stream's extra tile) need masking too: a suffix of the stream's tiles.
  if (per_r > 0) {
    const int qt_plain_end = (doc.hi_first + 1) / kBQ;  // tiles below it end by hi_first
    const int i_mask = max(1, min(per_r, (qt_plain_end - qt_first - st + 1) / 2));
    for (int r = 0; r < group; ++r) {
      const int t0 = r * per_r;
      iter(std::true_type{}, t0, 0);
      for (int i = 1; i < i_mask; ++i) iter(std::false_type{}, t0 + i, i);
      for (int i = i_mask; i < per_r; ++i) iter(std::true_type{}, t0 + i, i);
    }
  }
  wait_vm<0>();

  // stream-ordered combination of the two partials of each key half: once every wave is done
  // with the staged tiles (and their copies have landed), stream 1 parks its dK / dV partials
  // in LDS as 16-byte slots, element-major (slot index, then lane: conflict-free), above the
  // epilogue tile; after one barrier stream 0 adds them to its own.
  {
    constexpr int NT = HD / 32, SLOTS = 2 * NT * 4;  // f32x4 slots per lane: dK then dV
    constexpr int RED_AT = 65536;
    static_assert(RED_AT + 2 * SLOTS * 64 * 16 <= (int)sizeof(lds), "partials fit");
    f32x4* red = reinterpret_cast<f32x4*>(lds + RED_AT) + kb * SLOTS * 64 + lane;
    __syncthreads();
    if (st == 1) {
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = which == 0 ? dkt[dt] : dvt[dt];
            red[((which * NT + dt) * 4 + q) * 64] =
                f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          }
    }
    __syncthreads();
    if (st == 0) {
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 b = red[((which * NT + dt) * 4 + q) * 64];
            f32x16& a = which == 0 ? dkt[dt] : dvt[dt];
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * q + e] += b[e];
          }
    }
  }
  if constexpr (PRO) {
    // stream 0 holds the sums; the prologue backward of the 64 rows is shared by the waves
    constexpr int TILE_AT = 16384, RED_AT = TILE_AT + 64 * HD * 4;
    static_assert(sizeof(lds) >= RED_AT + 4 * HD * sizeof(float), "epilogue fits");
    float* tile = reinterpret_cast<float*>(lds + TILE_AT);
    if (st == 0) {
      acc_to_tile<HD>(tile + kb * 32 * HD, dkt, scale, lane);
      if (key < S) store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
    }
    lds_barrier();
    constexpr int RPW = 64 / (HD / 16);  // rows per wave pass
    float dg[16] = {};
    ProRowsIn<HD, 2 * RPW> pin;
    pin.load(pro, (size_t)kvbh * S, wv * 2 * RPW, k0, S, lane);
    pro_rows<HD, 2 * RPW>(pin, tile, wv * 2 * RPW, dk + (size_t)kvbh * S * HD, k0, S, lane, dg);
    pro_partial<HD>(dg, reinterpret_cast<float*>(lds + RED_AT), HD, pro, kvbh * nkt + kt, wv,
                    lane, tid);
    return;
  }
  if (st != 0) return;
  if (key < S) {
    store_col<bf16, HD>(dk + ((size_t)kvbh * S + key) * HD, dkt, scale, h);
    store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
  }
}

constexpr int kFwdBuf = 2;
constexpr int kDqBuf = 2;
constexpr int kDkdvSharedBuf = 3;
constexpr int kDkdvPrivateBuf = 2;

template <int HD, bool PROQ>
hipError_t fwd_launch(const AttnShape& s, const void* q, const void* k, const void* v, void* out,
                      float* lse, const ProFwd& pro, hipStream_t stream) {
  const int nqt = (s.seq_len + kBM - 1) / kBM;
  const int BH = s.batch * s.num_heads;
  const int BKV = s.batch * s.num_kv_heads;
  const int xcd = (BKV % 8 == 0) ? 1 : 0;
  ProfScope prof("attn_fwd", stream);
  hipLaunchKernelGGL((fwd_kernel<HD, kFwdBuf, PROQ>), dim3(BH * nqt), dim3(64 * kQW), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)out, lse, s.seq_len,
                     s.num_heads, s.num_kv_heads, kLog2e / sqrtf((float)HD), nqt, xcd, pro,
                     s.seg_lo);
  return hipPeekAtLastError();
}

// dk/dv kernel choice: the shared-tile kernel when its 128-key workgroups fill the
// machine; else, at head_dim 128, the pipelined one (64 keys per workgroup), else the
// private one (32 keys per workgroup).
bool dkdv_shared(int BKV, int S) { return (long long)BKV * ((S + 127) / 128) >= 1024; }
int dkdv_keys_per_block(int BKV, int S, int HD) {
  if (dkdv_shared(BKV, S)) return 128;
  return HD == 128 ? 64 : 32;
}

template <int HD, bool PRO>
hipError_t bwd_launch(const AttnShape& s, const void* q, const void* k, const void* v,
                      const void* out, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* delta, float* lse2, const ProBwd& pq, const ProBwd& pk,
                      hipStream_t stream) {
  const int S = s.seq_len;
  const int nqt = (S + kBM - 1) / kBM;
  const int BH = s.batch * s.num_heads;
  const int BKV = s.batch * s.num_kv_heads;
  const int xcd = (BKV % 8 == 0) ? 1 : 0;
  const float scale = 1.0f / sqrtf((float)HD), sl2 = kLog2e * scale;
  {
    ProfScope prof("attn_bwd_dq", stream);
    hipLaunchKernelGGL((dq_kernel<HD, kDqBuf, PRO>), dim3(BH * nqt), dim3(64 * kQW), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)out,
                       (const bf16*)dout, lse, lse2, delta, (bf16*)dq, S, s.num_heads,
                       s.num_kv_heads, sl2, scale, nqt, xcd, pq, s.seg_lo);
  }
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  ProfScope prof("attn_bwd_dkdv", stream);
  if (dkdv_shared(BKV, S)) {
    const int nkt = (S + 127) / 128;
    hipLaunchKernelGGL((dkdv_shared_kernel<HD, kDkdvSharedBuf, PRO>), dim3(BKV * nkt),
                       dim3(256), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                       (const bf16*)dout, (const float*)lse2, (const float*)delta, (bf16*)dk,
                       (bf16*)dv, S, s.num_heads, s.num_kv_heads, sl2, scale, nkt, xcd, pk,
                       s.seg_hi);
  } else if constexpr (HD == 128) {  // 64 keys per workgroup
    const int nkt = (S + 63) / 64;
    hipLaunchKernelGGL((dkdv_pipe_kernel<HD, PRO>), dim3(BKV * nkt), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                       (const float*)lse2, (const float*)delta, (bf16*)dk, (bf16*)dv, S,
                       s.num_heads, s.num_kv_heads, sl2, scale, nkt, xcd, pk, s.seg_hi);
  } else {  // 32 keys per workgroup
    const int nkt = (S + 31) / 32;
    hipLaunchKernelGGL((dkdv_private_kernel<HD, kDkdvPrivateBuf, PRO>), dim3(BKV * nkt),
                       dim3(256), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                       (const bf16*)dout, (const float*)lse2, (const float*)delta, (bf16*)dk,
                       (bf16*)dv, S, s.num_heads, s.num_kv_heads, sl2, scale, nkt, xcd, pk,
                       s.seg_hi);
  }
  return hipPeekAtLastError();
}

ProBwd make_pro(const void* x, const float* gamma, const float* rstd, const float* cos_tab,
                const float* sin_tab, float* partials, int nparts) {
  ProBwd p;
  p.x = static_cast<const bf16*>(x);
  p.gamma = gamma, p.rstd = rstd, p.cos_tab = cos_tab, p.sin_tab = sin_tab;
  p.partials = partials;
  p.nparts = nparts;
  return p;
}

}  // namespace

bool fast_bf16_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_attn_fwd_bf16_fast(const AttnShape& s, const void* q, const void* k,
                                     const void* v, void* out, float* lse,
                                     const QProFuse* pro, hipStream_t stream) {
  ProFwd pf{};
  if (pro != nullptr) {
    pf.x = static_cast<const bf16*>(pro->xq);
    pf.gamma = pro->gamma_q, pf.cos_tab = pro->cos_tab, pf.sin_tab = pro->sin_tab;
    pf.y = static_cast<bf16*>(pro->yq);
    pf.rstd = pro->rstd_q;
    pf.eps = pro->eps;
  }
  if (s.head_dim == 128)
    return pro != nullptr ? fwd_launch<128, true>(s, q, k, v, out, lse, pf, stream)
                          : fwd_launch<128, false>(s, q, k, v, out, lse, pf, stream);
  if (s.head_dim == 64)
    return pro != nullptr ? fwd_launch<64, true>(s, q, k, v, out, lse, pf, stream)
                          : fwd_launch<64, false>(s, q, k, v, out, lse, pf, stream);
  return hipErrorInvalidValue;
}

// dgamma partial slots: one per dq workgroup (kBM queries), one per dk/dv workgroup
// (128 or 32 keys; the workspace is sized for 32).
int fused_pro_parts_q(int64_t q_heads, int seq_len) {
  return (int)(q_heads * ((seq_len + kBM - 1) / kBM));
}
int fused_pro_parts_k(int64_t kv_heads, int seq_len) {
  return (int)(kv_heads * ((seq_len + 31) / 32));
}

hipError_t launch_attn_bwd_bf16_fast(const AttnShape& s, const void* q, const void* k,
                                     const void* v, const void* out, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv,
                                     float* delta, float* lse2, const ProFuse* pro,
                                     hipStream_t stream) {
  ProBwd pq{}, pk{};
  if (pro != nullptr) {
    const int BKV = s.batch * s.num_kv_heads, S = s.seq_len;
    pq = make_pro(pro->xq, pro->gamma_q, pro->rstd_q, pro->cos_tab, pro->sin_tab,
                  pro->partials_q, fused_pro_parts_q(s.batch * s.num_heads, S));
    pk = make_pro(pro->xk, pro->gamma_k, pro->rstd_k, pro->cos_tab, pro->sin_tab,
                  pro->partials_k, BKV * ((S + dkdv_keys_per_block(BKV, S, s.head_dim) - 1) /
                                          dkdv_keys_per_block(BKV, S, s.head_dim)));
  }
#define XATTN_CASE(HD, PRO)                                                                \
  e = bwd_launch<HD, PRO>(s, q, k, v, out, lse, dout, dq, dk, dv, delta, lse2, pq, pk, stream);
  hipError_t e = hipErrorInvalidValue;
  if (s.head_dim == 128) {
    if (pro != nullptr) { XATTN_CASE(128, true) } else { XATTN_CASE(128, false) }
  } else if (s.head_dim == 64) {
    if (pro != nullptr) { XATTN_CASE(64, true) } else { XATTN_CASE(64, false) }
  }
#undef XATTN_CASE
  if (e != hipSuccess || pro == nullptr) return e;
  return launch_dgamma_reduce_qk(s.head_dim, pq.partials, pq.nparts, pro->dgamma_q,
                                 pk.partials, pk.nparts, pro->dgamma_k, stream);
}

}  // namespace xattn
