// Causal GQA attention, forward and backward, on gfx950 MFMA.
//
// What is computed (Mint documentation 5.3.1; xtrain "Phase T9: Export to xserv"
// conventions table; xtrain "Phase T15: GQA"):
//   s_ij = q_i . k_j / sqrt(hd) for j <= i (later keys excluded), p = softmax_j(s) in fp32,
//   out_i = sum_j p_ij v_j, lse_i = ln sum_j exp(s_ij); query head qh of batch b reads KV
//   head b*Hkv + qh/group.  The backward is the chain rule with D_i = dO_i . out_i:
//   dS = P (dP - D), dq = dS K / sqrt(hd), dk = sum_r dS^T Q / sqrt(hd), dv = sum_r P^T dO,
//   where r runs over the group's query heads, summed in ascending r with no atomics (by
//   the dk/dv tile's one owning workgroup, or, for the smallest grids, by a fixed-order sum
//   of per-workgroup partials over contiguous ranges of r).
//
// Design (MI355X-first, not a translation of the pages' CUDA kernels):
//   * Tiles of 32 x 32 on v_mfma_f32_32x32x16_bf16 (fp32 io: v_mfma_f32_32x32x2_f32).
//     A wave owns 32 rows of the "resident" side (queries in the forward and dq kernels,
//     keys in the dk/dv kernel); its operand fragments stay in registers for the whole
//     kernel, while the streamed side goes HBM -> LDS in 16-byte coalesced chunks.
//   * Products are arranged so the score tile comes out with the resident index on the
//     lane (column) axis: per-row softmax statistics are then per-lane scalars, the row
//     max needs a single cross-half exchange, and the probability tile can be fed back to
//     the next MFMA straight from the accumulator registers.
//   * The operand that must be contracted over the streamed index (V in P.V, K in dS.K,
//     Q and dO in the dk/dv products) is read from the row-major LDS tile with gfx950's
//     transposing LDS read, so no transposed copy is ever stored.
//   * Online softmax in the exp2 domain with log2(e)/sqrt(hd) folded into one multiply.
//   * Work order: the heaviest causal tiles are dispatched first.
#include <algorithm>
#include <type_traits>

#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {

template <typename T, int HD>
struct Tile {
  static constexpr int VEC = V16<T>::n;            // elements per 16-byte chunk
  static constexpr int HDP = HD < 32 ? 32 : HD;    // LDS row length, padded to one MFMA tile
  static constexpr int LDS_ROW = HDP + VEC;        // +16 bytes per row against bank conflicts
  static constexpr int NCH = HD / (2 * VEC);       // 16-byte chunks per lane in a hd-contraction
  static constexpr int NDT = HDP / 32;             // 32-row MFMA tiles along hd
  static constexpr int CPR = HDP / VEC;            // 16-byte chunks per padded row
  static constexpr bool kBf16 = std::is_same<T, bf16>::value;
};

__device__ __forceinline__ bf16x8 pack8_bf16(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)p[j];
  return r;
}

// A operand of a product contracted over the streamed (row) index of an LDS tile:
// rows kb..kb+3 and kb+8..kb+11 (kb = row0 + 16*c2 + 4*h), column d = col0 + c32, as the
// eight k-slots of this lane.  Matches the accumulator rows 8*(i/4) + 4*h + (i%4) for
// i in [8*c2, 8*c2 + 8), i.e. the probabilities this lane packs for the same MFMA.
template <int LDS_ROW>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int row0, int c2, int col0,
                                             int lane) {
  const int g = lane >> 4, li = lane & 15, h = lane >> 5;
  const int row = row0 + 16 * c2 + 4 * h + (li >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (li & 3);
  const bf16x4 lo = lds_read_tr16(tile + row * LDS_ROW + col);
  const bf16x4 hi = lds_read_tr16(tile + (row + 8) * LDS_ROW + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc[dt] += (tile rows row0..row0+31, transposed) x (probability-like values in the
// accumulator layout of the 32x32 score tile).
template <typename T, int HD, int NDT>
__device__ __forceinline__ void accumulate_transposed(f32x16 (&acc)[NDT], const T* tile,
                                                      int row0, const float (&pv)[16],
                                                      int lane) {
  using C = Tile<T, HD>;
  static_assert(NDT == C::NDT, "accumulator tiles must cover the padded head dim");
  if constexpr (C::kBf16) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const bf16x8 b = pack8_bf16(pv + 8 * c2);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const bf16x8 a = tr_operand<C::LDS_ROW>(tile, row0, c2, 32 * dt, lane);
        acc[dt] = mfma_bf16(a, b, acc[dt]);
      }
    }
  } else {
    const int c32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int r = row0 + 8 * (t >> 2) + 4 * h + (t & 3);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
        acc[dt] = mfma_f32(tile[r * C::LDS_ROW + 32 * dt + c32], pv[t], acc[dt]);
    }
  }
}

// Score-like tile: sum over hd of tile[row0 + c32][:] (A, from LDS) with the lane's
// register fragment (B).
template <typename T, int HD, int NCH>
__device__ __forceinline__ f32x16 contract_hd(const T* tile, int row0,
                                              const vec16_t<T> (&frag)[NCH], int lane) {
  using C = Tile<T, HD>;
  static_assert(NCH == C::NCH, "fragment must cover head_dim");
  const int c32 = lane & 31, h = lane >> 5;
  f32x16 acc = zero16();
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    const vec16_t<T> a = load16(tile + (row0 + c32) * C::LDS_ROW + 2 * C::VEC * c + C::VEC * h);
    acc = mfma_chunk(a, frag[c], acc);
  }
  return acc;
}

// Lane's register fragment of row `row` of a [S, HD] matrix (zero past the end).
template <typename T, int HD, int NCH>
__device__ __forceinline__ void load_fragment(vec16_t<T> (&frag)[NCH], const T* base, int row,
                                              int S, int h) {
  using C = Tile<T, HD>;
  static_assert(NCH == C::NCH, "fragment must cover head_dim");
#pragma unroll
  for (int c = 0; c < C::NCH; ++c)
    frag[c] = row < S ? load16(base + (size_t)row * HD + 2 * C::VEC * c + C::VEC * h)
                      : vzero<T>();
}

// Copy of rows r0..r0+ROWS-1 of a [S, HD] matrix into a zero-padded LDS tile, in two halves
// so that the next tile's global reads can be in flight while the current tile is used:
// load() brings the rows into the thread's registers (zero past the end and in the padding),
// store() writes them to the tile.  NTHR threads, t the thread's index.
template <typename T, int HD, int ROWS, int NTHR>
struct RowPrefetch {
  using C = Tile<T, HD>;
  static constexpr int CH = ROWS * C::CPR;            // 16-byte chunks of the tile
  static constexpr int N = (CH + NTHR - 1) / NTHR;    // per thread
  vec16_t<T> x[N];
  __device__ __forceinline__ void load(const T* src, int r0, int S, int t) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = t + j * NTHR;
      const int gr = r0 + idx / C::CPR, cc = (idx % C::CPR) * C::VEC;
      x[j] = vzero<T>();
      if (idx < CH && gr < S && cc < HD) x[j] = load16(src + (size_t)gr * HD + cc);
    }
  }
  __device__ __forceinline__ void store(T* tile, int t) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = t + j * NTHR;
      if (idx < CH) store16(tile + (idx / C::CPR) * C::LDS_ROW + (idx % C::CPR) * C::VEC, x[j]);
    }
  }
};

// Store the lane's column of a 32-row-tiled [HD] accumulator (rows d = 32*dt + 8*g + 4*h
// + 0..3) as row `row` of an [S, HD] output, times `mul`.
template <typename TO, int HD, int NDT>
__device__ __forceinline__ void store_column(TO* dst, const f32x16 (&acc)[NDT], float mul,
                                             int h) {
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      if (d < HD) {
        if constexpr (std::is_same<TO, float>::value) {
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
  }
}

// Q side of the prologue forward applied to the lane's resident Q fragment (bf16 io,
// head_dim 16 or 32; Mint documentation 5.4.1 and 5.5.1): raw row t of the head whose rows
// start at head_row0, elements 16 c + 8 h + j of chunk c as load_fragment places them, is
// normalised and rotated with the standalone prologue forward's operations in its order
// (no multiply-add contraction; at head_dim 32 the lanes l and l ^ 32 own a row's columns
// as its two row lanes do, at head_dim 16 each takes the other's half so that both sum the
// whole row as its one row lane does), so the rows are bitwise those of
// xattn_qknorm_rope_fwd.  The rotated row becomes the fragment; with `store` it also goes to
// pro.yq and its rstd to pro.rstd_q.  Rows t >= S give a zero fragment and store nothing.
// Every lane of the wave calls.
template <int HD>
__device__ __forceinline__ void q_prologue_frag(bf16x8 (&qf)[HD / 16], const QProFuse& pro,
                                                size_t head_row0, int t, int S, bool store,
                                                int lane) {
#pragma clang fp contract(off)
  static_assert(HD == 16 || HD == 32, "fragment of one or two 16-byte chunks");
  constexpr int HALF = HD / 2;
  const int h = lane >> 5;
  const int f0 = HD == 32 ? 8 * h : 0;  // the lane's first-half columns f0 .. f0 + 7
  const bool valid = t < S;
  const int tc = valid ? t : S - 1;
  const size_t row = head_row0 + tc;
  const bf16* xq = static_cast<const bf16*>(pro.xq);
  float a[8], b[8], g1[8], g2[8], cs[8], sn[8];
  if constexpr (HD == 32) {
    const bf16x8 xa = load16(xq + row * HD + f0), xb = load16(xq + row * HD + HALF + f0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (float)xa[e];
      b[e] = (float)xb[e];
    }
  } else {
    const bf16x8 xo = load16(xq + row * HD + 8 * h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float own = (float)xo[e], other = xor_lanes<32>(own);
      a[e] = h ? other : own;
      b[e] = h ? own : other;
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const f32x4 ga = *reinterpret_cast<const f32x4*>(pro.gamma_q + f0 + 4 * u);
    const f32x4 gb = *reinterpret_cast<const f32x4*>(pro.gamma_q + HALF + f0 + 4 * u);
    const f32x4 ca = *reinterpret_cast<const f32x4*>(pro.cos_tab + (size_t)tc * HALF + f0 + 4 * u);
    const f32x4 sa = *reinterpret_cast<const f32x4*>(pro.sin_tab + (size_t)tc * HALF + f0 + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g1[4 * u + e] = ga[e];
      g2[4 * u + e] = gb[e];
      cs[4 * u + e] = ca[e];
      sn[4 * u + e] = sa[e];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += a[e] * a[e] + b[e] * b[e];
  if constexpr (HD == 32) ss = ss + xor_lanes<32>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / (float)HD) + pro.eps);
  bf16x8 y1, y2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float n1 = a[e] * r * g1[e];
    const float n2 = b[e] * r * g2[e];
    y1[e] = valid ? (bf16)(n1 * cs[e] - n2 * sn[e]) : (bf16)0.f;
    y2[e] = valid ? (bf16)(n1 * sn[e] + n2 * cs[e]) : (bf16)0.f;
  }
  bf16* yq = static_cast<bf16*>(pro.yq);
  if constexpr (HD == 32) {
    qf[0] = y1;
    qf[1] = y2;
    if (store && valid) {
      store16(yq + row * HD + f0, y1);
      store16(yq + row * HD + HALF + f0, y2);
    }
  } else {
    qf[0] = h ? y2 : y1;
    if (store && valid) store16(yq + row * HD + 8 * h, qf[0]);
  }
  if (store && valid && h == 0) pro.rstd_q[row] = r;
}

// The same for fp32 io at any head_dim (Mint documentation 5.4.1 and 5.5.1).  The fragment
// holds columns 8 c + 4 h + j of chunk c: lane half h owns the standalone kernel's 4-column
// parts p = 2 c + h of the first half (chunks c < HD / 16) with their second-half partners
// (chunk c + HD / 16).  The standalone kernel sums each part's squares in its lane, then
// adds the parts by a butterfly over its HD / 8 row lanes (pairs (2c, 2c + 1) first, then
// pairs of pairs, ...); here each part pair is one cross-half exchange and the upper levels
// are added in the same tree, so the rows and rstd are bitwise those of
// xattn_qknorm_rope_fwd.  Rows t >= S give a zero fragment and store nothing.
template <int HD>
__device__ __forceinline__ void q_prologue_frag(f32x4 (&qf)[HD / 8], const QProFuse& pro,
                                                size_t head_row0, int t, int S, bool store,
                                                int lane) {
#pragma clang fp contract(off)
  constexpr int HALF = HD / 2, NP = HD / 16;  // first-half parts per lane
  const int h = lane >> 5;
  const bool valid = t < S;
  const int tc = valid ? t : S - 1;
  const size_t row = head_row0 + tc;
  const float* xr = static_cast<const float*>(pro.xq) + row * HD + 4 * h;
  f32x4 a[NP], b[NP], g1[NP], g2[NP], cs[NP], sn[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const int f = 8 * c + 4 * h;  // the part's first column
    a[c] = *reinterpret_cast<const f32x4*>(xr + 8 * c);
    b[c] = *reinterpret_cast<const f32x4*>(xr + HALF + 8 * c);
    g1[c] = *reinterpret_cast<const f32x4*>(pro.gamma_q + f);
    g2[c] = *reinterpret_cast<const f32x4*>(pro.gamma_q + HALF + f);
    cs[c] = *reinterpret_cast<const f32x4*>(pro.cos_tab + (size_t)tc * HALF + f);
    sn[c] = *reinterpret_cast<const f32x4*>(pro.sin_tab + (size_t)tc * HALF + f);
  }
  float tr[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    float sp = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) sp += a[c][e] * a[c][e] + b[c][e] * b[c][e];
    tr[c] = sp + xor_lanes<32>(sp);  // parts 2c and 2c + 1
  }
#pragma unroll
  for (int n = NP; n > 1; n /= 2)
#pragma unroll
    for (int i = 0; i < n / 2; ++i) tr[i] = tr[2 * i] + tr[2 * i + 1];
  const float r = 1.0f / sqrtf(tr[0] * (1.0f / (float)HD) + pro.eps);
  float* yr = static_cast<float*>(pro.yq) + row * HD + 4 * h;
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    f32x4 y1, y2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float n1 = a[c][e] * r * g1[c][e];
      const float n2 = b[c][e] * r * g2[c][e];
      y1[e] = valid ? n1 * cs[c][e] - n2 * sn[c][e] : 0.f;
      y2[e] = valid ? n1 * sn[c][e] + n2 * cs[c][e] : 0.f;
    }
    qf[c] = y1;
    qf[c + NP] = y2;
    if (store && valid) {
      *reinterpret_cast<f32x4*>(yr + 8 * c) = y1;
      *reinterpret_cast<f32x4*>(yr + HALF + 8 * c) = y2;
    }
  }
  if (store && valid && h == 0) pro.rstd_q[row] = r;
}

// Prologue backward applied in the dq / dk stores of the kernels below (bf16 io, head_dim 16
// or 32; the arithmetic of the standalone prologue backward, Mint documentation 5.4.4 and
// 5.5.2), so the gradient w.r.t. the rotated rows never goes to HBM.  The lane's `mul` *
// acc is that gradient for row t of the head whose rows start at head_row0, column
// 8 g + 4 h + j in acc[4 g + j] (g < HD / 8): both columns of every rotation pair
// (c, c + HD / 2) are the lane's own, and the row's other columns are in lane l ^ 32.
// Writes dx of row t (when t < S) to dx_head + t * HD, and the dgamma terms of the wave's
// 32 rows, summed over the rows in a fixed order (rows t >= S add nothing), to partial slot
// `slot`.  Every lane of the wave calls.
template <int HD>
__device__ __forceinline__ void pro_column(const f32x16& acc, float mul, const ProBwd& pb,
                                           size_t head_row0, int t, int S,
                                           bf16* __restrict__ dx_head, int slot, int lane) {
  static_assert(HD == 16 || HD == 32, "one 32-column accumulator tile");
  constexpr int NG = HD / 8, HG = NG / 2, HALF = HD / 2;
  const int h = lane >> 5;
  const bool valid = t < S;
  const size_t row = head_row0 + (valid ? t : S - 1);
  const float r = pb.rstd[row];
  float xf[NG][4], gm[NG][4], n[NG][4];
  f32x4 cs[HG], sn[HG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int col = 8 * g + 4 * h;
    const bf16x4 xv = *reinterpret_cast<const bf16x4*>(pb.x + row * HD + col);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(pb.gamma + col);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xf[g][j] = (float)xv[j];
      gm[g][j] = gv[j];
    }
  }
  const size_t trow = (size_t)(valid ? t : S - 1) * HALF;
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    cs[g] = *reinterpret_cast<const f32x4*>(pb.cos_tab + trow + 8 * g + 4 * h);
    sn[g] = *reinterpret_cast<const f32x4*>(pb.sin_tab + trow + 8 * g + 4 * h);
  }
  float dot = 0.f;
#pragma unroll
  for (int g = 0; g < HG; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = acc[4 * g + j] * mul, b = acc[4 * (g + HG) + j] * mul;
      n[g][j] = a * cs[g][j] + b * sn[g][j];  // rotation by the negative angle
      n[g + HG][j] = b * cs[g][j] - a * sn[g][j];
      dot += gm[g][j] * n[g][j] * xf[g][j] + gm[g + HG][j] * n[g + HG][j] * xf[g + HG][j];
    }
  dot += xor_lanes<32>(dot);
  const float coef = dot * r * r * r * (1.0f / (float)HD);
  float dg[4 * NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = (bf16)(gm[g][j] * n[g][j] * r - xf[g][j] * coef);
      dg[4 * g + j] = valid ? n[g][j] * xf[g][j] * r : 0.f;
    }
    if (valid) *reinterpret_cast<bf16x4*>(dx_head + (size_t)t * HD + 8 * g + 4 * h) = o;
  }
  // sum over the rows (lane bits 16 .. 1): recursive halving, then the remaining bits; the
  // lane is left with register k of its half's columns
  int k;
  bool writer;
  if constexpr (NG == 4) {
    halving_sum<16, 16, 16, 2>(dg, lane);
    dg[0] += xor_lanes<1>(dg[0]);
    k = 8 * ((lane >> 4) & 1) + 4 * ((lane >> 3) & 1) + 2 * ((lane >> 2) & 1) + ((lane >> 1) & 1);
    writer = (lane & 1) == 0;
  } else {
    halving_sum<8, 8, 16, 4>(dg, lane);
    dg[0] += xor_lanes<2>(dg[0]);
    dg[0] += xor_lanes<1>(dg[0]);
    k = 4 * ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1) + ((lane >> 2) & 1);
    writer = (lane & 3) == 0;
  }
  if (writer) pb.partials[(size_t)(8 * (k >> 2) + 4 * h + (k & 3)) * pb.nparts + slot] = dg[0];
}

// Packed documents (block-causal mask): first / last row of row i's document, clamped into
// the sequence (so a bad array gives wrong values but no access outside the tensors);
// without documents 0 and S - 1.
__device__ __forceinline__ int doc_lo(const int* seg_lo, int i, int S) {
  return seg_lo == nullptr ? 0 : min(max(seg_lo[min(i, S - 1)], 0), S - 1);
}
__device__ __forceinline__ int doc_hi(const int* seg_hi, int i, int S) {
  return seg_hi == nullptr ? S - 1 : min(max(seg_hi[min(i, S - 1)], 0), S - 1);
}

constexpr int kWaves = 4;
constexpr int kBlockM = 32 * kWaves;  // queries per forward / dq workgroup
constexpr int kBlockN = 64;           // keys per LDS stage in forward / dq

// --------------------------------------------------------------------------------------
// forward: one workgroup per (batch*head, 128-query tile); 4 waves x 32 queries.
// --------------------------------------------------------------------------------------
template <typename T, int HD, bool QPRO>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       const T* __restrict__ v,
                                                       T* __restrict__ out,
                                                       float* __restrict__ lse, int S, int H,
                                                       int Hkv, float scale_log2,
                                                       const int* __restrict__ seg_lo,
                                                       QProFuse pro) {
  using C = Tile<T, HD>;
  __shared__ __attribute__((aligned(16))) T ks[kBlockN * C::LDS_ROW];
  __shared__ __attribute__((aligned(16))) T vs[kBlockN * C::LDS_ROW];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int bh = blockIdx.x;
  const int qt = gridDim.y - 1 - blockIdx.y;  // heaviest query tiles first
  const int b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const T* qp = q + (size_t)bh * S * HD;
  const T* kp = k + (size_t)kvbh * S * HD;
  const T* vp = v + (size_t)kvbh * S * HD;
  const int q0 = qt * kBlockM;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + c32;

  vec16_t<T> qf[C::NCH];
  if constexpr (QPRO) q_prologue_frag<HD>(qf, pro, (size_t)bh * S, qrow, S, true, lane);
  else load_fragment<T, HD>(qf, qp, qrow, S, h);
  f32x16 o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  // row i sees keys doc_lo(i) <= j <= i
  const bool docs = seg_lo != nullptr;
  const int lo_row = doc_lo(seg_lo, qrow, S), lo_wave = doc_lo(seg_lo, qw0, S);

  const int kend = min(S, q0 + kBlockM);
  const int ntiles = (kend + kBlockN - 1) / kBlockN;
  // the next stage's K / V rows are loaded into registers under the current stage
  RowPrefetch<T, HD, kBlockN, 256> pk, pv;
  const int kt0 = doc_lo(seg_lo, q0, S) / kBlockN;
  if (kt0 < ntiles) {
    pk.load(kp, kt0 * kBlockN, S, tid);
    pv.load(vp, kt0 * kBlockN, S, tid);
  }
  for (int kt = kt0; kt < ntiles; ++kt) {
    const int k0 = kt * kBlockN;
    __syncthreads();
    pk.store(ks, tid);
    pv.store(vs, tid);
    __syncthreads();
    if (kt + 1 < ntiles) {
      pk.load(kp, k0 + kBlockN, S, tid);
      pv.load(vp, k0 + kBlockN, S, tid);
    }
#pragma unroll
    for (int s = 0; s < kBlockN / 32; ++s) {
      const int kb = k0 + 32 * s;
      if (kb > qw0 + 31 || kb >= S) break;  // wave-uniform: keys all in the future / past end
      if (kb + 31 < lo_wave) continue;      // wave-uniform: before every row's document
      f32x16 st = contract_hd<T, HD>(ks, 32 * s, qf, lane);
      const bool edge = (kb + 31 > qw0) || (kb + 31 >= S) || docs;
      float sv[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = st[i] * scale_log2;
        if (edge) {
          const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > qrow || key >= S || key < lo_row) x = -INFINITY;
        }
        sv[i] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = fmaxf(tmax, xor_lanes<32>(tmax));
      const float m_new = fmaxf(m_run, tmax);
      // a row that has seen no visible key yet (possible with documents) stays empty
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_ref);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = fast_exp2(sv[i] - m_ref);
        psum += sv[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) o[dt] *= alpha;
      accumulate_transposed<T, HD>(o, vs, 32 * s, sv, lane);
    }
  }

  l_run += xor_lanes<32>(l_run);
  if (qrow < S) {
    store_column<T, HD, C::NDT>(out + ((size_t)bh * S + qrow) * HD, o, 1.0f / l_run, h);
    if (h == 0) lse[(size_t)bh * S + qrow] = (m_run + log2f(l_run)) * kLn2;
  }
}

// --------------------------------------------------------------------------------------
// backward, dq: one workgroup per (batch*head, 128-query tile); also writes
// delta_i = dO_i . out_i for the dk/dv kernel.
// --------------------------------------------------------------------------------------
template <typename T, int HD, typename TG, bool PRO>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ out, const T* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ delta, TG* __restrict__ dq, int S, int H, int Hkv, float scale_log2,
    float scale, const int* __restrict__ seg_lo, ProBwd pro) {
  using C = Tile<T, HD>;
  __shared__ __attribute__((aligned(16))) T ks[kBlockN * C::LDS_ROW];
  __shared__ __attribute__((aligned(16))) T vs[kBlockN * C::LDS_ROW];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int bh = blockIdx.x;
  const int qt = gridDim.y - 1 - blockIdx.y;
  const int b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const T* kp = k + (size_t)kvbh * S * HD;
  const T* vp = v + (size_t)kvbh * S * HD;
  const int q0 = qt * kBlockM;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + c32;
  const size_t head_off = (size_t)bh * S * HD;

  vec16_t<T> qf[C::NCH], df[C::NCH];
  load_fragment<T, HD>(qf, q + head_off, qrow, S, h);
  load_fragment<T, HD>(df, dout + head_off, qrow, S, h);
  // delta = dO . out over this lane's chunks, then across the two lane halves
  float dsum = 0.f;
  {
    vec16_t<T> of[C::NCH];
    load_fragment<T, HD>(of, out + head_off, qrow, S, h);
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
#pragma unroll
      for (int j = 0; j < C::VEC; ++j) dsum += to_f32(df[c][j]) * to_f32(of[c][j]);
  }
  const float D = dsum + xor_lanes<32>(dsum);
  const float lse2 = qrow < S ? lse[(size_t)bh * S + qrow] * kLog2e : 0.f;
  if (qrow < S && h == 0) delta[(size_t)bh * S + qrow] = D;

  f32x16 acc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = zero16();

  const bool docs = seg_lo != nullptr;
  const int lo_row = doc_lo(seg_lo, qrow, S), lo_wave = doc_lo(seg_lo, qw0, S);
  const int kend = min(S, q0 + kBlockM);
  const int ntiles = (kend + kBlockN - 1) / kBlockN;
  // the next stage's K / V rows are loaded into registers under the current stage
  RowPrefetch<T, HD, kBlockN, 256> pk, pv;
  const int kt0 = doc_lo(seg_lo, q0, S) / kBlockN;
  if (kt0 < ntiles) {
    pk.load(kp, kt0 * kBlockN, S, tid);
    pv.load(vp, kt0 * kBlockN, S, tid);
  }
  for (int kt = kt0; kt < ntiles; ++kt) {
    const int k0 = kt * kBlockN;
    __syncthreads();
    pk.store(ks, tid);
    pv.store(vs, tid);
    __syncthreads();
    if (kt + 1 < ntiles) {
      pk.load(kp, k0 + kBlockN, S, tid);
      pv.load(vp, k0 + kBlockN, S, tid);
    }
#pragma unroll
    for (int s = 0; s < kBlockN / 32; ++s) {
      const int kb = k0 + 32 * s;
      if (kb > qw0 + 31 || kb >= S) break;
      if (kb + 31 < lo_wave) continue;
      const f32x16 st = contract_hd<T, HD>(ks, 32 * s, qf, lane);   // S^T: keys x queries
      const f32x16 dpt = contract_hd<T, HD>(vs, 32 * s, df, lane);  // dP^T
      const bool edge = (kb + 31 > qw0) || (kb + 31 >= S) || docs;
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(st[i] * scale_log2 - lse2);
        if (edge) {
          const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > qrow || key >= S || key < lo_row) p = 0.f;
        }
        dsv[i] = p * (dpt[i] - D);
      }
      accumulate_transposed<T, HD>(acc, ks, 32 * s, dsv, lane);  // dQ^T += K^T dS^T
    }
  }
  if constexpr (PRO) {  // one dgamma slot per wave
    static_assert(std::is_same<TG, bf16>::value, "dx in the io dtype");
    pro_column<HD>(acc[0], scale, pro, (size_t)bh * S, qrow, S, dq + head_off,
                   (blockIdx.x * gridDim.y + blockIdx.y) * kWaves + w, lane);
  } else if (qrow < S) {
    store_column<TG, HD, C::NDT>(dq + ((size_t)bh * S + qrow) * HD, acc, scale, h);
  }
}

// --------------------------------------------------------------------------------------
// forward and dq for small grids (fewer 128-query workgroups than CUs): one workgroup per
// (batch*head, 32-query tile); wave w walks the key stages w, w + 4, ... (32 keys each)
// through its own LDS tiles, and the four waves' partial states are merged in wave order at
// the end.  Each wave's chain of products is a quarter as long as in the kernels above, and
// four times as many workgroups share the machine; the merge order depends on the shape
// only, so results stay bitwise reproducible.
// --------------------------------------------------------------------------------------
constexpr int kSplitKeys = 32;  // keys per wave stage in the split kernels
constexpr int kSplitM = 32;     // queries per split workgroup

template <typename T, int HD>
struct SplitLds {
  using C = Tile<T, HD>;
  static constexpr int TILE = kSplitKeys * C::LDS_ROW;  // elements per staged tile
  static constexpr int STAGE_BYTES = kWaves * 2 * TILE * (int)sizeof(T);
  static constexpr int PER = 16 * C::NDT + 2;           // merged floats per lane
  static constexpr int MERGE_BYTES = (kWaves - 1) * 64 * PER * (int)sizeof(float);
  static constexpr int BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
};

// A wave's own 32-row K and V stages: the stage's rows, loaded into registers one stage
// ahead, are written to the wave's LDS tiles, and the writes ordered before the wave's reads;
// then the wave's next stage is loaded (in flight under this stage's products).
template <typename T, int HD>
struct SplitStager {
  RowPrefetch<T, HD, kSplitKeys, 64> pk, pv;
  __device__ __forceinline__ void load(const T* kp, const T* vp, int kb, int S, int lane) {
    pk.load(kp, kb, S, lane);
    pv.load(vp, kb, S, lane);
  }
  __device__ __forceinline__ void commit(T* ks, T* vs, int lane) {
    pk.store(ks, lane);
    pv.store(vs, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
};

template <typename T, int HD, bool QPRO>
__global__ __launch_bounds__(256) void attn_fwd_split_kernel(const T* __restrict__ q,
                                                             const T* __restrict__ k,
                                                             const T* __restrict__ v,
                                                             T* __restrict__ out,
                                                             float* __restrict__ lse, int S,
                                                             int H, int Hkv, float scale_log2,
                                                             const int* __restrict__ seg_lo,
                                                             QProFuse pro) {
  using C = Tile<T, HD>;
  using L = SplitLds<T, HD>;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x;
  const int qt = gridDim.y - 1 - blockIdx.y;  // heaviest query tiles first
  const int b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const T* kp = k + (size_t)kvbh * S * HD;
  const T* vp = v + (size_t)kvbh * S * HD;
  const int q0 = qt * kSplitM, qrow = q0 + c32;
  T* ks = reinterpret_cast<T*>(lds) + (2 * w) * L::TILE;
  T* vs = ks + L::TILE;

  vec16_t<T> qf[C::NCH];
  if constexpr (QPRO)  // the four waves share the rows; wave 0 stores them
    q_prologue_frag<HD>(qf, pro, (size_t)bh * S, qrow, S, w == 0, lane);
  else
    load_fragment<T, HD>(qf, q + (size_t)bh * S * HD, qrow, S, h);
  f32x16 o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const bool docs = seg_lo != nullptr;
  const int lo_row = doc_lo(seg_lo, qrow, S), lo_wave = doc_lo(seg_lo, q0, S);
  const int ntiles = (min(S, q0 + kSplitM) + kSplitKeys - 1) / kSplitKeys;
  SplitStager<T, HD> stg;
  const int kt0 = lo_wave / kSplitKeys + w;
  if (kt0 < ntiles) stg.load(kp, vp, kt0 * kSplitKeys, S, lane);
  for (int kt = kt0; kt < ntiles; kt += kWaves) {
    const int kb = kt * kSplitKeys;  // <= q0 + 31 and < S: every stage has visible keys
    stg.commit(ks, vs, lane);
    if (kt + kWaves < ntiles) stg.load(kp, vp, kb + kWaves * kSplitKeys, S, lane);
    f32x16 st = contract_hd<T, HD>(ks, 0, qf, lane);
    const bool edge = (kb + 31 > q0) || (kb + 31 >= S) || docs;
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = st[i] * scale_log2;
      if (edge) {
        const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key > qrow || key >= S || key < lo_row) x = -INFINITY;
      }
      sv[i] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, xor_lanes<32>(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet: stays empty
    const float alpha = fast_exp2(m_run - m_ref);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = fast_exp2(sv[i] - m_ref);
      psum += sv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) o[dt] *= alpha;
    accumulate_transposed<T, HD>(o, vs, 0, sv, lane);
    __builtin_amdgcn_wave_barrier();  // the tiles' reads stay before the next stage's copy
  }

  // merge: waves 1..3 hand their (max, per-half sum, output) to wave 0 through LDS
  __syncthreads();
  float* mg = reinterpret_cast<float*>(lds);
  if (w > 0) {
    float* dst = mg + ((w - 1) * 64 + lane) * L::PER;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[16 * dt + i] = o[dt][i];
    dst[16 * C::NDT] = m_run;
    dst[16 * C::NDT + 1] = l_run;
  }
  __syncthreads();
  if (w != 0) return;
  float M = m_run;
#pragma unroll
  for (int u = 1; u < kWaves; ++u) M = fmaxf(M, mg[((u - 1) * 64 + lane) * L::PER + 16 * C::NDT]);
  const float ref = M == -INFINITY ? 0.f : M;
  const float f0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - ref);
  float l = l_run * f0;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] *= f0;
#pragma unroll
  for (int u = 1; u < kWaves; ++u) {  // wave order
    const float* src = mg + ((u - 1) * 64 + lane) * L::PER;
    const float mu = src[16 * C::NDT];
    const float f = mu == -INFINITY ? 0.f : fast_exp2(mu - ref);
    l += src[16 * C::NDT + 1] * f;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] += src[16 * dt + i] * f;
  }
  l += xor_lanes<32>(l);
  if (qrow < S) {
    store_column<T, HD, C::NDT>(out + ((size_t)bh * S + qrow) * HD, o, 1.0f / l, h);
    if (h == 0) lse[(size_t)bh * S + qrow] = (M + log2f(l)) * kLn2;
  }
}

template <typename T, int HD, typename TG, bool PRO>
__global__ __launch_bounds__(256) void attn_bwd_dq_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ out, const T* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ delta, TG* __restrict__ dq, int S, int H, int Hkv, float scale_log2,
    float scale, const int* __restrict__ seg_lo, ProBwd pro) {
  using C = Tile<T, HD>;
  using L = SplitLds<T, HD>;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x;
  const int qt = gridDim.y - 1 - blockIdx.y;
  const int b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const T* kp = k + (size_t)kvbh * S * HD;
  const T* vp = v + (size_t)kvbh * S * HD;
  const int q0 = qt * kSplitM, qrow = q0 + c32;
  const size_t head_off = (size_t)bh * S * HD;
  T* ks = reinterpret_cast<T*>(lds) + (2 * w) * L::TILE;
  T* vs = ks + L::TILE;

  vec16_t<T> qf[C::NCH], df[C::NCH];
  load_fragment<T, HD>(qf, q + head_off, qrow, S, h);
  load_fragment<T, HD>(df, dout + head_off, qrow, S, h);
  float dsum = 0.f;
  {
    vec16_t<T> of[C::NCH];
    load_fragment<T, HD>(of, out + head_off, qrow, S, h);
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
#pragma unroll
      for (int j = 0; j < C::VEC; ++j) dsum += to_f32(df[c][j]) * to_f32(of[c][j]);
  }
  const float D = dsum + xor_lanes<32>(dsum);
  const float lse2 = qrow < S ? lse[(size_t)bh * S + qrow] * kLog2e : 0.f;
  if (w == 0 && qrow < S && h == 0) delta[(size_t)bh * S + qrow] = D;

  f32x16 acc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = zero16();
  const bool docs = seg_lo != nullptr;
  const int lo_row = doc_lo(seg_lo, qrow, S), lo_wave = doc_lo(seg_lo, q0, S);
  const int ntiles = (min(S, q0 + kSplitM) + kSplitKeys - 1) / kSplitKeys;
  SplitStager<T, HD> stg;
  const int kt0 = lo_wave / kSplitKeys + w;
  if (kt0 < ntiles) stg.load(kp, vp, kt0 * kSplitKeys, S, lane);
  for (int kt = kt0; kt < ntiles; kt += kWaves) {
    const int kb = kt * kSplitKeys;
    stg.commit(ks, vs, lane);
    if (kt + kWaves < ntiles) stg.load(kp, vp, kb + kWaves * kSplitKeys, S, lane);
    const f32x16 st = contract_hd<T, HD>(ks, 0, qf, lane);   // S^T: keys x queries
    const f32x16 dpt = contract_hd<T, HD>(vs, 0, df, lane);  // dP^T
    const bool edge = (kb + 31 > q0) || (kb + 31 >= S) || docs;
    float dsv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = fast_exp2(st[i] * scale_log2 - lse2);
      if (edge) {
        const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key > qrow || key >= S || key < lo_row) p = 0.f;
      }
      dsv[i] = p * (dpt[i] - D);
    }
    accumulate_transposed<T, HD>(acc, ks, 0, dsv, lane);  // dQ^T += K^T dS^T
    __builtin_amdgcn_wave_barrier();
  }

  // merge: the waves' partial dQ added in wave order by wave 0
  __syncthreads();
  float* mg = reinterpret_cast<float*>(lds);
  if (w > 0) {
    float* dst = mg + ((w - 1) * 64 + lane) * L::PER;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[16 * dt + i] = acc[dt][i];
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int u = 1; u < kWaves; ++u) {
    const float* src = mg + ((u - 1) * 64 + lane) * L::PER;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] += src[16 * dt + i];
  }
  if constexpr (PRO) {  // one dgamma slot per workgroup (wave 0 holds its 32 rows)
    static_assert(std::is_same<TG, bf16>::value, "dx in the io dtype");
    pro_column<HD>(acc[0], scale, pro, (size_t)bh * S, qrow, S, dq + head_off,
                   blockIdx.x * gridDim.y + blockIdx.y, lane);
  } else if (qrow < S) {
    store_column<TG, HD, C::NDT>(dq + ((size_t)bh * S + qrow) * HD, acc, scale, h);
  }
}

// The split kernels serve shapes whose 128-query workgroups would not cover the CUs.
static inline bool use_split(const AttnShape& s) {
  const long long wg = (long long)s.batch * s.num_heads * ((s.seq_len + kBlockM - 1) / kBlockM);
  return wg < 256;
}

// --------------------------------------------------------------------------------------
// backward, dk/dv: one workgroup owns 32*KW keys of one KV head; QS query splits
// (QS * KW = 4 waves) walk interleaved 32-query tiles of every query head of the group,
// r ascending; the split partials are added in split order at the end.  Every dk/dv
// element therefore has one owner and a fixed summation order (with the query heads also
// split over workgroups, a fixed-order sum of their partials follows, below).
// --------------------------------------------------------------------------------------
constexpr int kBlockMQ = 32;  // queries per LDS stage in dk/dv

// Waves of a dk/dv workgroup: four, or QS when the query walk is split eight ways.
constexpr int dkdv_waves(int qs) { return qs > kWaves ? qs : kWaves; }

// With gsplit > 1 the group's query heads are split over blockIdx.z (heads
// z*group/gsplit .. (z+1)*group/gsplit - 1, ascending) and each workgroup writes its fp32
// partial dK (unscaled) and dV to part instead of dk / dv; dkdv_group_sum_kernel then adds
// the gsplit partials in z order.
template <typename T, int HD, typename TG, int QS, bool PRO>
__global__ __launch_bounds__(64 * dkdv_waves(QS)) void attn_bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, TG* __restrict__ dk, T* __restrict__ dv, int S, int H,
    int Hkv, float scale_log2, float scale, const int* __restrict__ seg_hi, int gsplit,
    float* __restrict__ part, ProBwd pro) {
  using C = Tile<T, HD>;
  constexpr int KW = dkdv_waves(QS) / QS;
  constexpr int BNK = 32 * KW;
  constexpr int TILE = kBlockMQ * C::LDS_ROW;
  // Q tiles of the QS splits, then their dO tiles (one buffer so that the split
  // reduction at the end can reuse all of it as fp32 scratch).
  __shared__ __attribute__((aligned(16))) T stage[2 * QS * TILE];
  __shared__ float lse_s[QS][kBlockMQ];
  __shared__ float del_s[QS][kBlockMQ];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int kw = w % KW, sp = w / KW;
  const int st_tid = tid % (64 * KW);
  const int kvbh = blockIdx.x;
  const int b = kvbh / Hkv, kvh = kvbh - b * Hkv;
  const int group = H / Hkv;
  const int r_lo = (int)blockIdx.z * group / gsplit;  // the workgroup's query heads
  const int nr = ((int)blockIdx.z + 1) * group / gsplit - r_lo;
  const int k0 = blockIdx.y * BNK;  // lowest key tiles (most work) dispatched first
  const int kw0 = k0 + 32 * kw;
  const int key = kw0 + c32;
  T* qtile = stage + sp * TILE;
  T* dtile = stage + (QS + sp) * TILE;

  vec16_t<T> kf[C::NCH], vf[C::NCH];
  load_fragment<T, HD>(kf, k + (size_t)kvbh * S * HD, key, S, h);
  load_fragment<T, HD>(vf, v + (size_t)kvbh * S * HD, key, S, h);
  f32x16 dkt[C::NDT], dvt[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) dkt[dt] = dvt[dt] = zero16();

  // key j is seen by queries j <= i <= doc_hi(j); query tiles end at the workgroup's last
  // key's last query
  const bool docs = seg_hi != nullptr;
  const int hi_key = doc_hi(seg_hi, key, S);
  const int qt_first = k0 / kBlockMQ;
  const int nqt = min((S + kBlockMQ - 1) / kBlockMQ,
                      doc_hi(seg_hi, k0 + BNK - 1, S) / kBlockMQ + 1);
  const int nsteps = max(0, (nqt - qt_first + QS - 1) / QS);
  const bool wave_live = kw0 < S;

  // Step u = (query head r = u / nsteps, split step u % nsteps).  The next step's Q / dO rows
  // and row statistics are loaded into registers while the current step computes, and stored
  // into LDS between the step's two barriers.
  constexpr int CH = kBlockMQ * C::CPR;                  // 16-byte chunks per tile
  constexpr int NPT = (CH + 64 * KW - 1) / (64 * KW);    // per staging thread
  vec16_t<T> pq[NPT], pd[NPT];
  float plse = INFINITY, pdel = 0.f;  // staging threads st_tid < kBlockMQ: one row each
  const int nall = nr * nsteps;
  auto fetch = [&](int u) {
    const int r = r_lo + u / nsteps, step = u - (u / nsteps) * nsteps;
    const size_t bh = (size_t)(b * H + kvh * group + r);
    const int q0 = (qt_first + step * QS + sp) * kBlockMQ;
    const bool real = qt_first + step * QS + sp < nqt;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int idx = st_tid + j * 64 * KW;
      const int gr = q0 + idx / C::CPR, cc = (idx % C::CPR) * C::VEC;
      pq[j] = vzero<T>();
      pd[j] = vzero<T>();
      if (real && idx < CH && gr < S && cc < HD) {
        pq[j] = load16(q + (bh * S + gr) * HD + cc);
        pd[j] = load16(dout + (bh * S + gr) * HD + cc);
      }
    }
    if (st_tid < kBlockMQ) {
      const int qi = q0 + st_tid;
      const bool in = real && qi < S;
      plse = in ? lse[bh * S + qi] * kLog2e : INFINITY;
      pdel = in ? delta[bh * S + qi] : 0.f;
    }
  };
  if (nall > 0) fetch(0);
  for (int u = 0; u < nall; ++u) {
    const int step = u % nsteps;
    const int qt = qt_first + step * QS + sp;
    const int q0 = qt * kBlockMQ;
    __syncthreads();  // every wave is done with the previous step's tiles
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int idx = st_tid + j * 64 * KW;
      if (idx < CH) {
        const int rr = idx / C::CPR, cc = (idx % C::CPR) * C::VEC;
        store16(qtile + rr * C::LDS_ROW + cc, pq[j]);
        store16(dtile + rr * C::LDS_ROW + cc, pd[j]);
      }
    }
    if (st_tid < kBlockMQ) {
      lse_s[sp][st_tid] = plse;
      del_s[sp][st_tid] = pdel;
    }
    __syncthreads();
    if (u + 1 < nall) fetch(u + 1);  // in flight under this step's products
    {
      if (qt >= nqt || !wave_live || q0 + kBlockMQ - 1 < kw0) continue;

      const f32x16 st = contract_hd<T, HD>(qtile, 0, kf, lane);   // S: queries x keys
      const f32x16 dpt = contract_hd<T, HD>(dtile, 0, vf, lane);  // dP
      const bool edge = q0 < kw0 + 31 || docs;
      float pv[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int mi = 8 * (i >> 2) + 4 * h + (i & 3);
        float p = fast_exp2(st[i] * scale_log2 - lse_s[sp][mi]);
        if (edge && (q0 + mi < key || q0 + mi > hi_key)) p = 0.f;
        pv[i] = p;
        dsv[i] = p * (dpt[i] - del_s[sp][mi]);
      }
      accumulate_transposed<T, HD>(dvt, dtile, 0, pv, lane);   // dV^T += dO^T P
      accumulate_transposed<T, HD>(dkt, qtile, 0, dsv, lane);  // dK^T += Q^T dS
    }
  }

  if constexpr (QS > 1) {
    // Fixed-order combination of the split partials through LDS, one 32-row tile of one
    // tensor at a time: total = split0 + split1 + ... + split(QS-1).
    static_assert((QS - 1) * KW * 64 * 16 * sizeof(float) <= 2 * QS * TILE * sizeof(T),
                  "reduction scratch must fit in the staging tiles");
    float* red = reinterpret_cast<float*>(stage);
#pragma unroll
    for (int which = 0; which < 2; ++which) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        __syncthreads();
        if (sp > 0) {
          float* slot = red + (((sp - 1) * KW + kw) * 64 + lane) * 16;
          const f32x16& src = which == 0 ? dkt[dt] : dvt[dt];
#pragma unroll
          for (int i = 0; i < 16; ++i) slot[i] = src[i];
        }
        __syncthreads();
        if (sp == 0) {
#pragma unroll
          for (int s2 = 1; s2 < QS; ++s2) {
            const float* slot = red + (((s2 - 1) * KW + kw) * 64 + lane) * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              if (which == 0) dkt[dt][i] += slot[i];
              else dvt[dt][i] += slot[i];
            }
          }
        }
      }
    }
  }
  if constexpr (PRO) {  // no group split; one dgamma slot per wave of keys
    static_assert(std::is_same<TG, bf16>::value, "dx in the io dtype");
    if (sp == 0) {
      pro_column<HD>(dkt[0], scale, pro, (size_t)kvbh * S, key, S, dk + (size_t)kvbh * S * HD,
                     (blockIdx.x * gridDim.y + blockIdx.y) * KW + kw, lane);
      if (key < S) store_column<T, HD, C::NDT>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
    }
  } else if (sp == 0 && key < S) {
    if (part != nullptr) {  // group split: fp32 partials, dK unscaled
      const size_t per = (size_t)gridDim.x * S * HD;  // one partial tensor
      float* pk = part + (size_t)blockIdx.z * 2 * per + ((size_t)kvbh * S + key) * HD;
      store_column<float, HD, C::NDT>(pk, dkt, 1.0f, h);
      store_column<float, HD, C::NDT>(pk + per, dvt, 1.0f, h);
    } else {
      store_column<TG, HD, C::NDT>(dk + ((size_t)kvbh * S + key) * HD, dkt, scale, h);
      store_column<T, HD, C::NDT>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
    }
  }
}

// dk = scale * (sum over z ascending of the partial dK), dv = the sum of the partial dV;
// partials [gsplit][2][n] fp32, four elements per thread.
template <typename T, typename TG>
__global__ __launch_bounds__(256) void dkdv_group_sum_kernel(const float* __restrict__ part,
                                                             TG* __restrict__ dk,
                                                             T* __restrict__ dv, size_t n,
                                                             int gsplit, float scale) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 sk = *reinterpret_cast<const f32x4*>(part + i);
  f32x4 sv = *reinterpret_cast<const f32x4*>(part + n + i);
  for (int z = 1; z < gsplit; ++z) {
    const f32x4 ak = *reinterpret_cast<const f32x4*>(part + (size_t)z * 2 * n + i);
    const f32x4 av = *reinterpret_cast<const f32x4*>(part + (size_t)z * 2 * n + n + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk[e] += ak[e];
      sv[e] += av[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dk[i + e] = from_f32<TG>(sk[e] * scale);
    dv[i + e] = from_f32<T>(sv[e]);
  }
}

// --------------------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------------------
static inline float scale_of(int hd) { return 1.0f / sqrtf((float)hd); }

// With QPRO the Q side of the prologue runs in the kernel (q unused; pro's rows are read,
// and yq / rstd_q written, instead).
template <typename T, int HD, bool QPRO>
static hipError_t fwd_impl(const AttnShape& s, const void* q, const void* k, const void* v,
                           void* out, float* lse, const QProFuse& pro, hipStream_t stream) {
  ProfScope prof("attn_fwd", stream);
  if (use_split(s)) {
    const dim3 grid(s.batch * s.num_heads, (s.seq_len + kSplitM - 1) / kSplitM);
    hipLaunchKernelGGL((attn_fwd_split_kernel<T, HD, QPRO>), grid, dim3(256), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)out, lse, s.seq_len,
                       s.num_heads, s.num_kv_heads, scale_of(HD) * kLog2e, s.seg_lo, pro);
    return hipPeekAtLastError();
  }
  const dim3 grid(s.batch * s.num_heads, (s.seq_len + kBlockM - 1) / kBlockM);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD, QPRO>), grid, dim3(256), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (T*)out, lse, s.seq_len, s.num_heads,
                     s.num_kv_heads, scale_of(HD) * kLog2e, s.seg_lo, pro);
  return hipPeekAtLastError();
}

hipError_t launch_attn_fwd(IoType io, const AttnShape& s, const void* q, const void* k,
                           const void* v, void* out, float* lse, const QProFuse* pro,
                           hipStream_t stream) {
  // bf16 at head_dim 64 / 128 always runs the attn_bf16.hip kernels
  if (io == IO_BF16 && fast_bf16_supported(s.head_dim))
    return launch_attn_fwd_bf16_fast(s, q, k, v, out, lse, pro, stream);
  if (pro != nullptr) {  // the Q side of the prologue inside the forward
#define XATTN_CASE(T, HD) \
    if (s.head_dim == HD) return fwd_impl<T, HD, true>(s, nullptr, k, v, out, lse, *pro, stream);
    if (io == IO_F32) {
      XATTN_CASE(float, 16) XATTN_CASE(float, 32) XATTN_CASE(float, 64) XATTN_CASE(float, 128)
    } else {
      XATTN_CASE(bf16, 16) XATTN_CASE(bf16, 32)
    }
#undef XATTN_CASE
    return hipErrorInvalidValue;
  }
  const QProFuse none{};
#define XATTN_CASE(T, HD) \
  if (s.head_dim == HD) return fwd_impl<T, HD, false>(s, q, k, v, out, lse, none, stream);
  if (io == IO_F32) {
    XATTN_CASE(float, 16) XATTN_CASE(float, 32) XATTN_CASE(float, 64) XATTN_CASE(float, 128)
  } else {
    XATTN_CASE(bf16, 16) XATTN_CASE(bf16, 32)
  }
#undef XATTN_CASE
  return hipErrorInvalidValue;
}

// Query splits for the dk/dv kernel: split the query walk only when there are too few
// key tiles to fill the machine (256 CUs); eight splits (eight waves of 32 keys each) when
// four still leave it short and the staged tiles fit in LDS.  Depends on the shape only, so
// results stay bitwise reproducible for a given shape.
template <typename T, int HD>
static int dkdv_splits(const AttnShape& s) {
  const long long bkv = (long long)s.batch * s.num_kv_heads;
  for (int qs = 1; qs <= 4; qs *= 2) {
    const int bnk = 32 * (kWaves / qs);
    const long long blocks = bkv * ((s.seq_len + bnk - 1) / bnk);
    if (blocks >= 1024) return qs;
  }
  constexpr size_t stage8 = 2 * 8 * (size_t)kBlockMQ * Tile<T, HD>::LDS_ROW * sizeof(T);
  const long long blocks4 = bkv * ((s.seq_len + 31) / 32);
  return (blocks4 < 256 && stage8 <= 144 * 1024) ? 8 : 4;
}

// Group splits of the dk/dv kernel: when even the split query walk leaves fewer than 256
// workgroups, the group's query heads are spread over up to `group` workgroups per key
// block (fp32 partials added afterwards in a fixed order).  Shape only, like the splits.
template <int QS>
static int dkdv_gsplit(const AttnShape& s) {
  constexpr int BNK = 32 * (dkdv_waves(QS) / QS);
  const long long blocks =
      (long long)s.batch * s.num_kv_heads * ((s.seq_len + BNK - 1) / BNK);
  const int group = s.num_heads / s.num_kv_heads;
  if (blocks >= 256 || group == 1) return 1;
  return (int)std::min<long long>(group, (256 + blocks - 1) / blocks);
}

// dk/dv launch; with `pro` (only where dkdv_gsplit is 1) the K side's prologue backward is
// applied in the dk stores.
template <typename T, int HD, typename TG, int QS, bool PRO>
static void launch_dkdv(const AttnShape& s, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* delta, void* dk,
                        void* dv, float* part, const ProBwd& pro, hipStream_t stream) {
  constexpr int BNK = 32 * (dkdv_waves(QS) / QS);
  const int gs = PRO ? 1 : dkdv_gsplit<QS>(s);
  const dim3 grid(s.batch * s.num_kv_heads, (s.seq_len + BNK - 1) / BNK, gs);
  ProfScope prof("attn_bwd_dkdv", stream);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HD, TG, QS, PRO>), grid,
                     dim3(64 * dkdv_waves(QS)), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, delta,
                     (TG*)dk, (T*)dv, s.seq_len, s.num_heads, s.num_kv_heads,
                     scale_of(HD) * kLog2e, scale_of(HD), s.seg_hi, gs,
                     gs > 1 ? part : nullptr, pro);
  if (gs > 1) {
    const size_t n = (size_t)s.batch * s.num_kv_heads * s.seq_len * HD;
    hipLaunchKernelGGL((dkdv_group_sum_kernel<T, TG>), dim3((unsigned)((n / 4 + 255) / 256)),
                       dim3(256), 0, stream, (const float*)part, (TG*)dk, (T*)dv, n, gs,
                       scale_of(HD));
  }
}

// The dk/dv kernel's query splits (QS) and group splits for a shape.
template <typename T, int HD>
static void dkdv_plan(const AttnShape& s, int* qs, int* gs) {
  *qs = dkdv_splits<T, HD>(s);
  switch (*qs) {
    case 1: *gs = dkdv_gsplit<1>(s); break;
    case 2: *gs = dkdv_gsplit<2>(s); break;
    case 8: *gs = dkdv_gsplit<8>(s); break;
    default: *gs = dkdv_gsplit<4>(s); break;
  }
}

template <typename T, int HD, typename TG, bool PRO>
static hipError_t bwd_run(const AttnShape& s, const void* q, const void* k, const void* v,
                          const void* out, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, float* delta, float* part, const ProBwd& pq,
                          const ProBwd& pk, hipStream_t stream) {
  {
    ProfScope prof("attn_bwd_dq", stream);
    if (use_split(s)) {
      const dim3 grid(s.batch * s.num_heads, (s.seq_len + kSplitM - 1) / kSplitM);
      hipLaunchKernelGGL((attn_bwd_dq_split_kernel<T, HD, TG, PRO>), grid, dim3(256), 0, stream,
                         (const T*)q, (const T*)k, (const T*)v, (const T*)out,
                         (const T*)dout, lse, delta, (TG*)dq, s.seq_len, s.num_heads,
                         s.num_kv_heads, scale_of(HD) * kLog2e, scale_of(HD), s.seg_lo, pq);
    } else {
      const dim3 grid(s.batch * s.num_heads, (s.seq_len + kBlockM - 1) / kBlockM);
      hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD, TG, PRO>), grid, dim3(256), 0, stream,
                         (const T*)q, (const T*)k, (const T*)v, (const T*)out,
                         (const T*)dout, lse, delta, (TG*)dq, s.seq_len, s.num_heads,
                         s.num_kv_heads, scale_of(HD) * kLog2e, scale_of(HD), s.seg_lo, pq);
    }
  }
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  int qs, gs;
  dkdv_plan<T, HD>(s, &qs, &gs);
  if (PRO && gs != 1) return hipErrorInvalidValue;
  switch (qs) {
    case 1:
      launch_dkdv<T, HD, TG, 1, PRO>(s, q, k, v, dout, lse, delta, dk, dv, part, pk, stream);
      break;
    case 2:
      launch_dkdv<T, HD, TG, 2, PRO>(s, q, k, v, dout, lse, delta, dk, dv, part, pk, stream);
      break;
    case 8:
      if constexpr (2 * 8 * (size_t)kBlockMQ * Tile<T, HD>::LDS_ROW * sizeof(T) <= 144 * 1024) {
        launch_dkdv<T, HD, TG, 8, PRO>(s, q, k, v, dout, lse, delta, dk, dv, part, pk, stream);
        break;
      }
      [[fallthrough]];
    default:
      launch_dkdv<T, HD, TG, 4, PRO>(s, q, k, v, dout, lse, delta, dk, dv, part, pk, stream);
      break;
  }
  return hipPeekAtLastError();
}

template <typename T, int HD, typename TG>
static hipError_t bwd_impl(const AttnShape& s, const void* q, const void* k, const void* v,
                           const void* out, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, float* delta, float* part, hipStream_t stream) {
  const ProBwd none{};
  return bwd_run<T, HD, TG, false>(s, q, k, v, out, lse, dout, dq, dk, dv, delta, part, none,
                                   none, stream);
}

template <typename T, int HD>
static size_t dkdv_partial_floats_impl(const AttnShape& s) {
  int qs, gs;
  dkdv_plan<T, HD>(s, &qs, &gs);
  return gs > 1 ? 2 * (size_t)gs * s.batch * s.num_kv_heads * s.seq_len * HD : 0;
}

// Partial slots of the fused prologue backward in the kernels above: one per dq wave (four
// per 128-query workgroup, or one per 32-query workgroup of the split kernel) and one per
// final dk wave (KW per key block).  False where the shape runs unfused: a dk/dv launch that
// splits the group's query heads over workgroups.
template <typename T, int HD>
static bool generic_pro_parts_impl(const AttnShape& s, int* nq, int* nk) {
  int qs, gs;
  dkdv_plan<T, HD>(s, &qs, &gs);
  if (gs != 1) return false;
  const int bh = s.batch * s.num_heads;
  *nq = use_split(s) ? bh * ((s.seq_len + kSplitM - 1) / kSplitM)
                     : bh * ((s.seq_len + kBlockM - 1) / kBlockM) * kWaves;
  const int kw = dkdv_waves(qs) / qs, bnk = 32 * kw;
  *nk = s.batch * s.num_kv_heads * ((s.seq_len + bnk - 1) / bnk) * kw;
  return true;
}

bool generic_pro_parts(IoType io, const AttnShape& s, int* nq, int* nk) {
  *nq = *nk = 0;
  if (io != IO_BF16) return false;
  if (s.head_dim == 16) return generic_pro_parts_impl<bf16, 16>(s, nq, nk);
  if (s.head_dim == 32) return generic_pro_parts_impl<bf16, 32>(s, nq, nk);
  return false;
}

size_t dkdv_partial_floats(IoType io, const AttnShape& s) {
  if (io == IO_BF16 && fast_bf16_supported(s.head_dim)) return 0;
#define XATTN_CASE(T, HD) \
  if (s.head_dim == HD) return dkdv_partial_floats_impl<T, HD>(s);
  if (io == IO_F32) {
    XATTN_CASE(float, 16) XATTN_CASE(float, 32) XATTN_CASE(float, 64) XATTN_CASE(float, 128)
  } else {
    XATTN_CASE(bf16, 16) XATTN_CASE(bf16, 32)
  }
#undef XATTN_CASE
  return 0;
}

hipError_t launch_attn_bwd(IoType io, const AttnShape& s, const void* q, const void* k,
                           const void* v, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* delta,
                           float* lse2, bool grads_f32, float* dkdv_part, const ProFuse* pro,
                           hipStream_t stream) {
  // bf16 at head_dim 64 / 128 always runs the attn_bf16.hip kernels (with fp32 gradients
  // never requested there: that path applies the prologue backward in its own stores)
  if (io == IO_BF16 && fast_bf16_supported(s.head_dim)) {
    if (grads_f32 || pro != nullptr) return hipErrorInvalidValue;
    return launch_attn_bwd_bf16_fast(s, q, k, v, out, lse, dout, dq, dk, dv, delta, lse2,
                                     nullptr, stream);
  }
  if (pro != nullptr) {  // bf16, head_dim 16 / 32: the prologue backward in the stores
    int nq, nk;
    if (grads_f32 || !generic_pro_parts(io, s, &nq, &nk)) return hipErrorInvalidValue;
    const ProBwd pq{static_cast<const bf16*>(pro->xq), pro->gamma_q, pro->rstd_q,
                    pro->cos_tab, pro->sin_tab, pro->partials_q, nq};
    const ProBwd pk{static_cast<const bf16*>(pro->xk), pro->gamma_k, pro->rstd_k,
                    pro->cos_tab, pro->sin_tab, pro->partials_k, nk};
    const hipError_t e =
        s.head_dim == 16
            ? bwd_run<bf16, 16, bf16, true>(s, q, k, v, out, lse, dout, dq, dk, dv, delta,
                                            nullptr, pq, pk, stream)
            : bwd_run<bf16, 32, bf16, true>(s, q, k, v, out, lse, dout, dq, dk, dv, delta,
                                            nullptr, pq, pk, stream);
    if (e != hipSuccess) return e;
    return launch_dgamma_reduce_qk(s.head_dim, pro->partials_q, nq, pro->dgamma_q,
                                   pro->partials_k, nk, pro->dgamma_k, stream);
  }
#define XATTN_CASE(T, HD, TG)                                                          \
  if (s.head_dim == HD)                                                                \
    return bwd_impl<T, HD, TG>(s, q, k, v, out, lse, dout, dq, dk, dv, delta, dkdv_part,   \
                               stream);
  if (io == IO_F32) {
    XATTN_CASE(float, 16, float) XATTN_CASE(float, 32, float) XATTN_CASE(float, 64, float)
    XATTN_CASE(float, 128, float)
  } else if (grads_f32) {
    XATTN_CASE(bf16, 16, float) XATTN_CASE(bf16, 32, float)
  } else {
    XATTN_CASE(bf16, 16, bf16) XATTN_CASE(bf16, 32, bf16)
  }
#undef XATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
