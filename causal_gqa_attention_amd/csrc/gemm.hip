// Dense GEMMs of the projections around attention (Mint documentation 5.3.1-5.3.2:
// Q = X Wq + bq, K = X Wk + bk, V = X Wv + bv, output Concat(heads) Wo + bo, weights
// [d_in, d_out] applied as x @ W; "Phase T12: bf16 mixed precision", precision table: the
// linear GEMMs take bf16 in and accumulate in fp32, weight gradients are fp32).
//
// Row-major operands, three forms: NN (C = A B, A [m, k], B [k, n]), NT (C = A B^T, B
// stored [n, k]) and TN (C = A^T B, A stored [k, m]).  A job may sum up to three K
// segments (own A and B each) in one fp32 accumulator before its single rounding, and one
// launch runs up to three jobs.  Outputs: io-dtype token rows (+ bias), io-dtype head
// layout ([B*heads, S, hd], + bias: the head split of the projections), or fp32 rows.
// fp32 outputs may split K over several workgroups; the partial products then land in a
// workspace and a second kernel adds them in split order, so every result has a fixed
// summation order (bitwise reproducible run to run).
//
// bf16 kernel (gfx950):
//   * 128 x 256 output tile per 512-thread workgroup, eight waves of 64 x 64 (2 x 2
//     v_mfma_f32_32x32x16_bf16 blocks), K in steps of 64, one workgroup per CU.
//   * Both operand tiles go HBM -> LDS with direct-to-LDS buffer loads (no register round
//     trip), two K steps ahead of the MFMAs (three staged steps, 144 KiB).  A lane's copy
//     offsets are set once per K segment and advanced by a uniform step.  A chunk that
//     lies outside its matrix gets a byte offset past the buffer's range, which the
//     hardware turns into zeros, so ragged m, n and k need no other handling.
//   * K-contiguous tiles ([128][64]: rows of 128 bytes) are read with ds_read_b128; the
//     16-byte chunks of row r are XOR-swizzled by (r >> 1) & 7 so that the 16 rows one
//     read phase touches sit on 16 distinct bank groups.  M/N-contiguous tiles ([64][128]:
//     rows of 256 bytes) are read with the transposing ds_read_b64_tr_b16 (two reads give
//     a lane its 8 k-slots of one column); their chunks are swizzled by 4 * (r & 3), which
//     spreads the four rows of a read phase over the four quarters of the bank window.
//   * The MFMA takes the B fragment as its A operand, so each accumulator holds a block of
//     C^T: a lane owns one output row and runs of four adjacent columns, which the
//     epilogue stores as 8- or 16-byte vectors (with the bias add and the rounding).
//   * An operand may be the token-row view of a head-major tensor [B*heads, S, hd] (the
//     attention output, the gradients w.r.t. q, k, v): the lane's chunk offset then holds
//     its token's or feature's head coordinates and a K step adds a uniform offset of the
//     next head (k = features) or the next 64 positions of a sequence (k = tokens), so the
//     tensor is read in place instead of being merged into token rows first.
#include <algorithm>

#include "lds_copy.h"
#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kTM = 128, kTK = 64;
constexpr int kOpBytes = kTM * kTK * 2;  // one staged 128-row operand tile: 16 KiB
constexpr uint32_t kOutside = 0x80000000u;  // a byte offset past every operand buffer

// Workgroup shape of the bf16 kernel: NAT x NBT staged 128-row operand tiles (A, B) per K
// step, a WM x WN grid of waves, each wave BM x BN blocks of 32 x 32 outputs.  The one in
// use (GemmShape<2>) is 128 x 256 with eight waves of 64 x 64 and three K steps staged
// (144 KiB, one workgroup per CU): the copies run two steps ahead and each staged A tile
// feeds twice the MFMAs of a 128 x 128 tile.
template <int NAT_, int NBT_, int WM_, int WN_, int BM_, int BN_, int NB_, int PER_>
struct GemmShapeT {
  static constexpr int NAT = NAT_, NBT = NBT_, WM = WM_, WN = WN_, BM = BM_, BN = BN_;
  static constexpr int kNB = NB_, kPerBlock = PER_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kTMW = kTM * NAT, kTN = kTM * NBT;  // output rows / columns
  static constexpr int kStage = (NAT + NBT) * kOpBytes;
  static constexpr int kCopyA = 16 * NAT / kWaves;  // 1 KiB copies per wave and step
  static constexpr int kCopyB = 16 * NBT / kWaves;
  static_assert(32 * BM * WM == kTMW && 32 * BN * WN == kTN, "waves cover the tile");
  static_assert(kCopyA >= 1 && kCopyB >= 1 && 16 % kCopyA == 0 && 16 % kCopyB == 0,
                "whole copies per wave, inside one tile");
  static_assert(kNB * kStage <= 160 * 1024, "staged steps fit the LDS");
};
template <int ID>
struct GemmShape;
template <>
struct GemmShape<2> : GemmShapeT<1, 2, 2, 4, 2, 2, 3, 1> {};
constexpr int kGemmShape = 2;  // the bf16 workgroup shape the launcher uses

// Jobs as the kernels see them: the host-side description plus the tile bookkeeping.
struct KJob {
  GemmJob j;
  int tiles_n, tiles, splits, steps_per_split, block_begin;
};
struct KArgs {
  KJob job[kGemmMaxJobs];
  int njobs, S, hd;
};

__device__ __forceinline__ int find_job(const KArgs& g, int& bid) {
  int j = 0;
#pragma unroll
  for (int q = 1; q < kGemmMaxJobs; ++q)
    if (q < g.njobs && bid >= g.job[q].block_begin) j = q;
  bid -= g.job[j].block_begin;
  return j;
}

// Per-lane copy cursor of one operand over the K steps of one segment: the lane's byte
// offset of each of its wave's four 1 KiB copies at k = 0 (kOutside for rows past the
// matrix), the chunk's k position inside the tile (for the ragged last step) and the byte
// step per K step.  K-contiguous tile: copy c (0..15 over the workgroup) holds rows 8c ..
// 8c+7, lane l the physical chunk l & 7 of row 8c + l / 8, i.e. the logical chunk
// (l & 7) ^ swizzle.  M/N-contiguous tile: copy c holds k-rows 4c .. 4c+3, lane l the
// physical chunk l & 15 of row 4c + l / 16.  Operand buffers stay below 2^31 bytes, so an
// offset at or past kOutside plus any in-matrix step stays past the buffer's range (and
// reads zeros).
template <int NC>
struct OpCursor {
  uint32_t off[NC];
  int kin[NC];
  uint32_t kstep;    // row-major: bytes per K step
  int heads, S, hd;  // head-major matrices (GemmMat::heads > 0)
  // Byte offset of the K step starting at k0 (uniform).  Row-major: k0 / kTK steps.
  // Head-major, K-contiguous (k = features): the head k0 / hd, column k0 % hd.  Head-major,
  // M/N-contiguous (k = tokens; the step's tokens share one sequence): sequence k0 / S,
  // position k0 % S.
  template <bool KC>
  __device__ __forceinline__ uint32_t step(int k0) const {
    if (heads == 0) return (uint32_t)(k0 / kTK) * kstep;
    if constexpr (KC) return (uint32_t)(((k0 / hd) * S * hd + k0 % hd) * 2);
    else return (uint32_t)(((size_t)(k0 / S) * heads * S * hd + (size_t)(k0 % S) * hd) * 2);
  }
};
// The wave's copies c0 .. c0 + NC - 1 of a 128-row (or 128-column) tile starting at r0.
template <bool KC, int NC>
__device__ __forceinline__ void cursor_init(OpCursor<NC>& cu, const GemmMat& a, int rows,
                                            int r0, int c0, int lane, int S, int hd) {
  cu.heads = a.heads;
  cu.S = S;
  cu.hd = hd;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = c0 + i;
    if constexpr (KC) {
      const int row = 8 * c + (lane >> 3);
      const int lc = (lane & 7) ^ (4 * (c & 1) + (lane >> 4));
      const int rg = r0 + row;
      cu.kin[i] = 8 * lc;
      size_t at;
      if (a.heads == 0) {
        at = (size_t)rg * a.ld + 8 * lc;
      } else {  // token rg = (b, s): row (b * heads) * S + s of the head-major tensor
        const size_t b = (size_t)rg / S;
        at = (b * a.heads * S + (rg - b * S)) * hd + 8 * lc;
      }
      cu.off[i] = rg < rows ? (uint32_t)(at * 2) : kOutside;
    } else {
      const int kr = 4 * c + (lane >> 4);
      const int lc = (lane & 15) ^ (4 * ((lane >> 4) & 3));
      const int rg = r0 + 8 * lc;
      cu.kin[i] = kr;
      size_t at;
      if (a.heads == 0) {
        at = (size_t)kr * a.ld + rg;
      } else {  // feature rg = (h, e); token k0 + kr at position kr after the step's
        const int h = rg / hd;
        at = ((size_t)h * S + kr) * hd + (rg - h * hd);
      }
      cu.off[i] = rg < rows ? (uint32_t)(at * 2) : kOutside;
    }
  }
  cu.kstep = KC ? (uint32_t)(kTK * 2) : (uint32_t)kTK * (uint32_t)a.ld * 2u;
}
// Offsets of the copies of the K step starting at k0 (kd = its byte step from k = 0): the
// chunks at or past kdim (only in a ragged last step) read zeros.
template <int NC>
__device__ __forceinline__ void cursor_offsets(uint32_t (&off)[NC], const OpCursor<NC>& cu,
                                               uint32_t kd, int k0, int kdim) {
  const bool ragged = k0 + kTK > kdim;  // uniform
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    off[i] = cu.off[i] + kd;
    if (ragged && k0 + cu.kin[i] >= kdim) off[i] = kOutside;
  }
}

// Fragment of 32 rows (K-contiguous tile) starting at tile row R0: logical chunk 2c + h of
// row R0 + lane % 32 sits at R0 * 128 + (a_lane ^ (c << 5)).
__device__ __forceinline__ uint32_t kc_lane(int lane) {
  const int r = lane & 31, h = lane >> 5;
  return (uint32_t)(r * 128) | (uint32_t)((h ^ ((r >> 1) & 7)) << 4);
}
// Transposing reads (M/N-contiguous tile) of the 8 k-slots 16c + 8h + {0..7} of column
// C0 + lane % 32: rows 16c + 8h + {0..3} at 16c*256 + (t_lane ^ ((C0 / 8) << 4)), rows
// + 4 at 1 KiB further.
__device__ __forceinline__ uint32_t mn_lane(int lane) {
  const int g = lane >> 4, li = lane & 15, h = lane >> 5;
  const int low = 2 * (g & 1) + ((li & 3) >> 1);
  return (uint32_t)((8 * h + (li >> 2)) * 256) | (uint32_t)((low ^ (4 * (li >> 2))) << 4) |
         (uint32_t)((li & 1) << 3);
}

template <bool KC>
__device__ __forceinline__ bf16x8 frag(lptr tile, uint32_t ln, int blk32, int c) {
  if constexpr (KC) {
    return *(lds_cbf16x8_t*)(tile + blk32 * 32 * 128 + (ln ^ (uint32_t)(c << 5)));
  } else {
    lptr p0 = tile + c * 16 * 256 + (ln ^ (uint32_t)((blk32 * 4) << 4));
    const bf16x4 lo = __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0));
    const bf16x4 hi = __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + 4 * 256)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <int FORM, int OUT, int ID>
__global__ __launch_bounds__(64 * GemmShape<ID>::kWaves, GemmShape<ID>::kPerBlock)
void gemm_bf16_kernel(KArgs g) {
  using G = GemmShape<ID>;
  constexpr int NAT = G::NAT, BM = G::BM, BN = G::BN;
  constexpr bool AK = FORM != GEMM_TN;  // A K-contiguous
  constexpr bool BK = FORM == GEMM_NT;  // B K-contiguous
  constexpr int NB = G::kNB, CA = G::kCopyA, CB = G::kCopyB;
  __shared__ __attribute__((aligned(1024))) char lds[NB * G::kStage];
  int bid = blockIdx.x;
  const KJob& kj = g.job[find_job(g, bid)];
  const GemmJob& jb = kj.j;
  const int split = bid / kj.tiles, t = bid - split * kj.tiles;
  const int tm = t / kj.tiles_n, tn = t - tm * kj.tiles_n;
  const int m0 = tm * G::kTMW, n0 = tn * G::kTN;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave (wm, wn) of the WM x WN grid owns rows 32 BM wm .. and columns 32 BN wn ..; it
  // copies chunks ca0 .. ca0 + CA - 1 of A tile cat and cb0 .. cb0 + CB - 1 of B tile cbt
  // (16 chunks of 1 KiB per 128-row tile)
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / G::WN, wn = wv % G::WN;
  const int cat = CA * wv / 16, ca0 = CA * wv % 16;
  const int cbt = CB * wv / 16, cb0 = CB * wv % 16;
  // the tile and first 32-block of the wave's rows (A) and columns (B)
  const int rat = 32 * BM * wm / kTM, rab = 32 * BM * wm % kTM / 32;
  const int rbt = 32 * BN * wn / kTM, rbb = 32 * BN * wn % kTM / 32;

  // the K steps of this workgroup over the segments (a split job has one segment)
  int steps = 0;
  for (int s = 0; s < jb.nseg; ++s) steps += (jb.seg[s].k + kTK - 1) / kTK;
  int st_begin = 0, st_end = steps;
  if (kj.splits > 1) {
    st_begin = split * kj.steps_per_split;
    st_end = min(steps, st_begin + kj.steps_per_split);
  }
  // issue cursor: segment, k inside it, and the segment's operands and lane offsets (set
  // once per segment; a K step then only adds its byte step)
  // (a split job has one segment, so only an unsplit job crosses segments, from k = 0)
  int iseg = 0, ik0 = st_begin * kTK;
  GemmSeg sg = jb.seg[0];
  while (ik0 >= sg.k) {
    ik0 = 0;
    sg = jb.seg[++iseg];
  }
  OpCursor<CA> ca;
  OpCursor<CB> cb;
  cursor_init<AK>(ca, sg.a, jb.m, m0 + kTM * cat, ca0, lane, g.S, g.hd);
  cursor_init<BK>(cb, sg.b, jb.n, n0 + kTM * cbt, cb0, lane, g.S, g.hd);
  auto issue = [&](int buf) {
    if (ik0 >= sg.k) {  // uniform: the cursor moves to the next segment
      do {
        ik0 = 0;
        sg = jb.seg[++iseg];
      } while (ik0 >= sg.k);
      cursor_init<AK>(ca, sg.a, jb.m, m0 + kTM * cat, ca0, lane, g.S, g.hd);
      cursor_init<BK>(cb, sg.b, jb.n, n0 + kTM * cbt, cb0, lane, g.S, g.hd);
    }
    char* stage = lds + buf * G::kStage;
    uint32_t oa[CA], ob[CB];
    cursor_offsets(oa, ca, ca.template step<AK>(ik0), ik0, sg.k);
    dma16_rows<CA>(stage + cat * kOpBytes + ca0 * 1024, static_cast<const char*>(sg.a.p),
                   sg.a.bytes, oa);
    cursor_offsets(ob, cb, cb.template step<BK>(ik0), ik0, sg.k);
    dma16_rows<CB>(stage + (NAT + cbt) * kOpBytes + cb0 * 1024,
                   static_cast<const char*>(sg.b.p), sg.b.bytes, ob);
    ik0 += kTK;
  };

  f32x16 acc[BM][BN];
#pragma unroll
  for (int i = 0; i < BM; ++i)
#pragma unroll
    for (int j = 0; j < BN; ++j) acc[i][j] = zero16();
  const uint32_t la = AK ? kc_lane(lane) : mn_lane(lane);
  const uint32_t lb = BK ? kc_lane(lane) : mn_lane(lane);
  const lptr lbase = to_lds(lds);
  const int nst = st_end - st_begin;
#pragma unroll
  for (int u = 0; u < NB - 1; ++u)
    if (u < nst) issue(u);
  for (int s = 0; s < nst; ++s) {
    // step s has landed (this wave's copies; later steps may stay in flight) ...
    if (s + NB - 1 <= nst) wait_vm<(NB - 2) * (CA + CB)>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // ... and every wave's; step s - 1's reads are done
    lds_acquire();
    if (s + NB - 1 < nst) issue((s + NB - 1) % NB);
    const lptr st0 = lbase + (s % NB) * G::kStage;
    const lptr ta = st0 + rat * kOpBytes, tb = st0 + (NAT + rbt) * kOpBytes;
    bf16x8 fa[BM][4], fb[BN][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < BM; ++i) fa[i][c] = frag<AK>(ta, la, rab + i, c);
#pragma unroll
      for (int j = 0; j < BN; ++j) fb[j][c] = frag<BK>(tb, lb, rbb + j, c);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < BM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j) acc[i][j] = mfma_bf16(fb[j][c], fa[i][c], acc[i][j]);
  }

  // epilogue: lane row m0 + 32 BM wm + 32 i + lane % 32, columns n0 + 32 BN wn + 32 j +
  // 8 q + 4 h + {0..3} in acc[i][j][4q .. 4q+3]
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < BM; ++i) {
    const int row = m0 + 32 * BM * wm + 32 * i + (lane & 31);
    if (row >= jb.m) continue;
    int b = 0, sq = row;
    if constexpr (OUT == GEMM_OUT_IO_HEADS) {
      b = row / g.S;
      sq = row - b * g.S;
    }
#pragma unroll
    for (int j = 0; j < BN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + 32 * BN * wn + 32 * j + 8 * q + 4 * h;
        if (col >= jb.n) continue;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        if constexpr (OUT == GEMM_OUT_F32) {
          float* dst = kj.splits > 1 ? jb.part + (size_t)split * jb.m * jb.ldc : (float*)jb.c;
          *reinterpret_cast<f32x4*>(dst + (size_t)row * jb.ldc + col) = v;
        } else {
          if (jb.bias != nullptr) {
            const f32x4 bv = *reinterpret_cast<const f32x4*>(jb.bias + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += bv[e];
          }
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          size_t at;
          if constexpr (OUT == GEMM_OUT_IO_HEADS) {
            const int hh = col / g.hd, e0 = col - hh * g.hd;
            at = (((size_t)b * jb.c_heads + hh) * g.S + sq) * g.hd + e0;
          } else {
            at = (size_t)row * jb.ldc + col;
          }
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(jb.c) + at) = o;
        }
      }
  }
}

// fp32 io: a plain LDS-tiled kernel (64 x 64 tile, 4 x 4 outputs per lane, K steps of 16)
// with the same forms, jobs, segments and outputs; fp32 FMAs in a fixed k order.
template <int FORM, int OUT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(KArgs g) {
  constexpr int T = 64, KS = 16;
  __shared__ float sa[KS][T + 4], sb[KS][T + 4];
  int bid = blockIdx.x;
  const KJob& kj = g.job[find_job(g, bid)];
  const GemmJob& jb = kj.j;
  const int split = bid / kj.tiles, t = bid - split * kj.tiles;
  const int tm = t / kj.tiles_n, tn = t - tm * kj.tiles_n;
  const int m0 = tm * T, n0 = tn * T;
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  int steps = 0;
  for (int s = 0; s < jb.nseg; ++s) steps += (jb.seg[s].k + KS - 1) / KS;
  int st_begin = 0, st_end = steps;
  if (kj.splits > 1) {
    st_begin = split * kj.steps_per_split;
    st_end = min(steps, st_begin + kj.steps_per_split);
  }
  int seg = 0, k0 = st_begin * KS;
  for (int s = st_begin; s < st_end; ++s) {
    while (k0 >= jb.seg[seg].k) {
      k0 = 0;
      ++seg;
    }
    const GemmSeg& sg = jb.seg[seg];
    const float* A = static_cast<const float*>(sg.a.p);
    const float* B = static_cast<const float*>(sg.b.p);
    // 1024 elements per operand tile, 4 per lane
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = tid + 256 * e, kk = x / T, mn = x % T;
      const int kg = k0 + kk, mg = m0 + mn, ng = n0 + mn;
      float av = 0.f, bv = 0.f;
      if (kg < sg.k && mg < jb.m)
        av = FORM != GEMM_TN ? A[(size_t)mg * sg.a.ld + kg] : A[(size_t)kg * sg.a.ld + mg];
      if (kg < sg.k && ng < jb.n)
        bv = FORM == GEMM_NT ? B[(size_t)ng * sg.b.ld + kg] : B[(size_t)kg * sg.b.ld + ng];
      sa[kk][mn] = av;
      sb[kk][mn] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sa[kk][tr * 4 + i], sb[kk][tc * 4 + j], acc[i][j]);
    __syncthreads();
    k0 += KS;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + tr * 4 + i;
    if (row >= jb.m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tc * 4 + j;
      if (col >= jb.n) continue;
      float v = acc[i][j];
      if constexpr (OUT == GEMM_OUT_F32) {
        float* dst = kj.splits > 1 ? jb.part + (size_t)split * jb.m * jb.ldc : (float*)jb.c;
        dst[(size_t)row * jb.ldc + col] = v;
      } else {
        if (jb.bias != nullptr) v += jb.bias[col];
        size_t at;
        if constexpr (OUT == GEMM_OUT_IO_HEADS) {
          const int b = row / g.S, sq = row - b * g.S, hh = col / g.hd, e0 = col - hh * g.hd;
          at = (((size_t)b * jb.c_heads + hh) * g.S + sq) * g.hd + e0;
        } else {
          at = (size_t)row * jb.ldc + col;
        }
        static_cast<float*>(jb.c)[at] = v;
      }
    }
  }
}

// c[i] = sum over splits s (ascending) of part[s][i], [m, n] fp32 (ldc == n).
__global__ __launch_bounds__(256) void splitk_sum_kernel(KArgs g) {
  const KJob& kj = g.job[blockIdx.y];
  const GemmJob& jb = kj.j;
  if (kj.splits <= 1) return;
  const size_t n4 = (size_t)jb.m * jb.ldc / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(jb.part) + i;
  f32x4 s = p[0];
  for (int q = 1; q < kj.splits; ++q) {
    const f32x4 v = p[q * n4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += v[e];
  }
  reinterpret_cast<f32x4*>(jb.c)[i] = s;
}

template <int FORM>
hipError_t launch_form(IoType io, int out, const KArgs& a, int blocks, dim3 block,
                       hipStream_t stream) {
#define XATTN_GEMM(K, O) hipLaunchKernelGGL((K<FORM, O>), dim3(blocks), block, 0, stream, a)
#define XATTN_GEMM16(O)                                                                   \
  hipLaunchKernelGGL((gemm_bf16_kernel<FORM, O, kGemmShape>), dim3(blocks),              \
                     dim3(64 * GemmShape<kGemmShape>::kWaves), 0, stream, a)
  if (io == IO_BF16) {
    if (out == GEMM_OUT_IO_ROWS) XATTN_GEMM16(GEMM_OUT_IO_ROWS);
    else if (out == GEMM_OUT_IO_HEADS) XATTN_GEMM16(GEMM_OUT_IO_HEADS);
    else XATTN_GEMM16(GEMM_OUT_F32);
  } else {
    if (out == GEMM_OUT_IO_ROWS) XATTN_GEMM(gemm_f32_kernel, GEMM_OUT_IO_ROWS);
    else if (out == GEMM_OUT_IO_HEADS) XATTN_GEMM(gemm_f32_kernel, GEMM_OUT_IO_HEADS);
    else XATTN_GEMM(gemm_f32_kernel, GEMM_OUT_F32);
  }
#undef XATTN_GEMM
#undef XATTN_GEMM16
  return hipPeekAtLastError();
}

// Tile bookkeeping shared by the launcher and the workspace query.
int plan_jobs(IoType io, const GemmJob* jobs, int njobs, KArgs* out) {
  using G = GemmShape<kGemmShape>;
  const bool b16 = io == IO_BF16;
  const int tm = b16 ? G::kTMW : 64, tn = b16 ? G::kTN : 64, kstep = b16 ? kTK : 16;
  const int fill = b16 ? 256 * G::kPerBlock : 512;  // workgroups resident on the chip
  int blocks = 0, all_tiles = 0;
  for (int q = 0; q < njobs; ++q) {
    KJob& k = out->job[q];
    k.j = jobs[q];
    k.tiles_n = (k.j.n + tn - 1) / tn;
    k.tiles = ((k.j.m + tm - 1) / tm) * k.tiles_n;
    all_tiles += k.tiles;
  }
  for (int q = 0; q < njobs; ++q) {
    KJob& k = out->job[q];
    int steps = 0;
    for (int s = 0; s < k.j.nseg; ++s) steps += (k.j.seg[s].k + kstep - 1) / kstep;
    // fp32 outputs split K (at least 8 steps per split) when the launch's tiles cannot fill
    // the chip; a job never gets more splits than it would alone (the workspace query
    // plans one job)
    k.splits = 1;
    if (k.j.part != nullptr && k.j.nseg == 1 && all_tiles < fill)
      k.splits = std::max(1, std::min(steps / 8, (fill + k.tiles - 1) / k.tiles));
    k.steps_per_split = (steps + k.splits - 1) / k.splits;
    k.splits = (steps + k.steps_per_split - 1) / k.steps_per_split;  // no empty split
    k.block_begin = blocks;
    blocks += k.tiles * k.splits;
  }
  out->njobs = njobs;
  return blocks;
}

}  // namespace

size_t gemm_partial_floats(IoType io, const GemmJob& job) {
  KArgs a{};
  GemmJob j = job;
  j.part = reinterpret_cast<float*>(16);  // any non-null: split allowed
  plan_jobs(io, &j, 1, &a);
  return a.job[0].splits > 1 ? (size_t)a.job[0].splits * j.m * j.n : 0;
}

hipError_t launch_gemm(IoType io, int form, int out, const GemmJob* jobs, int njobs, int S,
                       int hd, hipStream_t stream) {
  if (njobs < 1 || njobs > kGemmMaxJobs) return hipErrorInvalidValue;
  KArgs a{};
  a.S = S;
  a.hd = hd;
  const int blocks = plan_jobs(io, jobs, njobs, &a);
  hipError_t e;
  ProfScope prof(io == IO_BF16 ? "proj_gemm" : "proj_gemm_f32", stream);
  const dim3 block(256);
  if (form == GEMM_NN) e = launch_form<GEMM_NN>(io, out, a, blocks, block, stream);
  else if (form == GEMM_NT) e = launch_form<GEMM_NT>(io, out, a, blocks, block, stream);
  else e = launch_form<GEMM_TN>(io, out, a, blocks, block, stream);
  if (e != hipSuccess) return e;
  bool split = false;
  size_t most = 0;
  for (int q = 0; q < njobs; ++q) {
    split = split || a.job[q].splits > 1;
    most = std::max(most, (size_t)jobs[q].m * jobs[q].n / 4);
  }
  if (!split) return hipSuccess;
  ProfScope prof2("proj_gemm_splitk_sum", stream);
  hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)((most + 255) / 256), njobs), dim3(256),
                     0, stream, a);
  return hipPeekAtLastError();
}

}  // namespace xattn
