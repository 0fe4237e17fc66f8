// Causal GQA attention for bf16 io at head_dim 64 and 128 (the dim768 and long-context
// shapes), forward and backward, tuned for gfx950.  Same mathematics as attn.hip
// (Mint documentation 5.3.1; xtrain "Phase T9: Export to xserv" conventions table;
// xtrain "Phase T15: GQA" head mapping and deterministic group sum), restructured for
// throughput:
//
//   * HBM -> LDS staging with gfx950 direct-to-LDS loads (global_load_lds_dwordx4): no
//     register round trip, issued one or two tiles ahead so loads overlap the MFMA work.
//     A wave-level load writes 64 x 16 contiguous bytes, so tile rows are unpadded and
//     bank conflicts are avoided by XOR-swizzling the 16-byte chunks of each row.
//   * One barrier per stage: the wait for this stage's loads (vmcnt), the barrier and an
//     LDS-only acquire fence; no release fence (it would drain the prefetches).
//   * Forward softmax rescales the output accumulator only when the running max grows by
//     more than 2^8 (exact: numerator and denominator use the same reference max).
//   * dk/dv: when the KV tiles are too few to fill the machine, each wave of a workgroup
//     streams its own interleaved query tiles through private LDS buffers (no barriers in
//     the main loop); the four partial dK/dV are added in wave order at the end.
//   * Work is mapped to blocks so that the blocks of one KV head land on one XCD (its L2),
//     heaviest causal tiles first.
#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// XOR swizzle of the 16-byte chunks of a bf16 row of HD elements.  For HD = 128 the 16
// rows read together by a 16-lane LDS phase get 16 distinct chunk positions, and the four
// rows read by a transposing read phase get disjoint 64-byte windows; HD = 64 (two rows per
// 256-byte bank window) is arranged the same way.
template <int HD>
struct Sw {
  static constexpr int CPR = HD / 8;
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (HD == 128) return 4 * (row & 3) + ((row >> 2) & 3);
    else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  }
  __device__ static __forceinline__ int at(int row, int col) {
    return row * HD + ((((col >> 3) ^ swz(row))) << 3) + (col & 7);
  }
};

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void lds_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// Direct HBM -> LDS copy of rows g0 .. g0+ROWS-1 of a [S, HD] bf16 matrix (rows past the
// end re-read row S-1; callers mask them) into a swizzled tile, shared by NW waves.
template <int HD, int ROWS, int NW>
__device__ __forceinline__ void dma_rows(bf16* tile, const bf16* __restrict__ src, int g0,
                                         int S, int wv, int lane) {
  constexpr int CPR = HD / 8;
  constexpr int PER = ROWS * CPR / (64 * NW);
  static_assert(ROWS * CPR % (64 * NW) == 0, "tile must split into whole wave loads");
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p0 = (wv * PER + j) * 64;
    const int p = p0 + lane;
    const int row = p / CPR;
    const int c = (p % CPR) ^ Sw<HD>::swz(row);
    const int gr = min(g0 + row, S - 1);
    __builtin_amdgcn_global_load_lds(src + (size_t)gr * HD + c * 8,
                                     (lds_void_t*)(tile + p0 * 8), 16, 0, 0);
  }
}

// Per-query fp32 pair (lse2, delta) for 32 rows q0.. into LDS: [0,32) lse2, [32,64) delta.
// NW waves share it: wave wv moves entries wv*64/NW .. with 4-byte loads.
template <int NW>
__device__ __forceinline__ void dma_rowstats(float* dst, const float* __restrict__ lse2,
                                             const float* __restrict__ delta, int q0, int S,
                                             int wv, int lane) {
  constexpr int PER = 64 / NW;
  if (lane < PER) {
    const int e = wv * PER + lane;
    const int r = min(q0 + (e & 31), S - 1);
    const float* src = (e < 32 ? lse2 : delta) + r;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst + wv * PER), 4, 0, 0);
  }
}

template <int HD>
__device__ __forceinline__ bf16x8 lds_rows_a(const bf16* tile, int row0, int c, int lane) {
  const int row = row0 + (lane & 31);
  return *reinterpret_cast<const bf16x8*>(
      tile + row * HD + (((2 * c + (lane >> 5)) ^ Sw<HD>::swz(row)) << 3));
}

// sum over hd of tile rows row0..row0+31 (A) with the lane's register fragment (B)
template <int HD>
__device__ __forceinline__ f32x16 contract_rows(const bf16* tile, int row0,
                                                const bf16x8 (&frag)[HD / 16], int lane) {
  f32x16 acc = zero16();
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) acc = mfma_bf16(lds_rows_a<HD>(tile, row0, c, lane), frag[c], acc);
  return acc;
}

// A operand contracted over the tile's row index: rows row0+16*c2+4h+{0..3, 8..11},
// column 32*dt + (lane % 32).
template <int HD>
__device__ __forceinline__ bf16x8 lds_tr_a(const bf16* tile, int row0, int c2, int dt,
                                           int lane) {
  const int g = lane >> 4, li = lane & 15, h = lane >> 5;
  const int row = row0 + 16 * c2 + 4 * h + (li >> 2);
  const int col = 32 * dt + 16 * (g & 1) + 4 * (li & 3);
  const bf16x4 lo = lds_read_tr16(tile + Sw<HD>::at(row, col));
  const bf16x4 hi = lds_read_tr16(tile + Sw<HD>::at(row + 8, col));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int HD>
__device__ __forceinline__ void acc_tr(f32x16 (&acc)[HD / 32], const bf16* tile, int row0,
                                       const float (&pv)[16], int lane) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    bf16x8 b;
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = (bf16)pv[8 * c2 + j];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
      acc[dt] = mfma_bf16(lds_tr_a<HD>(tile, row0, c2, dt, lane), b, acc[dt]);
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

constexpr int kBM = 128;  // queries per forward / dq block (4 waves x 32)
constexpr int kBN = 64;   // keys per stage

// ---------------------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------------------
template <int HD, int NBUF>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const bf16* __restrict__ q,
                                                     const bf16* __restrict__ k,
                                                     const bf16* __restrict__ v,
                                                     bf16* __restrict__ out,
                                                     float* __restrict__ lse, int S, int H,
                                                     int Hkv, float scale_log2, int nqt,
                                                     int xcd) {
  constexpr int TILE = kBN * HD;
  constexpr int NL = 2 * (kBN * HD / 8) / 256;  // loads per wave per stage (K and V)
  __shared__ __attribute__((aligned(1024))) bf16 lds[NBUF][2][TILE];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = gridDim.x / nqt;
  const QMap mp = map_qblock(blockIdx.x, BH, H, Hkv, nqt, xcd != 0);
  const int bh = mp.bh, b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const bf16* kp = k + (size_t)kvbh * S * HD;
  const bf16* vp = v + (size_t)kvbh * S * HD;
  const int q0 = mp.qt * kBM, qw0 = q0 + 32 * wv, qrow = qw0 + c32;

  bf16x8 qf[HD / 16];
  load_frag<HD>(qf, q + (size_t)bh * S * HD, qrow, S, lane);
  f32x16 o[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) o[dt] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (min(S, q0 + kBM) + kBN - 1) / kBN;
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < ntiles) {
      dma_rows<HD, kBN, 4>(lds[t][0], kp, t * kBN, S, wv, lane);
      dma_rows<HD, kBN, 4>(lds[t][1], vp, t * kBN, S, wv, lane);
    }
  for (int kt = 0; kt < ntiles; ++kt) {
    if (NBUF > 2 && kt + 1 < ntiles) stage_barrier<(NBUF > 2 ? NL : 0)>();
    else stage_barrier<0>();
    const int nxt = kt + NBUF - 1;
    if (nxt < ntiles) {
      dma_rows<HD, kBN, 4>(lds[nxt % NBUF][0], kp, nxt * kBN, S, wv, lane);
      dma_rows<HD, kBN, 4>(lds[nxt % NBUF][1], vp, nxt * kBN, S, wv, lane);
    }
    const bf16* ks = lds[kt % NBUF][0];
    const bf16* vs = lds[kt % NBUF][1];
    const int k0 = kt * kBN;
#pragma unroll
    for (int s = 0; s < kBN / 32; ++s) {
      const int kb = k0 + 32 * s;
      if (kb > qw0 + 31 || kb >= S) break;  // wave-uniform
      const f32x16 st = contract_rows<HD>(ks, 32 * s, qf, lane);
      const bool edge = (kb + 31 > qw0) || (kb + 31 >= S);
      float sv[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = st[i];
        if (edge) {
          const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > qrow || key >= S) x = -INFINITY;
        }
        sv[i] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = fmaxf(tmax, shfl_xor(tmax, 32)) * scale_log2;
      // rescale only when the reference max grows by more than 2^8
      if (__any(tmax > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = fast_exp2(sv[i] * scale_log2 - m_run);
        psum += sv[i];
      }
      l_run += psum;
      acc_tr<HD>(o, vs, 32 * s, sv, lane);
    }
  }
  l_run += shfl_xor(l_run, 32);
  if (qrow < S) {
    store_col<bf16, HD>(out + ((size_t)bh * S + qrow) * HD, o, 1.0f / l_run, h);
    if (h == 0) lse[(size_t)bh * S + qrow] = (m_run + log2f(l_run)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------------
// backward, dq (+ per-query delta = dO . out and lse2 = lse * log2 e for the dk/dv kernel)
// ---------------------------------------------------------------------------------------
template <int HD, int NBUF, typename TG>
__global__ __launch_bounds__(256, 2) void dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ out, const bf16* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ lse2_out, float* __restrict__ delta, TG* __restrict__ dq, int S, int H,
    int Hkv, float scale_log2, float scale, int nqt, int xcd) {
  constexpr int TILE = kBN * HD;
  constexpr int NL = 2 * (kBN * HD / 8) / 256;
  __shared__ __attribute__((aligned(1024))) bf16 lds[NBUF][2][TILE];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = gridDim.x / nqt;
  const QMap mp = map_qblock(blockIdx.x, BH, H, Hkv, nqt, xcd != 0);
  const int bh = mp.bh, b = bh / H, qh = bh - b * H;
  const int kvbh = b * Hkv + qh / (H / Hkv);
  const bf16* kp = k + (size_t)kvbh * S * HD;
  const bf16* vp = v + (size_t)kvbh * S * HD;
  const int q0 = mp.qt * kBM, qw0 = q0 + 32 * wv, qrow = qw0 + c32;
  const size_t hoff = (size_t)bh * S * HD;

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
  const float D = dsum + shfl_xor(dsum, 32);
  const float lse2 = qrow < S ? lse[(size_t)bh * S + qrow] * kLog2e : 0.f;
  if (qrow < S && h == 0) {
    delta[(size_t)bh * S + qrow] = D;
    lse2_out[(size_t)bh * S + qrow] = lse2;
  }
  f32x16 acc[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) acc[dt] = zero16();

  const int ntiles = (min(S, q0 + kBM) + kBN - 1) / kBN;
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < ntiles) {
      dma_rows<HD, kBN, 4>(lds[t][0], kp, t * kBN, S, wv, lane);
      dma_rows<HD, kBN, 4>(lds[t][1], vp, t * kBN, S, wv, lane);
    }
  for (int kt = 0; kt < ntiles; ++kt) {
    if (NBUF > 2 && kt + 1 < ntiles) stage_barrier<(NBUF > 2 ? NL : 0)>();
    else stage_barrier<0>();
    const int nxt = kt + NBUF - 1;
    if (nxt < ntiles) {
      dma_rows<HD, kBN, 4>(lds[nxt % NBUF][0], kp, nxt * kBN, S, wv, lane);
      dma_rows<HD, kBN, 4>(lds[nxt % NBUF][1], vp, nxt * kBN, S, wv, lane);
    }
    const bf16* ks = lds[kt % NBUF][0];
    const bf16* vs = lds[kt % NBUF][1];
    const int k0 = kt * kBN;
#pragma unroll
    for (int s = 0; s < kBN / 32; ++s) {
      const int kb = k0 + 32 * s;
      if (kb > qw0 + 31 || kb >= S) break;
      const f32x16 st = contract_rows<HD>(ks, 32 * s, qf, lane);   // S^T
      const f32x16 dpt = contract_rows<HD>(vs, 32 * s, df, lane);  // dP^T
      const bool edge = (kb + 31 > qw0) || (kb + 31 >= S);
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(st[i] * scale_log2 - lse2);
        if (edge) {
          const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > qrow || key >= S) p = 0.f;
        }
        dsv[i] = p * (dpt[i] - D);
      }
      acc_tr<HD>(acc, ks, 32 * s, dsv, lane);  // dQ^T += K^T dS^T
    }
  }
  if (qrow < S) store_col<TG, HD>(dq + ((size_t)bh * S + qrow) * HD, acc, scale, h);
}

// ---------------------------------------------------------------------------------------
// backward, dk/dv
// ---------------------------------------------------------------------------------------
constexpr int kBQ = 32;  // queries per dk/dv stage

// One 32x32 (queries x keys) step of the dk/dv recurrence on a staged Q / dO tile.
template <int HD>
__device__ __forceinline__ void dkdv_step(f32x16 (&dkt)[HD / 32], f32x16 (&dvt)[HD / 32],
                                          const bf16* qs, const bf16* dos, const float* stats,
                                          const bf16x8 (&kf)[HD / 16],
                                          const bf16x8 (&vf)[HD / 16], int q0, int key,
                                          int kw0, int S, float scale_log2, int lane) {
  const int h = lane >> 5;
  const f32x16 st = contract_rows<HD>(qs, 0, kf, lane);    // S: queries x keys
  const f32x16 dpt = contract_rows<HD>(dos, 0, vf, lane);  // dP
  const bool edge = (q0 < kw0 + 31) || (q0 + kBQ > S);
  float pv[16], dsv[16];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int m0 = 8 * g + 4 * h;
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(stats + m0);
    const f32x4 dd = *reinterpret_cast<const f32x4*>(stats + 32 + m0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * g + j;
      float p = fast_exp2(st[i] * scale_log2 - l2[j]);
      if (edge) {
        const int qi = q0 + m0 + j;
        if (qi < key || qi >= S) p = 0.f;
      }
      pv[i] = p;
      dsv[i] = p * (dpt[i] - dd[j]);
    }
  }
  acc_tr<HD>(dvt, dos, 0, pv, lane);  // dV^T += dO^T P
  acc_tr<HD>(dkt, qs, 0, dsv, lane);  // dK^T += Q^T dS
}

// Shared variant: 4 waves own 128 consecutive keys of one KV head and share each staged
// 32-query tile of every query head of the group.
template <int HD, int NBUF, typename TG>
__global__ __launch_bounds__(256, 1) void dkdv_shared_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, TG* __restrict__ dk, bf16* __restrict__ dv, int S, int H,
    int Hkv, float scale_log2, float scale, int nkt, int xcd) {
  constexpr int TILE = kBQ * HD;
  constexpr int NL = 2 * (kBQ * HD / 8) / 256 + 1;
  __shared__ __attribute__((aligned(1024))) bf16 lds[NBUF][2][TILE];
  __shared__ __attribute__((aligned(16))) float stats[NBUF][64];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BKV = gridDim.x / nkt;
  int kvbh, kt;
  if (xcd) {
    const int lin = blockIdx.x, x = lin & 7, slot = lin >> 3, per = BKV / 8;
    kt = slot / per;
    kvbh = x + 8 * (slot % per);
  } else {
    kvbh = blockIdx.x % BKV;
    kt = blockIdx.x / BKV;
  }
  const int b = kvbh / Hkv, kvh = kvbh - b * Hkv, group = H / Hkv;
  const int k0 = kt * 128, kw0 = k0 + 32 * wv, key = kw0 + c32;
  bf16x8 kf[HD / 16], vf[HD / 16];
  load_frag<HD>(kf, k + (size_t)kvbh * S * HD, key, S, lane);
  load_frag<HD>(vf, v + (size_t)kvbh * S * HD, key, S, lane);
  f32x16 dkt[HD / 32], dvt[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) dkt[dt] = dvt[dt] = zero16();

  const int qt_first = k0 / kBQ, nqt = (S + kBQ - 1) / kBQ;
  const int per_r = nqt - qt_first;
  const int nst = group * per_r;
  auto issue = [&](int t, int buf) {
    const int r = t / per_r, qt = qt_first + t % per_r;
    const int bh = b * H + kvh * group + r;
    dma_rows<HD, kBQ, 4>(lds[buf][0], q + (size_t)bh * S * HD, qt * kBQ, S, wv, lane);
    dma_rows<HD, kBQ, 4>(lds[buf][1], dout + (size_t)bh * S * HD, qt * kBQ, S, wv, lane);
    dma_rowstats<4>(stats[buf], lse2 + (size_t)bh * S, delta + (size_t)bh * S, qt * kBQ, S,
                    wv, lane);
  };
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < nst) issue(t, t);
  for (int t = 0; t < nst; ++t) {
    if (NBUF > 2 && t + 1 < nst) stage_barrier<(NBUF > 2 ? NL : 0)>();
    else stage_barrier<0>();
    if (t + NBUF - 1 < nst) issue(t + NBUF - 1, (t + NBUF - 1) % NBUF);
    const int q0 = (qt_first + t % per_r) * kBQ;
    if (kw0 < S && q0 + kBQ - 1 >= kw0)
      dkdv_step<HD>(dkt, dvt, lds[t % NBUF][0], lds[t % NBUF][1], stats[t % NBUF], kf, vf, q0,
                    key, kw0, S, scale_log2, lane);
  }
  if (key < S) {
    store_col<TG, HD>(dk + ((size_t)kvbh * S + key) * HD, dkt, scale, h);
    store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
  }
}

// Private variant: 4 waves own the same 32 keys of one KV head; wave w walks query tiles
// w, w+4, w+8, ... (of every query head of the group, r ascending) through its own LDS
// buffers, so the main loop needs no barrier.  Partials are added in wave order.
template <int HD, int NBUF, typename TG>
__global__ __launch_bounds__(256, 1) void dkdv_private_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, TG* __restrict__ dk, bf16* __restrict__ dv, int S, int H,
    int Hkv, float scale_log2, float scale, int nkt, int xcd) {
  constexpr int TILE = kBQ * HD;
  constexpr int NL = 2 * (kBQ * HD / 8) / 64 + 1;
  __shared__ __attribute__((aligned(1024))) bf16 lds[4][NBUF][2][TILE];
  __shared__ __attribute__((aligned(16))) float stats[4][NBUF][64];
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BKV = gridDim.x / nkt;
  int kvbh, kt;
  if (xcd) {
    const int lin = blockIdx.x, x = lin & 7, slot = lin >> 3, per = BKV / 8;
    kt = slot / per;
    kvbh = x + 8 * (slot % per);
  } else {
    kvbh = blockIdx.x % BKV;
    kt = blockIdx.x / BKV;
  }
  const int b = kvbh / Hkv, kvh = kvbh - b * Hkv, group = H / Hkv;
  const int kw0 = kt * 32, key = kw0 + c32;
  bf16x8 kf[HD / 16], vf[HD / 16];
  load_frag<HD>(kf, k + (size_t)kvbh * S * HD, key, S, lane);
  load_frag<HD>(vf, v + (size_t)kvbh * S * HD, key, S, lane);
  f32x16 dkt[HD / 32], dvt[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) dkt[dt] = dvt[dt] = zero16();

  const int qt_first = kw0 / kBQ, nqt = (S + kBQ - 1) / kBQ;
  const int per_r = (nqt - qt_first - wv + 3) / 4;  // this wave's tiles per query head
  const int nst = group * per_r;
  auto issue = [&](int t, int buf) {
    const int r = t / per_r, qt = qt_first + wv + 4 * (t % per_r);
    const int bh = b * H + kvh * group + r;
    dma_rows<HD, kBQ, 1>(lds[wv][buf][0], q + (size_t)bh * S * HD, qt * kBQ, S, 0, lane);
    dma_rows<HD, kBQ, 1>(lds[wv][buf][1], dout + (size_t)bh * S * HD, qt * kBQ, S, 0, lane);
    dma_rowstats<1>(stats[wv][buf], lse2 + (size_t)bh * S, delta + (size_t)bh * S, qt * kBQ,
                    S, 0, lane);
  };
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < nst) issue(t, t);
  for (int t = 0; t < nst; ++t) {
    if (NBUF > 2 && t + 1 < nst) stage_wait_private<(NBUF > 2 ? NL : 0)>();
    else stage_wait_private<0>();
    if (t + NBUF - 1 < nst) issue(t + NBUF - 1, (t + NBUF - 1) % NBUF);
    const int q0 = (qt_first + wv + 4 * (t % per_r)) * kBQ;
    dkdv_step<HD>(dkt, dvt, lds[wv][t % NBUF][0], lds[wv][t % NBUF][1], stats[wv][t % NBUF],
                  kf, vf, q0, key, kw0, S, scale_log2, lane);
  }

  // wave-ordered combination of the four partials, one 32-row tile of one tensor at a time
  float* red = reinterpret_cast<float*>(&lds[0][0][0][0]);
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
  if (wv == 0 && key < S) {
    store_col<TG, HD>(dk + ((size_t)kvbh * S + key) * HD, dkt, scale, h);
    store_col<bf16, HD>(dv + ((size_t)kvbh * S + key) * HD, dvt, 1.0f, h);
  }
}

constexpr int kFwdBuf = 2;
constexpr int kDqBuf = 2;
constexpr int kDkdvSharedBuf = 3;
constexpr int kDkdvPrivateBuf = 2;

template <int HD>
hipError_t fwd_launch(const AttnShape& s, const void* q, const void* k, const void* v, void* out,
                      float* lse, hipStream_t stream) {
  const int nqt = (s.seq_len + kBM - 1) / kBM;
  const int BH = s.batch * s.num_heads;
  const int BKV = s.batch * s.num_kv_heads;
  const int xcd = (BKV % 8 == 0) ? 1 : 0;
  ProfScope prof("attn_fwd", stream);
  hipLaunchKernelGGL((fwd_kernel<HD, kFwdBuf>), dim3(BH * nqt), dim3(256), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)out, lse, s.seq_len,
                     s.num_heads, s.num_kv_heads, kLog2e / sqrtf((float)HD), nqt, xcd);
  return hipPeekAtLastError();
}

template <int HD, typename TG>
hipError_t bwd_launch(const AttnShape& s, const void* q, const void* k, const void* v,
                      const void* out, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* delta, float* lse2, hipStream_t stream) {
  const int S = s.seq_len;
  const int nqt = (S + kBM - 1) / kBM;
  const int BH = s.batch * s.num_heads;
  const int BKV = s.batch * s.num_kv_heads;
  const int xcd = (BKV % 8 == 0) ? 1 : 0;
  const float scale = 1.0f / sqrtf((float)HD), sl2 = kLog2e * scale;
  {
    ProfScope prof("attn_bwd_dq", stream);
    hipLaunchKernelGGL((dq_kernel<HD, kDqBuf, TG>), dim3(BH * nqt), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)out,
                       (const bf16*)dout, lse, lse2, delta, (TG*)dq, S, s.num_heads,
                       s.num_kv_heads, sl2, scale, nqt, xcd);
  }
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  const long long shared_blocks = (long long)BKV * ((S + 127) / 128);
  ProfScope prof("attn_bwd_dkdv", stream);
  if (shared_blocks >= 1024) {
    const int nkt = (S + 127) / 128;
    hipLaunchKernelGGL((dkdv_shared_kernel<HD, kDkdvSharedBuf, TG>), dim3(BKV * nkt), dim3(256),
                       0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                       (const bf16*)dout, (const float*)lse2, (const float*)delta, (TG*)dk,
                       (bf16*)dv, S, s.num_heads, s.num_kv_heads, sl2, scale, nkt, xcd);
  } else {
    const int nkt = (S + 31) / 32;
    hipLaunchKernelGGL((dkdv_private_kernel<HD, kDkdvPrivateBuf, TG>), dim3(BKV * nkt),
                       dim3(256), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                       (const bf16*)dout, (const float*)lse2, (const float*)delta, (TG*)dk,
                       (bf16*)dv, S, s.num_heads, s.num_kv_heads, sl2, scale, nkt, xcd);
  }
  return hipPeekAtLastError();
}

}  // namespace

bool fast_bf16_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_attn_fwd_bf16_fast(const AttnShape& s, const void* q, const void* k,
                                     const void* v, void* out, float* lse, hipStream_t stream) {
  if (s.head_dim == 128) return fwd_launch<128>(s, q, k, v, out, lse, stream);
  if (s.head_dim == 64) return fwd_launch<64>(s, q, k, v, out, lse, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_bf16_fast(const AttnShape& s, const void* q, const void* k,
                                     const void* v, const void* out, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv,
                                     float* delta, float* lse2, bool grads_f32,
                                     hipStream_t stream) {
#define XATTN_CASE(HD, TG)                                                                \
  return bwd_launch<HD, TG>(s, q, k, v, out, lse, dout, dq, dk, dv, delta, lse2, stream);
  if (s.head_dim == 128) {
    if (grads_f32) { XATTN_CASE(128, float) }
    XATTN_CASE(128, bf16)
  }
  if (s.head_dim == 64) {
    if (grads_f32) { XATTN_CASE(64, float) }
    XATTN_CASE(64, bf16)
  }
#undef XATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
