// KV-cache decode attention: a few new tokens per sequence attend to every cached key.
//
// What is computed (Mint documentation 10.3 "KV cache": each new token computes its own
// Q/K/V, its K/V are appended to the layer's cache in place, and its query attends to all
// cached keys, which are causal by construction; the result equals full-sequence attention.
// Mint 14.2 item 5: per-head extract / RoPE / append / attention launches dominate a GPU
// decode step, so they are merged):
//   for new token i in [0, Sq) of sequence b at absolute position t = pos + i:
//     q, k = QK-norm + RoPE at position t (the prologue forward of the training path),
//     k and v are written to cache row t of their KV head,
//     out = softmax_j(q . k_j / sqrt(hd)) v_j over cache rows j <= t, lse = ln sum exp.
//
// Layout on MI355X.  Decode reads the whole cache once and holds only (group x Sq) query
// rows per KV head, so it is bound by HBM bandwidth: a KV head's cache is split into key
// ranges, one wave per (KV head, range, up to 16 query rows), and the ranges are combined in
// range order by a second launch, so the result is bitwise reproducible.  The prologue
// forward runs inside the split launch: each wave normalises and rotates its query rows, and
// the waves whose range holds a new token's row write that token's rotated key and its value
// into the caches before streaming the range (their own loads then read them back).  Per
// sequence cache lengths (device array) set each sequence's positions and key count.
// Three split kernels: bf16 with head dim 64 / 128 on the matrix cores (2c), bf16 with
// head dim 16 / 32 with bf16 dot products (2b), fp32 on the VALU (2); one combine (3).
#include <math.h>

#include <type_traits>

#include "xattn_device.h"
#include "xattn_internal.h"

namespace xattn {
namespace {

struct DecodeArgs {
  const void* xq;        // [B*H, Sq, HD] raw new queries
  const void* xk;        // [B*Hkv, Sq, HD] raw new keys
  const void* v;         // [B*Hkv, Sq, HD] new values
  const float* gamma_q;  // [HD]
  const float* gamma_k;  // [HD]
  const float* cos_tab;  // [cap, HD/2]
  const float* sin_tab;  // [cap, HD/2]
  void* k_cache;         // [B*Hkv, cap, HD]
  void* v_cache;         // [B*Hkv, cap, HD]
  void* out;             // [B*H, Sq, HD]
  float* lse;            // [B*H*Sq]
  float* part_o;         // workspace [B*Hkv][nsplit][R][HD]
  float* part_ml;        // workspace [B*Hkv][nsplit][R][2]: running max (log2 units), sum
  const int* cache_lens;  // [B] cached rows per sequence, or null: every sequence has pos
  int B, H, Hkv, Sq, pos, cap, nsplit, ks;  // ks: keys per range
  int nchunk;             // waves per (KV head, range): the query rows in chunks of RM
  float eps, scale_log2;
};

// Cached rows of sequence b: its own length, clamped so that its new rows stay inside the
// cache (a bad length gives wrong results but no access outside the tensors).
__device__ __forceinline__ int seq_pos(const DecodeArgs& a, int b) {
  return a.cache_lens != nullptr ? min(max(a.cache_lens[b], 0), a.cap - a.Sq) : a.pos;
}

// Sum over each aligned group of N consecutive lanes (N a power of two up to 64), the same
// bits in every lane of the group: DPP quad permutations, the half-row and row mirrors
// (each pairs a lane with one in the other half of its 8- or 16-lane group), then xor
// exchanges across rows.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v += dpp_mov<0x140>(v); // row_mirror
  if constexpr (N >= 32) v += xor_lanes<16>(v);
  if constexpr (N >= 64) v += xor_lanes<32>(v);
  return v;
}

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* p, float (&out)[N]) {
  constexpr int per = V16<T>::n;
#pragma unroll
  for (int k = 0; k < N / per; ++k) {
    const vec16_t<T> w = load16(p + k * per);
#pragma unroll
    for (int j = 0; j < per; ++j) out[k * per + j] = to_f32(w[j]);
  }
}

// ---------------------------------------------------------------------------------------
// 1. prologue forward in the split kernel's lane layout.  A row of HD columns is spread over
// LPK lanes, lane part p holding columns [p*VEC, p*VEC + VEC); the partner of column c
// (c < HD/2) in its rotation pair is c + HD/2, held by part p + LPK/2.  Returns the lane's
// VEC columns of y = rotate_t(gamma * x * rsqrt(mean x^2 + eps)) rounded to the io dtype
// (the prologue forward's arithmetic: normalise, scale by gamma, rotate by the angles of
// position t).
// ---------------------------------------------------------------------------------------
template <typename T, int HD>
__device__ __forceinline__ void prologue_lanes(const T* __restrict__ xrow,
                                               const float* __restrict__ gamma,
                                               const float* __restrict__ cos_tab,
                                               const float* __restrict__ sin_tab, int t,
                                               float eps, int part, float (&y)[V16<T>::n]) {
  constexpr int VEC = V16<T>::n, LPK = HD / VEC, HALF = HD / 2, PH = LPK / 2;
  static_assert(HALF % VEC == 0, "each half spans whole lane parts");
  float x[VEC], g[VEC], cs[VEC], sn[VEC];
  load_vec<T, VEC>(xrow + part * VEC, x);
  const int cp = (part % PH) * VEC;  // column of the pair's first-half member
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    g[e] = gamma[part * VEC + e];
    cs[e] = cos_tab[(size_t)t * HALF + cp + e];
    sn[e] = sin_tab[(size_t)t * HALF + cp + e];
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) ss += x[e] * x[e];
  ss = lane_group_sum<LPK>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / (float)HD) + eps);
  const bool first = part < PH;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float n = x[e] * r * g[e];
    const float m = xor_lanes<PH>(n);  // the pair's other member
    const float n1 = first ? n : m, n2 = first ? m : n;
    const float v = first ? n1 * cs[e] - n2 * sn[e] : n1 * sn[e] + n2 * cs[e];
    y[e] = to_f32(from_f32<T>(v));
  }
}

// ---------------------------------------------------------------------------------------
// 2. split attention.  Wave w = (KV row bkv, row chunk ch, range sp) handles cache rows
// [sp*ks, min(Lk, sp*ks + ks)), Lk = pos + Sq (pos: the sequence's cached rows), for the
// query rows r = ch*RM .. ch*RM + RM - 1 of the KV head; query row r = g*Sq + i (g < group,
// i < Sq) is query head kvh*group + g at position pos + i and sees cache rows j <= pos + i.
// Lane l owns the VEC columns part = l % LPK of the key rows j0 + l / LPK (KPW keys per wave
// load); each lane group keeps its own (max, sum, accumulator) per query row, merged at the
// end.  When the rows of a KV head take several chunks, each chunk's wave streams the range
// again (mostly from L2: the chunks of a range are neighbouring waves).
// ---------------------------------------------------------------------------------------
constexpr int kDecodeUnroll = 4;  // wave loads of K and of V in flight per lane

template <typename T, int HD, int RM>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int VEC = V16<T>::n, LPK = HD / VEC, KPW = 64 / LPK, UN = kDecodeUnroll;
  const int lane = threadIdx.x & 63;
  // the wave's index is wave-uniform: in a scalar register, so is everything derived from it
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= a.B * a.Hkv * a.nchunk * a.nsplit) return;  // whole waves; no barrier
  const int bkv = w / (a.nchunk * a.nsplit), rem = w - bkv * (a.nchunk * a.nsplit);
  const int sp = rem / a.nchunk, ch = rem - sp * a.nchunk;  // a range's chunks: neighbours
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv, group = a.H / a.Hkv;
  const int pos = seq_pos(a, b);
  const int R = group * a.Sq, Lk = pos + a.Sq;
  const int r0 = ch * RM, nr = min(RM, R - r0);  // this wave's query rows
  const int k0 = sp * a.ks, k1 = min(Lk, k0 + a.ks);
  const int part = lane % LPK, kg = lane / LPK;
  // a wave whose range holds no new token issues its first loads now, under the prologue
  const int n0 = max(k0, pos);
  const bool appends = n0 < k1;  // wave-uniform
  const T* kc = static_cast<const T*>(a.k_cache) + (size_t)bkv * a.cap * HD + part * VEC;
  const T* vc = static_cast<const T*>(a.v_cache) + (size_t)bkv * a.cap * HD + part * VEC;

  // the lane's 16 bytes of UN key / value rows; the next group's loads are issued before
  // the current group's arithmetic
  vec16_t<T> kv[UN], vv[UN], kn[UN], vn[UN];
  auto load_group = [&](int j0, vec16_t<T> (&kk)[UN], vec16_t<T> (&vk)[UN]) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * KPW + kg;
      const size_t jr = (size_t)(j < k1 ? j : k0) * HD;  // past the range: a row of it
      kk[u] = load16(kc + jr);
      vk[u] = load16(vc + jr);
    }
  };
  if (!appends) load_group(k0, kv, vv);

  float q[RM][VEC];
  int lim[RM];  // last visible cache row of each query row (-1: padding row)
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    lim[r] = -1;
#pragma unroll
    for (int e = 0; e < VEC; ++e) q[r][e] = 0.f;
    if (r < nr) {  // wave-uniform
      const int g = (r0 + r) / a.Sq, i = (r0 + r) - g * a.Sq;
      const T* xr = static_cast<const T*>(a.xq) +
                    ((size_t)(b * a.H + kvh * group + g) * a.Sq + i) * HD;
      prologue_lanes<T, HD>(xr, a.gamma_q, a.cos_tab, a.sin_tab, pos + i, a.eps, part, q[r]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[r][e] *= a.scale_log2;
      lim[r] = pos + i;
    }
  }
  // Append: the new tokens' rows of this range (cache rows pos .. pos + Sq - 1 that fall in
  // [k0, k1)) get the rotated key and the value, KPW rows per pass; then the stores are
  // made visible to this wave's own loads below.  Every row chunk's wave of the range
  // writes them (the same bytes), so each reads back rows it has written itself.
  if (appends) {
    for (int j0 = n0; j0 < k1; j0 += KPW) {
      const int j = j0 + kg;
      const int i = (j < k1 ? j : n0) - pos;  // token (clamped for idle lanes)
      const size_t src = ((size_t)bkv * a.Sq + i) * HD;
      float yk[VEC];
      prologue_lanes<T, HD>(static_cast<const T*>(a.xk) + src, a.gamma_k, a.cos_tab,
                            a.sin_tab, pos + i, a.eps, part, yk);
      if (j < k1) {
        const size_t dst = ((size_t)bkv * a.cap + j) * HD + part * VEC;
        T* kd = static_cast<T*>(a.k_cache) + dst;
#pragma unroll
        for (int e = 0; e < VEC; ++e) kd[e] = from_f32<T>(yk[e]);
        store16(static_cast<T*>(a.v_cache) + dst,
                load16(static_cast<const T*>(a.v) + src + part * VEC));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    load_group(k0, kv, vv);
  }
  float m[RM], l[RM], o[RM][VEC];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[r][e] = 0.f;
  }
  for (int j0 = k0; j0 < k1; j0 += KPW * UN) {
    if (j0 + KPW * UN < k1) load_group(j0 + KPW * UN, kn, vn);  // wave-uniform
    int jj[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * KPW + kg;
      jj[u] = j < k1 ? j : 0x7fffffff;  // past the range: never visible
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r < nr) {  // wave-uniform
      float s[UN];
      float smax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d += q[r][e] * to_f32(kv[u][e]);
        d = lane_group_sum<LPK>(d);
        s[u] = jj[u] <= lim[r] ? d : -INFINITY;
        smax = fmaxf(smax, s[u]);
      }
      const float mn = fmaxf(m[r], smax);
      // reference point: mn, or 0 while this lane group has seen no visible key (then
      // every term below is exp2(-inf) = 0 and the state stays empty)
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[r] - mref);  // 0 when m was -inf
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[r][e] *= alpha;
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const float p = fast_exp2(s[u] - mref);  // 0 for masked keys
        l[r] += p;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[r][e] += p * to_f32(vv[u][e]);
      }
      m[r] = mn;
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      kv[u] = kn[u];
      vv[u] = vn[u];
    }
  }

  // merge the lane groups (same columns, other keys): fixed xor butterfly
  auto merge = [&](auto mask_tag) {
    constexpr int MSK = decltype(mask_tag)::value;
    if constexpr (MSK >= LPK && MSK < 64) {
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        if (r >= nr) continue;  // wave-uniform
        const float mp = xor_lanes<MSK>(m[r]), lp = xor_lanes<MSK>(l[r]);
        const float mn = fmaxf(m[r], mp);
        const float a1 = m[r] == -INFINITY ? 0.f : fast_exp2(m[r] - mn);
        const float a2 = mp == -INFINITY ? 0.f : fast_exp2(mp - mn);
        l[r] = l[r] * a1 + lp * a2;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float op = xor_lanes<MSK>(o[r][e]);
          o[r][e] = o[r][e] * a1 + op * a2;
        }
        m[r] = mn;
      }
    }
  };
  merge(std::integral_constant<int, 1>{});
  merge(std::integral_constant<int, 2>{});
  merge(std::integral_constant<int, 4>{});
  merge(std::integral_constant<int, 8>{});
  merge(std::integral_constant<int, 16>{});
  merge(std::integral_constant<int, 32>{});
  if (kg != 0) return;
  const size_t base = ((size_t)bkv * a.nsplit + sp) * R + r0;
  {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= nr) continue;  // wave-uniform
      float* po = a.part_o + (base + r) * HD + part * VEC;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        f32x4 w4;
#pragma unroll
        for (int j = 0; j < 4; ++j) w4[j] = o[r][e + j];
        *reinterpret_cast<f32x4*>(po + e) = w4;
      }
      if (part == 0) {
        a.part_ml[(base + r) * 2] = m[r];
        a.part_ml[(base + r) * 2 + 1] = l[r];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// 2b. split attention, bf16 io.  The same waves, ranges and append as above, with the
// arithmetic on bf16 pairs: a key row of HD columns is spread over LPK = HD / 16 lanes, lane
// part p holding the 16 columns [8p, 8p + 8) and [HD/2 + 8p, HD/2 + 8p + 8) (two 16-byte
// loads), so every column's RoPE partner (c + HD/2) sits in the same lane and a dot product
// takes log2(LPK) lane exchanges.  Scores: bf16 q . k by dot2 with fp32 accumulation (the
// rotated q is rounded to bf16, as the prologue forward stores it).  P is rounded to bf16
// for P V, like the training forward, which takes dot2 over pairs of keys (the two keys'
// values of a column paired by a byte permute, shared by every query row).  The softmax
// reference of a row is raised only when a score exceeds it by more than 8 in log2 units
// (probabilities up to 2^8 cannot overflow the fp32 sums), so the accumulators are rescaled
// about once per range instead of once per key group.
// ---------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

struct Row16 {  // a lane's two 16-byte chunks of one row
  bf16x8 a, b;
};

template <int HD>
__device__ __forceinline__ Row16 load_row16(const bf16* row, int part) {
  return {load16(row + part * 8), load16(row + HD / 2 + part * 8)};
}

// Cache rows are streamed once per decode step (and a model's caches together exceed the
// last-level cache), so they are read with the non-temporal hint: they do not displace
// other data on the way, which measured 10 to 15 % faster for caches of 0.5 GB and more.
__device__ __forceinline__ bf16x8 load16_stream(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}
template <int HD>
__device__ __forceinline__ Row16 load_row16_stream(const bf16* row, int part) {
  return {load16_stream(row + part * 8), load16_stream(row + HD / 2 + part * 8)};
}

__device__ __forceinline__ bf16x2 as_pair(unsigned u) { return __builtin_bit_cast(bf16x2, u); }

// dot of the lane's 16 columns (fp32 accumulation)
__device__ __forceinline__ float dot16(const Row16& x, const Row16& y) {
  const u32x4 xa = __builtin_bit_cast(u32x4, x.a), xb = __builtin_bit_cast(u32x4, x.b);
  const u32x4 ya = __builtin_bit_cast(u32x4, y.a), yb = __builtin_bit_cast(u32x4, y.b);
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_fdot2_f32_bf16(as_pair(xa[i]), as_pair(ya[i]), d, false);
#pragma unroll
  for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_fdot2_f32_bf16(as_pair(xb[i]), as_pair(yb[i]), d, false);
  return d;
}

// The prologue forward on the lane's 16 columns: normalise the row, scale by gamma, rotate
// each pair (c, c + HD/2) by the angles of position t, round to bf16.
template <int HD>
__device__ __forceinline__ Row16 prologue_row16(const bf16* __restrict__ xrow,
                                                const float* __restrict__ gamma,
                                                const float* __restrict__ cos_tab,
                                                const float* __restrict__ sin_tab, int t,
                                                float eps, int part) {
  constexpr int LPK = HD / 16, HALF = HD / 2;
  const Row16 x = load_row16<HD>(xrow, part);
  float xa[8], xb[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    xa[e] = (float)x.a[e];
    xb[e] = (float)x.b[e];
    ss += xa[e] * xa[e];
    ss += xb[e] * xb[e];
  }
  ss = lane_group_sum<LPK>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / (float)HD) + eps);
  Row16 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = part * 8 + e;
    const float na = xa[e] * r * gamma[c], nb = xb[e] * r * gamma[HALF + c];
    const float cs = cos_tab[(size_t)t * HALF + c], sn = sin_tab[(size_t)t * HALF + c];
    y.a[e] = (bf16)(na * cs - nb * sn);
    y.b[e] = (bf16)(na * sn + nb * cs);
  }
  return y;
}

template <int HD, int RM>
__global__ __launch_bounds__(256) void decode_split_bf16_kernel(DecodeArgs a) {
  constexpr int LPK = HD / 16, KPW = 64 / LPK, HALF = HD / 2, UN = 2;
  static_assert(UN % 2 == 0, "keys are paired for P V");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= a.B * a.Hkv * a.nchunk * a.nsplit) return;  // whole waves; no barrier
  const int bkv = w / (a.nchunk * a.nsplit), rem = w - bkv * (a.nchunk * a.nsplit);
  const int sp = rem / a.nchunk, ch = rem - sp * a.nchunk;  // a range's chunks: neighbours
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv, group = a.H / a.Hkv;
  const int pos = seq_pos(a, b);
  const int R = group * a.Sq, Lk = pos + a.Sq;
  const int r0 = ch * RM, nr = min(RM, R - r0);
  const int k0 = sp * a.ks, k1 = min(Lk, k0 + a.ks);
  const int part = lane % LPK, kg = lane / LPK;
  const int n0 = max(k0, pos);
  const bool appends = n0 < k1;
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + (size_t)bkv * a.cap * HD;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + (size_t)bkv * a.cap * HD;

  constexpr int G = KPW * UN;  // keys per group
  Row16 kb[UN], vb[UN], k1b[UN], v1b[UN], k2b[UN], v2b[UN];
  auto load_group = [&](int j0, Row16 (&kk)[UN], Row16 (&vk)[UN]) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * KPW + kg;
      const size_t jr = (size_t)(j < k1 ? j : k0) * HD;  // past the range: a row of it
      kk[u] = load_row16_stream<HD>(kc + jr, part);
      vk[u] = load_row16_stream<HD>(vc + jr, part);
    }
  };
  auto load_first = [&] {
    load_group(k0, kb, vb);
    load_group(k0 + G, k1b, v1b);
    load_group(k0 + 2 * G, k2b, v2b);
  };
  if (!appends) load_first();

  Row16 q[RM];
  int lim[RM];  // last visible cache row of each query row (-1: padding row)
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    lim[r] = -1;
    q[r].a = bf16x8{};
    q[r].b = bf16x8{};
    if (r < nr) {
      const int g = (r0 + r) / a.Sq, i = (r0 + r) - g * a.Sq;
      const bf16* xr = static_cast<const bf16*>(a.xq) +
                       ((size_t)(b * a.H + kvh * group + g) * a.Sq + i) * HD;
      q[r] = prologue_row16<HD>(xr, a.gamma_q, a.cos_tab, a.sin_tab, pos + i, a.eps, part);
      lim[r] = pos + i;
    }
  }
  // append the new tokens' rows of this range (see the generic kernel)
  if (appends) {
    for (int j0 = n0; j0 < k1; j0 += KPW) {
      const int j = j0 + kg;
      const int i = (j < k1 ? j : n0) - pos;  // token (clamped for idle lanes)
      const size_t src = ((size_t)bkv * a.Sq + i) * HD;
      const Row16 yk = prologue_row16<HD>(static_cast<const bf16*>(a.xk) + src, a.gamma_k,
                                          a.cos_tab, a.sin_tab, pos + i, a.eps, part);
      if (j < k1) {
        const size_t dst = ((size_t)bkv * a.cap + j) * HD + part * 8;
        bf16* kd = static_cast<bf16*>(a.k_cache) + dst;
        bf16* vd = static_cast<bf16*>(a.v_cache) + dst;
        const Row16 vr = load_row16<HD>(static_cast<const bf16*>(a.v) + src, part);
        store16(kd, yk.a);
        store16(kd + HALF, yk.b);
        store16(vd, vr.a);
        store16(vd + HALF, vr.b);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    load_first();
  }

  float o[RM][16], l[RM], ref[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    ref[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[r][c] = 0.f;
  }
  const float sl2 = a.scale_log2;
  // one key group (KPW * UN keys) from the lane's registers kk / vk
  auto group_step = [&](int j0, const Row16 (&kk)[UN], const Row16 (&vk)[UN]) {
    int jj[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * KPW + kg;
      jj[u] = j < k1 ? j : 0x7fffffff;  // past the range: never visible
    }
    // values of key pairs (2u, 2u + 1) per column: vp[u][c] = (v_2u[c], v_2u+1[c])
    unsigned vp[UN / 2][16];
#pragma unroll
    for (int u = 0; u < UN / 2; ++u) {
      const u32x4 a0 = __builtin_bit_cast(u32x4, vk[2 * u].a);
      const u32x4 a1 = __builtin_bit_cast(u32x4, vk[2 * u + 1].a);
      const u32x4 b0 = __builtin_bit_cast(u32x4, vk[2 * u].b);
      const u32x4 b1 = __builtin_bit_cast(u32x4, vk[2 * u + 1].b);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vp[u][2 * i] = __builtin_amdgcn_perm(a1[i], a0[i], 0x05040100u);
        vp[u][2 * i + 1] = __builtin_amdgcn_perm(a1[i], a0[i], 0x07060302u);
        vp[u][8 + 2 * i] = __builtin_amdgcn_perm(b1[i], b0[i], 0x05040100u);
        vp[u][8 + 2 * i + 1] = __builtin_amdgcn_perm(b1[i], b0[i], 0x07060302u);
      }
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) {  // padding rows see no key (lim -1): p = 0
      float s[UN];
      float smax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const float d = lane_group_sum<LPK>(dot16(q[r], kk[u]));
        s[u] = jj[u] <= lim[r] ? d * sl2 : -INFINITY;
        smax = fmaxf(smax, s[u]);
      }
      const float nref = smax > ref[r] + 8.f ? smax : ref[r];
      if (__builtin_amdgcn_ballot_w64(nref != ref[r]) != 0) {  // wave-uniform
        const float alpha = nref == ref[r] ? 1.f : fast_exp2(ref[r] - nref);  // 0 from -inf
        l[r] *= alpha;
#pragma unroll
        for (int c = 0; c < 16; ++c) o[r][c] *= alpha;
        ref[r] = nref;
      }
      const float base = ref[r] == -INFINITY ? 0.f : ref[r];  // no visible key yet: p = 0
#pragma unroll
      for (int u = 0; u < UN / 2; ++u) {
        const float p0 = fast_exp2(s[2 * u] - base), p1 = fast_exp2(s[2 * u + 1] - base);
        l[r] += p0 + p1;
        const bf16x2 pp = {(bf16)p0, (bf16)p1};
#pragma unroll
        for (int c = 0; c < 16; ++c)
          o[r][c] = __builtin_amdgcn_fdot2_f32_bf16(pp, as_pair(vp[u][c]), o[r][c], false);
      }
    }
  };
  // Three register buffers in a ring: while one group is used, the next two are in flight
  // (loads complete in issue order, so a group waits only for its own).  Every trip runs all
  // three steps and issues all three loads, with no exit in between, so that each buffer
  // keeps its registers: groups past the range are masked out (their loads read a row of the
  // range).
  for (int j0 = k0; j0 < k1; j0 += 3 * G) {
    group_step(j0, kb, vb);
    load_group(j0 + 3 * G, kb, vb);
    group_step(j0 + G, k1b, v1b);
    load_group(j0 + 4 * G, k1b, v1b);
    group_step(j0 + 2 * G, k2b, v2b);
    load_group(j0 + 5 * G, k2b, v2b);
  }

  // merge the lane groups (same columns, other keys): fixed xor butterfly
  auto merge = [&](auto mask_tag) {
    constexpr int MSK = decltype(mask_tag)::value;
    if constexpr (MSK >= LPK && MSK < 64) {
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        if (r >= nr) continue;  // wave-uniform
        const float mp = xor_lanes<MSK>(ref[r]), lp = xor_lanes<MSK>(l[r]);
        const float mn = fmaxf(ref[r], mp);
        const float a1 = ref[r] == -INFINITY ? 0.f : fast_exp2(ref[r] - mn);
        const float a2 = mp == -INFINITY ? 0.f : fast_exp2(mp - mn);
        l[r] = l[r] * a1 + lp * a2;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const float op = xor_lanes<MSK>(o[r][c]);
          o[r][c] = o[r][c] * a1 + op * a2;
        }
        ref[r] = mn;
      }
    }
  };
  merge(std::integral_constant<int, 1>{});
  merge(std::integral_constant<int, 2>{});
  merge(std::integral_constant<int, 4>{});
  merge(std::integral_constant<int, 8>{});
  merge(std::integral_constant<int, 16>{});
  merge(std::integral_constant<int, 32>{});
  if (kg != 0) return;
  const size_t base = ((size_t)bkv * a.nsplit + sp) * R + r0;
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r >= nr) continue;  // wave-uniform
    float* po = a.part_o + (base + r) * HD + part * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        f32x4 w4;
#pragma unroll
        for (int j = 0; j < 4; ++j) w4[j] = o[r][8 * h + e + j];
        *reinterpret_cast<f32x4*>(po + h * HALF + e) = w4;
      }
    }
    if (part == 0) {
      a.part_ml[(base + r) * 2] = ref[r];
      a.part_ml[(base + r) * 2 + 1] = l[r];
    }
  }
}

// ---------------------------------------------------------------------------------------
// 2c. split attention, bf16 io, head dim 64 or 128, on the matrix cores.  The same waves,
// ranges and append; a wave holds 16 query rows of its KV head (rows past the head's count
// are zero padding), so a key tile of 16 keys is one 16 x 16 score block:
//   S^T (keys x rows) = K Q^T by v_mfma_f32_16x16x32_bf16 over the head dim, K from the
//   lane's registers (lane l: key l % 16, head-dim chunk 4t + l / 16, t < HD / 32), Q^T from
//   the rotated queries (lane l: row l % 16, the same chunks);
//   O^T (cols x rows) += V^T P^T by v_mfma_f32_16x16x16_bf16 per 16 output columns: the score
//   block's accumulator layout (lane l: row l % 16, keys 4 (l / 16) + v) is already the
//   layout of P^T as the second operand, and V^T comes from the key tile staged in LDS and
//   read back transposed (ds_read_b64_tr_b16).
// A lane thus holds one query row throughout (its scores, probabilities and output
// columns), a row's maximum takes two lane exchanges per tile, and the lane groups need no
// merge at the end: the key sums happen inside the matrix instructions.  P is rounded to
// bf16 for P V (like the training forward); the softmax reference is raised lazily as in the
// dot2 kernel.  K and V tiles stream through a ring of three register buffers.
// ---------------------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void decode_split_mfma_kernel(DecodeArgs a) {
  constexpr int RM = 16;         // query rows per wave
  constexpr int NT = HD / 32;    // score MFMAs per key tile (32 head-dim columns each)
  constexpr int NC = HD / 16;    // output MFMAs per key tile (16 columns each)
  constexpr int CPR = HD / 8;    // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;  // rows per 1 KiB wave load
  constexpr int NV = 16 / RPL;   // V loads per key tile
  constexpr int RB = HD * 2;     // bytes per row
  constexpr int HALF = HD / 2;
  constexpr int TILE_B = 16 * RB;
  static_assert(HD == 64 || HD == 128, "head dim 64 or 128");
  // two LDS V tiles per wave (the next tile is written while the last one's reads drain)
  __shared__ __align__(16) char lds_v[4][2][TILE_B];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wv);
  if (w >= a.B * a.Hkv * a.nchunk * a.nsplit) return;  // whole waves; no barrier
  const int bkv = w / (a.nchunk * a.nsplit), rem = w - bkv * (a.nchunk * a.nsplit);
  const int sp = rem / a.nchunk, ch = rem - sp * a.nchunk;  // a range's chunks: neighbours
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv, group = a.H / a.Hkv;
  const int pos = seq_pos(a, b);
  const int R = group * a.Sq, Lk = pos + a.Sq;
  const int r0 = ch * RM, nr = min(RM, R - r0);
  const int k0 = sp * a.ks, k1 = min(Lk, k0 + a.ks);
  const int n0 = max(k0, pos);
  const bool appends = n0 < k1;
  const int n = lane & 15, g = lane >> 4;  // query row and lane group
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + (size_t)bkv * a.cap * HD;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + (size_t)bkv * a.cap * HD;

  // the lane's share of one key tile: K as score operands, V rows as loaded
  struct Tile {
    bf16x8 k[NT];
    bf16x8 v[NV];
  };
  auto load_tile = [&](int j0, Tile& t) {
    {
      const int j = j0 + n;
      const size_t jr = (size_t)(j < k1 ? j : k0) * HD;  // past the range: a row of it
#pragma unroll
      for (int i = 0; i < NT; ++i) t.k[i] = load16_stream(kc + jr + 32 * i + 8 * g);
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int j = j0 + u * RPL + lane / CPR;
      const size_t jr = (size_t)(j < k1 ? j : k0) * HD;
      t.v[u] = load16_stream(vc + jr + 8 * (lane % CPR));
    }
  };
  Tile t0, t1, t2;
  // a wave whose range holds no new token issues its first tile before the query prologue
  // and the next two after it (the prologue's inputs and three tiles would not fit the
  // registers of two waves per SIMD at once)
  if (!appends) load_tile(k0, t0);

  // rotated queries, row n of the wave (zero for padding rows): the prologue forward with
  // the row spread over the four lane groups (chunk t holds columns 32t + 8g .. + 8; the
  // RoPE partner of chunk t < NT/2 is chunk t + NT/2 of the same lane)
  bf16x8 q[NT];
  int lim;  // last visible cache row of the lane's query row (-1: padding row)
  {
    const int rn = min(n, nr - 1);
    const int gq = (r0 + rn) / a.Sq, i = (r0 + rn) - gq * a.Sq;
    const bf16* xr = static_cast<const bf16*>(a.xq) +
                     ((size_t)(b * a.H + kvh * group + gq) * a.Sq + i) * HD;
    const int t_pos = pos + i;
    float x[NT][8];
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 xv = load16(xr + 32 * t + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[t][e] = (float)xv[e];
        ss += x[t][e] * x[t][e];
      }
    }
    ss += xor_lanes<16>(ss);
    ss += xor_lanes<32>(ss);
    const float rr = 1.0f / sqrtf(ss * (1.0f / (float)HD) + a.eps);
    const bool live = n < nr;
#pragma unroll
    for (int t = 0; t < NT / 2; ++t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * t + 8 * g + e;  // < HD / 2
        const float na = x[t][e] * rr * a.gamma_q[c];
        const float nb = x[t + NT / 2][e] * rr * a.gamma_q[c + HALF];
        const float cs = a.cos_tab[(size_t)t_pos * HALF + c];
        const float sn = a.sin_tab[(size_t)t_pos * HALF + c];
        q[t][e] = (bf16)(live ? na * cs - nb * sn : 0.f);
        q[t + NT / 2][e] = (bf16)(live ? na * sn + nb * cs : 0.f);
      }
    }
    lim = live ? t_pos : -1;
  }
  // append the new tokens' rows of this range (the dot2 kernel's lane layout: a row over
  // HD / 16 lanes, HD / 16 ... rows per pass), then make the stores visible to the loads
  if (appends) {
    constexpr int LPK = HD / 16, KPW = 64 / LPK;
    const int part = lane % LPK, kg = lane / LPK;
    for (int j0 = n0; j0 < k1; j0 += KPW) {
      const int j = j0 + kg;
      const int i = (j < k1 ? j : n0) - pos;  // token (clamped for idle lanes)
      const size_t src = ((size_t)bkv * a.Sq + i) * HD;
      const Row16 yk = prologue_row16<HD>(static_cast<const bf16*>(a.xk) + src, a.gamma_k,
                                          a.cos_tab, a.sin_tab, pos + i, a.eps, part);
      if (j < k1) {
        const size_t dst = ((size_t)bkv * a.cap + j) * HD + part * 8;
        bf16* kd = static_cast<bf16*>(a.k_cache) + dst;
        bf16* vd = static_cast<bf16*>(a.v_cache) + dst;
        const Row16 vr = load_row16<HD>(static_cast<const bf16*>(a.v) + src, part);
        store16(kd, yk.a);
        store16(kd + HALF, yk.b);
        store16(vd, vr.a);
        store16(vd + HALF, vr.b);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    load_tile(k0, t0);
  }
  load_tile(k0 + 16, t1);
  load_tile(k0 + 32, t2);

  f32x4 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float l = 0.f, ref = -INFINITY;
  const float sl2 = a.scale_log2;
  char* vbase = lds_v[wv][0];
  // LDS tile: row = key, 16-byte chunk c of a row stored at chunk c ^ 2 (row % (CPR / 2)),
  // so that the transposed reads (four rows x 32 bytes per 16 lanes) and the row writes
  // spread over all banks
  auto swz = [](int row) { return 2 * (row & (CPR / 2 - 1)); };
  auto tile_step = [&](int j0, const Tile& t, int slot) {
    char* vt_lds = vbase + slot * TILE_B;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int row = u * RPL + lane / CPR, c = lane % CPR;
      *reinterpret_cast<bf16x8*>(vt_lds + row * RB + ((c ^ swz(row)) << 4)) = t.v[u];
    }
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NT; ++i) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[i], q[i], st, 0, 0, 0);
    // the lane's scores: row n, keys j0 + 4g + v
    float s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + 4 * g + v;
      s[v] = (j < k1 && j <= lim) ? st[v] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, xor_lanes<16>(mx));
    mx = fmaxf(mx, xor_lanes<32>(mx));
    const float smax = mx * sl2;  // scaled to log2 units (sl2 > 0)
    const float nref = smax > ref + 8.f ? smax : ref;
    if (__builtin_amdgcn_ballot_w64(nref != ref) != 0) {  // wave-uniform
      const float alpha = nref == ref ? 1.f : fast_exp2(ref - nref);  // 0 from -inf
      l *= alpha;
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] *= alpha;
      ref = nref;
    }
    const float base = ref == -INFINITY ? 0.f : ref;  // no visible key yet: p = 0
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = fast_exp2(fmaf(s[v], sl2, -base));
      l += p[v];
    }
    const bf16x4 pb = {(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
    const i16x4 pt = __builtin_bit_cast(i16x4, pb);
    // V^T blocks: lane a of group g reads row 4g + a / 4, columns 16c + 4 (a % 4) .. + 4
    const int vrow = 4 * g + (n >> 2);
    const int vbyte = 8 * (n & 3);  // byte offset of the 4 columns in the 32-byte pair
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int chunk = 2 * c + (vbyte >> 4);
      const char* pa = vt_lds + vrow * RB + ((chunk ^ swz(vrow)) << 4) + (vbyte & 15);
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(uintptr_t)(uint32_t)(uintptr_t)pa);
      o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pt, o[c], 0, 0, 0);
    }
  };
  // three register buffers in a ring, as in the dot2 kernel (no exit inside a trip, so each
  // buffer keeps its registers; tiles past the range are masked out)
  for (int j0 = k0, slot = 0; j0 < k1; j0 += 48, slot ^= 1) {
    tile_step(j0, t0, slot);
    load_tile(j0 + 48, t0);
    tile_step(j0 + 16, t1, slot ^ 1);
    load_tile(j0 + 64, t1);
    tile_step(j0 + 32, t2, slot);
    load_tile(j0 + 80, t2);
  }
  l += xor_lanes<16>(l);
  l += xor_lanes<32>(l);
  if (n >= nr) return;
  const size_t pbase = ((size_t)bkv * a.nsplit + sp) * R + r0 + n;
  float* po = a.part_o + pbase * HD + 4 * g;
#pragma unroll
  for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4*>(po + 16 * c) = o[c];
  if (g == 0) {
    a.part_ml[pbase * 2] = ref;
    a.part_ml[pbase * 2 + 1] = l;
  }
}

// ---------------------------------------------------------------------------------------
// 3. combine.  One wave per output row (b, query head, i); lane l takes the 8 columns
// 8 (l % (HD/8)) .. of the ranges l / (HD/8), + 64 / (HD/8), ..., eight ranges per pass
// with all their loads in flight together, added in range order under a running maximum;
// the lanes' states are then merged by a fixed xor butterfly (bitwise reproducible).
// ---------------------------------------------------------------------------------------
template <typename T, int HD>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int CC = HD / 8;   // column chunks of 8 per row
  constexpr int SG = 64 / CC;  // range groups per wave: lane l takes ranges l / CC + SG k
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= a.B * a.H * a.Sq) return;
  const int i = w % a.Sq, bh = w / a.Sq, b = bh / a.H, qh = bh - b * a.H;
  const int group = a.H / a.Hkv, kvh = qh / group, g = qh - kvh * group;
  const int R = group * a.Sq, r = g * a.Sq + i;
  const size_t base = (size_t)(b * a.Hkv + kvh) * a.nsplit * R + r;  // + range * R
  const int cc = lane % CC, sg = lane / CC;
  // running state of the lane's ranges: reference M (log2 units), sum L, columns acc
  float M = -INFINITY, L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  constexpr int KB = 8;  // ranges per lane per pass, all loaded before any is used
  for (int s0 = sg; s0 < a.nsplit; s0 += KB * SG) {
    float ms[KB], ls[KB];
    f32x4 o0[KB], o1[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int sp = s0 + k * SG;
      const size_t idx = base + (size_t)(sp < a.nsplit ? sp : sg) * R;
      const float m = a.part_ml[idx * 2];
      ms[k] = sp < a.nsplit ? m : -INFINITY;  // past the last range: weight 0
      ls[k] = a.part_ml[idx * 2 + 1];
      const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o + idx * HD + 8 * cc);
      o0[k] = po[0];
      o1[k] = po[1];
    }
    float cm = M;
#pragma unroll
    for (int k = 0; k < KB; ++k) cm = fmaxf(cm, ms[k]);
    const float alpha = M == -INFINITY ? 0.f : fast_exp2(M - cm);
    L *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int k = 0; k < KB; ++k) {  // range order
      const float f = ms[k] == -INFINITY ? 0.f : fast_exp2(ms[k] - cm);
      L += ls[k] * f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += o0[k][e] * f;
        acc[4 + e] += o1[k][e] * f;
      }
    }
    M = cm;
  }
  // the lanes' states, merged by a fixed xor butterfly over the range groups
#pragma unroll
  for (int m = CC; m < 64; m *= 2) {
    const float mp = shfl_xor(M, m), lp = shfl_xor(L, m);
    const float mn = fmaxf(M, mp);
    const float a1 = M == -INFINITY ? 0.f : fast_exp2(M - mn);
    const float a2 = mp == -INFINITY ? 0.f : fast_exp2(mp - mn);
    L = L * a1 + lp * a2;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a1 + shfl_xor(acc[e], m) * a2;
    M = mn;
  }
  if (sg == 0) {
    T* dst = static_cast<T*>(a.out) + (size_t)w * HD + 8 * cc;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = from_f32<T>(acc[e] / L);
  }
  if (lane == 0) a.lse[w] = (M + log2f(L)) * kLn2;
}

// Query rows per KV head (group * Sq) a split-kernel instantiation holds in registers.
template <typename T>
constexpr int decode_rows_max() { return 64 / V16<T>::n; }

// Rows per wave: the smallest instantiation whose register rows cover the R query rows of a
// KV head, or the largest one, in several row chunks, when none does.
template <typename T, int HD, int RMV>
hipError_t split_launch(int R, DecodeArgs a, hipStream_t stream) {
  if constexpr (std::is_same_v<T, bf16> && (HD == 64 || HD == 128)) {
    a.nchunk = (R + 15) / 16;  // 16 query rows per wave
    const int waves = a.B * a.Hkv * a.nchunk * a.nsplit;
    hipLaunchKernelGGL((decode_split_mfma_kernel<HD>), dim3((waves + 3) / 4), dim3(256), 0,
                       stream, a);
    return hipSuccess;
  } else {
    if constexpr (RMV < decode_rows_max<T>()) {
      if (R > RMV) return split_launch<T, HD, 2 * RMV>(R, a, stream);
    }
    a.nchunk = (R + RMV - 1) / RMV;
    const int waves = a.B * a.Hkv * a.nchunk * a.nsplit;
    if constexpr (std::is_same_v<T, bf16>)
      hipLaunchKernelGGL((decode_split_bf16_kernel<HD, RMV>), dim3((waves + 3) / 4),
                         dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<T, HD, RMV>), dim3((waves + 3) / 4), dim3(256),
                         0, stream, a);
    return hipSuccess;
  }
}

template <typename T, int HD>
hipError_t decode_launch(const DecodeArgs& a, hipStream_t stream) {
  hipError_t e;
  const int R = (a.H / a.Hkv) * a.Sq;
  {
    ProfScope prof("decode_split", stream);
    e = split_launch<T, HD, 1>(R, a, stream);
    if (e != hipSuccess) return e;
  }
  e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  ProfScope prof("decode_combine", stream);
  const int outs = a.B * a.H * a.Sq;
  hipLaunchKernelGGL((decode_combine_kernel<T, HD>), dim3((outs + 3) / 4), dim3(256), 0, stream,
                     a);
  return hipPeekAtLastError();
}

}  // namespace


// Key ranges: at least 64 keys each, and at most 1024 / (B*Hkv) of them, so that the waves
// of a one-chunk launch fit one per SIMD in a single round (measured against eight per CU:
// equal at 134 MB per step, 3.5-4.5 % faster at 0.5-2 GB, and a smaller combine); range
// lengths are whole 16-key tiles.  Both bounds grow with the cache rows, so
// decode_max_splits(capacity) bounds every call with that capacity.
int decode_max_splits(int batch, int num_kv_heads, int cache_rows) {
  const int bkv = batch * num_kv_heads;
  const int cap_splits = bkv >= 1024 ? 1 : 1024 / bkv;
  int n = (cache_rows + 63) / 64;
  if (n > cap_splits) n = cap_splits;
  return n < 1 ? 1 : n;
}

DecodePlan decode_plan(const DecodeShape& d, int cache_rows) {
  DecodePlan p;
  const int n = decode_max_splits(d.batch, d.num_kv_heads, cache_rows);
  p.ks = ((cache_rows + n - 1) / n + 15) / 16 * 16;
  p.nsplit = (cache_rows + p.ks - 1) / p.ks;
  return p;
}

hipError_t launch_decode(IoType io, const DecodeShape& d, const DecodeBufs& bufs,
                         hipStream_t stream) {
  DecodeArgs a;
  a.xq = bufs.xq, a.xk = bufs.xk, a.v = bufs.v;
  a.gamma_q = bufs.gamma_q, a.gamma_k = bufs.gamma_k;
  a.cos_tab = bufs.cos_tab, a.sin_tab = bufs.sin_tab;
  a.k_cache = bufs.k_cache, a.v_cache = bufs.v_cache, a.out = bufs.out, a.lse = bufs.lse;
  a.part_o = bufs.part_o, a.part_ml = bufs.part_ml;
  a.cache_lens = bufs.cache_lens;
  a.nchunk = 1;
  a.B = d.batch, a.H = d.num_heads, a.Hkv = d.num_kv_heads, a.Sq = d.q_len;
  a.pos = d.cache_len, a.cap = d.capacity;
  const DecodePlan p = decode_plan(d, d.cache_len + d.q_len);
  a.nsplit = p.nsplit, a.ks = p.ks;
  a.eps = d.eps;
  a.scale_log2 = kLog2e / sqrtf((float)d.head_dim);
#define XATTN_CASE(T, HD) \
  if (d.head_dim == HD) return decode_launch<T, HD>(a, stream);
  if (io == IO_F32) {
    XATTN_CASE(float, 16) XATTN_CASE(float, 32) XATTN_CASE(float, 64) XATTN_CASE(float, 128)
  } else {
    XATTN_CASE(bf16, 16) XATTN_CASE(bf16, 32) XATTN_CASE(bf16, 64) XATTN_CASE(bf16, 128)
  }
#undef XATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
