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
// rows per KV head, so it is bound by HBM bandwidth, not by arithmetic: a KV head's cache
// is split into key ranges, one wave per (KV head, range); a wave streams its range with
// 16-byte loads (a key row spread over HD*size/16 lanes, several keys per wave load, four
// loads in flight per lane), keeps every query row of the group in registers, and runs an
// online softmax per lane group with one rescale per four keys.  The lane groups of a wave
// are merged by a fixed xor butterfly, the ranges in range order by a second launch, so the
// result is bitwise reproducible.  The prologue forward runs inside the split launch: each
// wave normalises and rotates its group's query rows in the lane layout of its loads, and
// the wave whose range holds a new token's row writes that token's rotated key and its
// value into the caches before streaming the range (its own loads then read them back).
// Two launches: split attention (with prologue and append), combine.
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
  int B, H, Hkv, Sq, pos, cap, nsplit, ks;  // ks: keys per range
  float eps, scale_log2;
};

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
// 2. split attention.  Wave w = (KV row bkv, range sp) handles cache rows [sp*ks,
// min(Lk, sp*ks + ks)), Lk = pos + Sq.  Query row r = g*Sq + i (g < group, i < Sq) is query
// head kvh*group + g at position pos + i and sees cache rows j <= pos + i.  Lane l owns the
// VEC columns part = l % LPK of the key rows j0 + l / LPK (KPW keys per wave load); each lane
// group keeps its own (max, sum, accumulator) per query row, merged at the end.
// ---------------------------------------------------------------------------------------
constexpr int kDecodeUnroll = 4;  // wave loads of K and of V in flight per lane

template <typename T, int HD, int RM>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int VEC = V16<T>::n, LPK = HD / VEC, KPW = 64 / LPK, UN = kDecodeUnroll;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.B * a.Hkv * a.nsplit) return;  // whole waves; the kernel has no barrier
  const int bkv = w / a.nsplit, sp = w - bkv * a.nsplit;
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv, group = a.H / a.Hkv;
  const int R = group * a.Sq, Lk = a.pos + a.Sq;
  const int k0 = sp * a.ks, k1 = min(Lk, k0 + a.ks);
  const int part = lane % LPK, kg = lane / LPK;
  // a wave whose range holds no new token issues its first loads now, under the prologue
  const int n0 = max(k0, a.pos);
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
    if (r < R) {  // wave-uniform
      const int g = r / a.Sq, i = r - g * a.Sq;
      const T* xr = static_cast<const T*>(a.xq) +
                    ((size_t)(b * a.H + kvh * group + g) * a.Sq + i) * HD;
      prologue_lanes<T, HD>(xr, a.gamma_q, a.cos_tab, a.sin_tab, a.pos + i, a.eps, part, q[r]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[r][e] *= a.scale_log2;
      lim[r] = a.pos + i;
    }
  }
  // Append: the new tokens' rows of this range (cache rows pos .. pos + Sq - 1 that fall in
  // [k0, k1)) get the rotated key and the value, KPW rows per pass; then the stores are
  // made visible to this wave's own loads below.
  if (appends) {
    for (int j0 = n0; j0 < k1; j0 += KPW) {
      const int j = j0 + kg;
      const int i = (j < k1 ? j : n0) - a.pos;  // token (clamped for idle lanes)
      const size_t src = ((size_t)bkv * a.Sq + i) * HD;
      float yk[VEC];
      prologue_lanes<T, HD>(static_cast<const T*>(a.xk) + src, a.gamma_k, a.cos_tab,
                            a.sin_tab, a.pos + i, a.eps, part, yk);
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
      if (r < R) {  // wave-uniform
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
        if (r >= R) continue;  // wave-uniform
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
  const size_t base = ((size_t)bkv * a.nsplit + sp) * R;
  {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= R) continue;  // wave-uniform
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
// 3. combine.  One wave per output row (b, query head, i): the common maximum over the
// ranges (lane s reading ranges s, s + 64, ...; an exact max, so any order), then the
// ranges' sums and partial accumulators added in range order.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lanes<32>(v));
  v = fmaxf(v, xor_lanes<16>(v));
  v = fmaxf(v, xor_lanes<8>(v));
  v = fmaxf(v, xor_lanes<4>(v));
  v = fmaxf(v, xor_lanes<2>(v));
  v = fmaxf(v, xor_lanes<1>(v));
  return v;
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int PER = (HD + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.B * a.H * a.Sq) return;
  const int i = w % a.Sq, bh = w / a.Sq, b = bh / a.H, qh = bh - b * a.H;
  const int group = a.H / a.Hkv, kvh = qh / group, g = qh - kvh * group;
  const int R = group * a.Sq, r = g * a.Sq + i;
  const size_t base = (size_t)(b * a.Hkv + kvh) * a.nsplit * R + r;  // + range * R
  float M = -INFINITY;
  for (int c = 0; c < a.nsplit; c += 64)
    if (c + lane < a.nsplit) M = fmaxf(M, a.part_ml[(base + (size_t)(c + lane) * R) * 2]);
  M = wave_max(M);
  float L = 0.f, acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const size_t idx = base + (size_t)sp * R;
    const float ms = a.part_ml[idx * 2];
    const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
    L += a.part_ml[idx * 2 + 1] * f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      if (d < HD) acc[k] += a.part_o[idx * HD + d] * f;
    }
  }
  T* dst = static_cast<T*>(a.out) + (size_t)w * HD;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    if (d < HD) dst[d] = from_f32<T>(acc[k] / L);
  }
  if (lane == 0) a.lse[w] = (M + log2f(L)) * kLn2;
}

// Query rows per KV head (group * Sq) a split-kernel instantiation holds in registers.
template <typename T>
constexpr int decode_rows_max() { return 64 / V16<T>::n; }

// The smallest instantiation whose register rows cover the R query rows.
template <typename T, int HD, int RMV>
hipError_t split_launch(int R, dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  if constexpr (RMV > decode_rows_max<T>()) {
    return hipErrorInvalidValue;
  } else {
    if (R > RMV) return split_launch<T, HD, 2 * RMV>(R, grid, a, stream);
    hipLaunchKernelGGL((decode_split_kernel<T, HD, RMV>), grid, dim3(256), 0, stream, a);
    return hipSuccess;
  }
}

template <typename T, int HD>
hipError_t decode_launch(const DecodeArgs& a, hipStream_t stream) {
  hipError_t e;
  const int R = (a.H / a.Hkv) * a.Sq;
  const int waves = a.B * a.Hkv * a.nsplit;
  {
    ProfScope prof("decode_split", stream);
    e = split_launch<T, HD, 1>(R, dim3((waves + 3) / 4), a, stream);
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

int decode_rows_limit(IoType io) {
  return io == IO_F32 ? decode_rows_max<float>() : decode_rows_max<bf16>();
}

// Key ranges: at least 64 keys each, and no more than needed for about 2048 waves (eight
// per CU).  Both bounds grow with the cache rows, so decode_max_splits(capacity) bounds
// every call with that capacity.
int decode_max_splits(int batch, int num_kv_heads, int cache_rows) {
  const int bkv = batch * num_kv_heads;
  const int cap_splits = bkv >= 2048 ? 1 : (2048 + bkv - 1) / bkv;
  int n = (cache_rows + 63) / 64;
  if (n > cap_splits) n = cap_splits;
  return n < 1 ? 1 : n;
}

DecodePlan decode_plan(const DecodeShape& d, int cache_rows) {
  DecodePlan p;
  const int n = decode_max_splits(d.batch, d.num_kv_heads, cache_rows);
  p.ks = (cache_rows + n - 1) / n;
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
