// C-ABI layer of libxattn: argument validation, workspace carving, dispatch.
//
// Error discipline: every argument is checked before anything is enqueued, so a
// rejected call has no side effects; launch errors are read with hipPeekAtLastError
// (the sticky error is left for the caller to see); no exception crosses the ABI and
// nothing here exits the process.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "../../include/xattn.h"
#include "xattn_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // exclusive bound on any element count

struct Fail {
  xattn_status status;
};

[[noreturn]] void fail(xattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  throw Fail{st};
}

void check_ptr(const void* p, const char* name) {
  if (p == nullptr) fail(XATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    fail(XATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
}

void check_pos(int64_t v, const char* name) {
  if (v <= 0) fail(XATTN_ERR_INVALID_ARG, "%s must be positive (got %lld)", name, (long long)v);
}

// a * b * c * d with an overflow check against kMaxElems (all factors already > 0)
int64_t count4(int64_t a, int64_t b, int64_t c, int64_t d, const char* what) {
  const long double n = (long double)a * (long double)b * (long double)c * (long double)d;
  if (n >= (long double)kMaxElems)
    fail(XATTN_ERR_INVALID_ARG, "%s: element count %.0Lf does not fit in int32", what, n);
  return a * b * c * d;
}

void check_head_dim(int64_t hd) {
  if (hd <= 0 || hd % 2 != 0)
    fail(XATTN_ERR_INVALID_ARG, "head_dim must be positive and even (got %lld)", (long long)hd);
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    fail(XATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (16, 32, 64, 128)", (long long)hd);
}

xattn::IoType check_dtype(int32_t dt) {
  if (dt != XATTN_F32 && dt != XATTN_BF16)
    fail(XATTN_ERR_INVALID_ARG, "dtype %d is not XATTN_F32 or XATTN_BF16", (int)dt);
  return dt == XATTN_F32 ? xattn::IO_F32 : xattn::IO_BF16;
}

size_t io_size(xattn::IoType io) { return io == xattn::IO_F32 ? 4 : 2; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

// Outputs must not overlap inputs or each other.
void check_no_overlap(std::initializer_list<Range> outs, std::initializer_list<Range> ins) {
  auto overlap = [](const Range& a, const Range& b) {
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
  };
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Range& i : ins)
      if (overlap(*o, i)) fail(XATTN_ERR_INVALID_ARG, "output %s overlaps input %s", o->name, i.name);
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) fail(XATTN_ERR_INVALID_ARG, "outputs %s and %s overlap", o->name, o2->name);
  }
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(XATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

template <typename F>
xattn_status guarded(F&& f) {
  try {
    f();
    g_last_error.clear();
    return XATTN_OK;
  } catch (const Fail& e) {
    return e.status;
  } catch (...) {
    g_last_error = "internal error";
    return XATTN_ERR_INVALID_ARG;
  }
}

struct DimsChecked {
  xattn::AttnShape s;
  xattn::IoType io;
  int64_t q_elems, kv_elems, rows_q;
};

DimsChecked check_dims(const xattn_dims* d) {
  if (d == nullptr) fail(XATTN_ERR_INVALID_ARG, "dims is NULL");
  check_pos(d->batch, "batch");
  check_pos(d->seq_len, "seq_len");
  check_pos(d->num_heads, "num_heads");
  check_pos(d->num_kv_heads, "num_kv_heads");
  check_head_dim(d->head_dim);
  if (d->num_heads % d->num_kv_heads != 0)
    fail(XATTN_ERR_INVALID_ARG, "num_heads (%lld) must be a multiple of num_kv_heads (%lld)",
         (long long)d->num_heads, (long long)d->num_kv_heads);
  DimsChecked c;
  c.io = check_dtype(d->dtype);
  c.q_elems = count4(d->batch, d->num_heads, d->seq_len, d->head_dim, "q");
  c.kv_elems = count4(d->batch, d->num_kv_heads, d->seq_len, d->head_dim, "k/v");
  c.rows_q = d->batch * d->num_heads * d->seq_len;
  c.s = {(int)d->batch, (int)d->seq_len, (int)d->num_heads, (int)d->num_kv_heads,
         (int)d->head_dim};
  if ((d->seg_lo == nullptr) != (d->seg_hi == nullptr))
    fail(XATTN_ERR_INVALID_ARG, "seg_lo and seg_hi must both be set or both be NULL");
  if (d->seg_lo != nullptr) {
    check_ptr(d->seg_lo, "seg_lo");
    check_ptr(d->seg_hi, "seg_hi");
    c.s.seg_lo = d->seg_lo;
    c.s.seg_hi = d->seg_hi;
  }
  return c;
}

// Ranges of the document arrays, for the overlap checks (empty without documents).
Range seg_lo_range(const DimsChecked& c) {
  return {c.s.seg_lo, c.s.seg_lo ? (size_t)c.s.seq_len * 4 : 0, "seg_lo"};
}
Range seg_hi_range(const DimsChecked& c) {
  return {c.s.seg_hi, c.s.seg_hi ? (size_t)c.s.seq_len * 4 : 0, "seg_hi"};
}

// The bf16 fast path applies the prologue backward inside its dq / dk stores.
bool fused_prologue_bwd(const DimsChecked& c) {
  return c.io == xattn::IO_BF16 && xattn::fast_bf16_supported(c.s.head_dim);
}

// So do the generic bf16 kernels (head_dim 16 / 32) where the dk/dv launch does not split
// the group's query heads; nq / nk: their dgamma partial slots.
bool generic_fused_prologue_bwd(const DimsChecked& c, int* nq, int* nk) {
  return xattn::generic_pro_parts(c.io, c.s, nq, nk);
}

size_t bwd_workspace(const DimsChecked& c, bool with_prologue) {
  size_t n = 2 * align256((size_t)c.rows_q * sizeof(float));  // delta, lse * log2(e)
  n += align256(xattn::dkdv_partial_floats(c.io, c.s) * sizeof(float));  // group-split dk/dv
  if (with_prologue && fused_prologue_bwd(c)) {
    const int64_t hq = (int64_t)c.s.batch * c.s.num_heads;
    const int64_t hk = (int64_t)c.s.batch * c.s.num_kv_heads;
    const size_t col = (size_t)c.s.head_dim * sizeof(float);  // dgamma partials per slot
    n += align256((size_t)xattn::fused_pro_parts_q(hq, c.s.seq_len) * col);
    n += align256((size_t)xattn::fused_pro_parts_k(hk, c.s.seq_len) * col);
  } else if (int nq, nk; with_prologue && generic_fused_prologue_bwd(c, &nq, &nk)) {
    const size_t col = (size_t)c.s.head_dim * sizeof(float);
    n += align256((size_t)nq * col) + align256((size_t)nk * col);
  } else if (with_prologue) {
    const int64_t rows_k = (int64_t)c.s.batch * c.s.num_kv_heads * c.s.seq_len;
    n += align256((size_t)c.q_elems * sizeof(float));      // dq w.r.t. the rotated q
    n += align256((size_t)c.kv_elems * sizeof(float));     // dk w.r.t. the rotated k
    n += align256((size_t)xattn::qknorm_rope_bwd_blocks(c.rows_q) * c.s.head_dim * sizeof(float));
    n += align256((size_t)xattn::qknorm_rope_bwd_blocks(rows_k) * c.s.head_dim * sizeof(float));
  }
  return n;
}

// ---- projections ------------------------------------------------------------------------
struct ProjChecked {
  DimsChecked c;
  int M, d, nq, nk;  // token rows, model dim, Q and K/V feature widths
  size_t io;
};

ProjChecked check_proj(const xattn_dims* dims, int64_t model_dim) {
  ProjChecked p;
  p.c = check_dims(dims);
  check_pos(model_dim, "model_dim");
  if (model_dim % 8 != 0) fail(XATTN_ERR_INVALID_ARG, "model_dim must be a multiple of 8");
  const int64_t M = (int64_t)p.c.s.batch * p.c.s.seq_len;
  const int64_t nq = (int64_t)p.c.s.num_heads * p.c.s.head_dim;
  const int64_t nk = (int64_t)p.c.s.num_kv_heads * p.c.s.head_dim;
  count4(M, model_dim, 1, 1, "token rows x model_dim");
  count4(model_dim, nq, 1, 1, "weights");
  count4(M, nq, 1, 1, "merged heads");
  // every GEMM operand buffer stays below 2^31 bytes (the kernels' byte offsets are 32-bit)
  const int64_t es = (int64_t)io_size(p.c.io);
  for (int64_t n : {M * model_dim, model_dim * nq, M * nq})
    if (n * es >= kMaxElems)
      fail(XATTN_ERR_INVALID_ARG, "projection operand of %lld bytes exceeds 2^31 bytes",
           (long long)(n * es));
  p.M = (int)M, p.d = (int)model_dim, p.nq = (int)nq, p.nk = (int)nk;
  p.io = io_size(p.c.io);
  return p;
}

// The projection GEMMs' jobs (gemm.hip).  Operands are row-major; `w` below is the io
// dtype's size.  Token rows: x, y, dx [M, d]; merged heads [M, n].
xattn::GemmMat mat(const void* p, int rows, int ld, size_t w) {
  return {p, ld, (uint32_t)((size_t)rows * ld * w), 0};
}
// The token rows [M, heads*hd] of a head-major tensor [B*heads, S, hd], read in place.
xattn::GemmMat mat_heads(const void* p, int rows, int heads, int hd, size_t w) {
  return {p, heads * hd, (uint32_t)((size_t)rows * heads * hd * w), heads};
}
// The bf16 GEMMs read head-major operands in place when every K step of 64 stays inside
// one head (hd % 64 == 0) and inside one sequence (S % 64 == 0); otherwise the tensors are
// merged into token rows first.
bool heads_in_place(const ProjChecked& p) {
  return p.c.io == xattn::IO_BF16 && p.c.s.head_dim % 64 == 0 && p.c.s.seq_len % 64 == 0;
}
xattn::GemmJob job1(xattn::GemmMat a, xattn::GemmMat b, int k, int m, int n, void* c, int ldc,
                    int c_heads, const float* bias, float* part) {
  xattn::GemmJob j{};
  j.seg[0] = {a, b, k};
  j.nseg = 1;
  j.m = m, j.n = n, j.c = c, j.ldc = ldc, j.c_heads = c_heads, j.bias = bias, j.part = part;
  return j;
}
// dW = x^T g: A = x stored [M, d], B = g stored [M, n] (heads > 0: g head-major with that
// many heads)
xattn::GemmJob dw_job(const ProjChecked& p, const void* x, const void* g, int n, float* dw,
                      float* part, int heads = 0) {
  const xattn::GemmMat gm =
      heads > 0 ? mat_heads(g, p.M, heads, p.c.s.head_dim, p.io) : mat(g, p.M, n, p.io);
  return job1(mat(x, p.M, p.d, p.io), gm, p.M, p.d, n, dw, n, 0, nullptr, part);
}
// dWo = merge(out)^T dy: A = out [M, nq] (merged rows, or head-major when heads > 0),
// B = dy [M, d]
xattn::GemmJob dwo_job(const ProjChecked& p, const void* om, const void* dy, float* dwo,
                       float* part, int heads = 0) {
  const xattn::GemmMat am =
      heads > 0 ? mat_heads(om, p.M, heads, p.c.s.head_dim, p.io) : mat(om, p.M, p.nq, p.io);
  return job1(am, mat(dy, p.M, p.d, p.io), p.M, p.nq, p.d, dwo, p.d, 0, nullptr, part);
}

// Workspace regions of the projection calls (each call uses a prefix of its own plan).
size_t proj_scratch_bytes(const ProjChecked& p) {
  const size_t M = p.M, f32 = 4, parts = (size_t)xattn::colsum_parts(p.M) * 4;
  const auto split = [&](const xattn::GemmJob& j) {
    return align256(xattn::gemm_partial_floats(p.c.io, j) * f32);
  };
  const size_t out_fwd = align256(M * p.nq * p.io);
  const size_t out_bwd = align256(M * p.nq * p.io) + align256(parts * p.d) +
                         split(dwo_job(p, nullptr, nullptr, nullptr, nullptr));
  const size_t qkv_bwd = align256(M * p.nq * p.io) + 2 * align256(M * p.nk * p.io) +
                         align256(parts * p.nq) + 2 * align256(parts * p.nk) +
                         split(dw_job(p, nullptr, nullptr, p.nq, nullptr, nullptr)) +
                         2 * split(dw_job(p, nullptr, nullptr, p.nk, nullptr, nullptr));
  return std::max(std::max(out_fwd, out_bwd), std::max(qkv_bwd, (size_t)256));
}

size_t proj_workspace(const ProjChecked& p) { return proj_scratch_bytes(p); }

// Sequential carving of a workspace into 256-byte aligned regions.
struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* r = reinterpret_cast<T*>(base + off);
    off += align256(bytes);
    return r;
  }
};

void check_ws(void* ws, size_t have, size_t need) {
  check_ptr(ws, "workspace");
  if (have < need) fail(XATTN_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", have, need);
}

struct DecodeChecked {
  xattn::DecodeShape d;
  xattn::IoType io;
  int64_t q_elems, kv_new_elems, cache_elems, rows_q;
};

DecodeChecked check_decode_dims(const xattn_decode_dims* d, float eps) {
  if (d == nullptr) fail(XATTN_ERR_INVALID_ARG, "dims is NULL");
  check_pos(d->batch, "batch");
  check_pos(d->num_heads, "num_heads");
  check_pos(d->num_kv_heads, "num_kv_heads");
  check_head_dim(d->head_dim);
  if (d->num_heads % d->num_kv_heads != 0)
    fail(XATTN_ERR_INVALID_ARG, "num_heads (%d) must be a multiple of num_kv_heads (%d)",
         d->num_heads, d->num_kv_heads);
  check_pos(d->q_len, "q_len");
  if (d->cache_len < 0) fail(XATTN_ERR_INVALID_ARG, "cache_len must be >= 0");
  check_pos(d->capacity, "capacity");
  if ((int64_t)d->cache_len + d->q_len > d->capacity)
    fail(XATTN_ERR_INVALID_ARG, "cache_len + q_len (%lld) exceeds capacity (%d)",
         (long long)d->cache_len + d->q_len, d->capacity);
  DecodeChecked c;
  c.io = check_dtype(d->dtype);
  if (!(eps >= 0.f) || !std::isfinite(eps))
    fail(XATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  c.q_elems = count4(d->batch, d->num_heads, d->q_len, d->head_dim, "xq");
  c.kv_new_elems = count4(d->batch, d->num_kv_heads, d->q_len, d->head_dim, "xk");
  c.cache_elems = count4(d->batch, d->num_kv_heads, d->capacity, d->head_dim, "k_cache");
  c.rows_q = (int64_t)d->batch * d->num_heads * d->q_len;
  c.d = {d->batch, d->num_heads, d->num_kv_heads, d->head_dim, d->q_len, d->cache_len,
         d->capacity, eps};
  return c;
}

// the range partials of the output and of (max, sum), each 256-byte aligned
struct DecodeWorkspace {
  size_t part_o, part_ml, total;
};
DecodeWorkspace decode_workspace(const DecodeChecked& c) {
  const xattn::DecodeShape& d = c.d;
  const size_t ranges = (size_t)d.batch * d.num_kv_heads *
                        xattn::decode_max_splits(d.batch, d.num_kv_heads, d.capacity) *
                        (size_t)(d.num_heads / d.num_kv_heads) * d.q_len;
  DecodeWorkspace w;
  w.part_o = 0;
  w.part_ml = w.part_o + align256(ranges * d.head_dim * sizeof(float));
  w.total = w.part_ml + align256(ranges * 2 * sizeof(float));
  return w;
}

}  // namespace

void xattn::set_last_error(const char* msg) { g_last_error = msg; }

namespace {

xattn_status decode_impl(const xattn_decode_dims* dims, const int32_t* cache_lens,
                         const void* xq, const void* xk, const void* v, const float* gamma_q,
                         const float* gamma_k, const float* cos_tab, const float* sin_tab,
                         float eps, void* k_cache, void* v_cache, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    const DecodeChecked c = check_decode_dims(dims, eps);
    for (auto [p, name] : {std::pair<const void*, const char*>{xq, "xq"}, {xk, "xk"}, {v, "v"},
                           {gamma_q, "gamma_q"}, {gamma_k, "gamma_k"}, {cos_tab, "cos_tab"},
                           {sin_tab, "sin_tab"}, {k_cache, "k_cache"}, {v_cache, "v_cache"},
                           {out, "out"}, {lse, "lse"}, {workspace, "workspace"}})
      check_ptr(p, name);
    if (cache_lens != nullptr) check_ptr(cache_lens, "cache_lens");
    const DecodeWorkspace w = decode_workspace(c);
    if (workspace_bytes < w.total)
      fail(XATTN_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, w.total);
    const size_t es = io_size(c.io);
    const size_t qb = (size_t)c.q_elems * es, nb = (size_t)c.kv_new_elems * es;
    const size_t cb = (size_t)c.cache_elems * es, hdb = (size_t)c.d.head_dim * 4;
    const size_t tb = (size_t)c.d.capacity * (c.d.head_dim / 2) * 4;
    check_no_overlap({{k_cache, cb, "k_cache"}, {v_cache, cb, "v_cache"}, {out, qb, "out"},
                      {lse, (size_t)c.rows_q * 4, "lse"}, {workspace, w.total, "workspace"}},
                     {{xq, qb, "xq"}, {xk, nb, "xk"}, {v, nb, "v"}, {gamma_q, hdb, "gamma_q"},
                      {gamma_k, hdb, "gamma_k"}, {cos_tab, tb, "cos_tab"},
                      {sin_tab, tb, "sin_tab"},
                      {cache_lens, cache_lens ? (size_t)c.d.batch * 4 : 0, "cache_lens"}});
    char* ws = static_cast<char*>(workspace);
    xattn::DecodeBufs b;
    b.xq = xq, b.xk = xk, b.v = v, b.gamma_q = gamma_q, b.gamma_k = gamma_k;
    b.cos_tab = cos_tab, b.sin_tab = sin_tab, b.k_cache = k_cache, b.v_cache = v_cache;
    b.out = out, b.lse = lse;
    b.part_o = reinterpret_cast<float*>(ws + w.part_o);
    b.part_ml = reinterpret_cast<float*>(ws + w.part_ml);
    b.cache_lens = cache_lens;
    hip_check(xattn::launch_decode(c.io, c.d, b, (hipStream_t)stream), "decode launch");
  });
}

}  // namespace

extern "C" {

const char* xattn_version(void) { return "libxattn 0.1.0 (gfx950)"; }

const char* xattn_status_string(int32_t status) {
  // an integer, not the enum type: C callers may pass any value, and loading an
  // out-of-range value as the enum would be undefined
  switch (status) {
    case XATTN_OK: return "XATTN_OK";
    case XATTN_ERR_INVALID_ARG: return "XATTN_ERR_INVALID_ARG: invalid argument";
    case XATTN_ERR_UNSUPPORTED: return "XATTN_ERR_UNSUPPORTED: shape not supported";
    case XATTN_ERR_HIP: return "XATTN_ERR_HIP: HIP runtime error";
  }
  return "unknown xattn_status";
}

const char* xattn_last_error(void) { return g_last_error.c_str(); }

xattn_status xattn_profile_start(void) {
  return guarded([&] { xattn::profile_start(); });
}

xattn_status xattn_profile_stop(xattn_kernel_time* entries, int32_t max_entries,
                                int32_t* n_entries) {
  return guarded([&] {
    if (n_entries == nullptr) fail(XATTN_ERR_INVALID_ARG, "n_entries is NULL");
    if (max_entries < 0 || (max_entries > 0 && entries == nullptr))
      fail(XATTN_ERR_INVALID_ARG, "entries must hold max_entries >= 0 records");
    struct Name {
      char s[48];
    };
    std::vector<Name> names(max_entries > 0 ? max_entries : 1);
    std::vector<long long> launches(names.size());
    std::vector<double> ms(names.size());
    hipError_t err = hipSuccess;
    const int n = xattn::profile_stop(reinterpret_cast<char(*)[48]>(names.data()),
                                      launches.data(), ms.data(), max_entries, &err);
    for (int i = 0; i < n && i < max_entries; ++i) {
      std::memcpy(entries[i].name, names[i].s, 48);
      entries[i].launches = launches[i];
      entries[i].total_ms = ms[i];
    }
    *n_entries = n;
    hip_check(err, "profile event wait");
  });
}

xattn_status xattn_rope_cache(float* cos_tab, float* sin_tab, int64_t seq_len,
                              int64_t head_dim, double theta, void* stream) {
  return guarded([&] {
    check_ptr(cos_tab, "cos_tab");
    check_ptr(sin_tab, "sin_tab");
    check_pos(seq_len, "seq_len");
    check_head_dim(head_dim);
    if (!(theta > 0.0) || !std::isfinite(theta))
      fail(XATTN_ERR_INVALID_ARG, "theta must be positive and finite");
    const int64_t n = count4(seq_len, head_dim / 2, 1, 1, "rope table");
    check_no_overlap({{cos_tab, (size_t)n * 4, "cos_tab"}, {sin_tab, (size_t)n * 4, "sin_tab"}}, {});
    hip_check(xattn::launch_rope_cache(cos_tab, sin_tab, (int)seq_len, (int)head_dim, theta,
                                       (hipStream_t)stream),
              "rope_cache launch");
  });
}

xattn_status xattn_segments(const int32_t* cu_seqlens, int32_t ndocs, int64_t seq_len,
                            int32_t* seg_lo, int32_t* seg_hi, int32_t* positions, void* stream) {
  return guarded([&] {
    check_ptr(cu_seqlens, "cu_seqlens");
    check_ptr(seg_lo, "seg_lo");
    check_ptr(seg_hi, "seg_hi");
    if (positions != nullptr) check_ptr(positions, "positions");
    check_pos(ndocs, "ndocs");
    check_pos(seq_len, "seq_len");
    if (seq_len >= ((int64_t)1 << 31)) fail(XATTN_ERR_INVALID_ARG, "seq_len must stay below 2^31");
    if (ndocs > seq_len) fail(XATTN_ERR_INVALID_ARG, "ndocs (%d) exceeds seq_len", ndocs);
    const size_t rb = (size_t)seq_len * 4;
    check_no_overlap({{seg_lo, rb, "seg_lo"}, {seg_hi, rb, "seg_hi"},
                      {positions, positions ? rb : 0, "positions"}},
                     {{cu_seqlens, (size_t)(ndocs + 1) * 4, "cu_seqlens"}});
    hip_check(xattn::launch_segments(cu_seqlens, ndocs, (int)seq_len, seg_lo, seg_hi, positions,
                                     (hipStream_t)stream),
              "segments launch");
  });
}

xattn_status xattn_rope_cache_at(float* cos_tab, float* sin_tab, const int32_t* positions,
                                 int64_t rows, int64_t head_dim, double theta, void* stream) {
  return guarded([&] {
    check_ptr(cos_tab, "cos_tab");
    check_ptr(sin_tab, "sin_tab");
    check_ptr(positions, "positions");
    check_pos(rows, "rows");
    check_head_dim(head_dim);
    if (!(theta > 0.0) || !std::isfinite(theta))
      fail(XATTN_ERR_INVALID_ARG, "theta must be positive and finite");
    const int64_t n = count4(rows, head_dim / 2, 1, 1, "rope table");
    check_no_overlap({{cos_tab, (size_t)n * 4, "cos_tab"}, {sin_tab, (size_t)n * 4, "sin_tab"}},
                     {{positions, (size_t)rows * 4, "positions"}});
    hip_check(xattn::launch_rope_cache_at(cos_tab, sin_tab, positions, (int)rows, (int)head_dim,
                                          theta, (hipStream_t)stream),
              "rope_cache_at launch");
  });
}

xattn_status xattn_qknorm_rope_fwd(const void* x, const float* gamma, const float* cos_tab,
                                   const float* sin_tab, void* y, float* rstd, int64_t rows,
                                   int64_t seq_len, int64_t head_dim, float eps,
                                   int32_t dtype, void* stream) {
  return guarded([&] {
    check_ptr(x, "x");
    check_ptr(gamma, "gamma");
    check_ptr(cos_tab, "cos_tab");
    check_ptr(sin_tab, "sin_tab");
    check_ptr(y, "y");
    check_ptr(rstd, "rstd");
    check_pos(rows, "rows");
    check_pos(seq_len, "seq_len");
    check_head_dim(head_dim);
    const xattn::IoType io = check_dtype(dtype);
    if (!(eps >= 0.f) || !std::isfinite(eps))
      fail(XATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const int64_t n = count4(rows, seq_len, head_dim, 1, "x");
    const size_t xb = (size_t)n * io_size(io);
    const size_t tb = (size_t)seq_len * (head_dim / 2) * 4;
    check_no_overlap({{y, xb, "y"}, {rstd, (size_t)(rows * seq_len) * 4, "rstd"}},
                     {{x, xb, "x"}, {gamma, (size_t)head_dim * 4, "gamma"},
                      {cos_tab, tb, "cos_tab"}, {sin_tab, tb, "sin_tab"}});
    hip_check(xattn::launch_qknorm_rope_fwd(io, (int)head_dim, x, gamma, cos_tab, sin_tab, y,
                                            rstd, (int)(rows * seq_len), (int)seq_len, eps,
                                            (hipStream_t)stream),
              "qknorm_rope_fwd launch");
  });
}

xattn_status xattn_qknorm_rope_fwd_table(const void* x, const float* gamma,
                                         const int32_t* positions, double theta,
                                         float* cos_tab, float* sin_tab, void* y, float* rstd,
                                         int64_t rows, int64_t seq_len, int64_t head_dim,
                                         float eps, int32_t dtype, void* stream) {
  return guarded([&] {
    check_ptr(x, "x");
    check_ptr(gamma, "gamma");
    if (positions != nullptr) check_ptr(positions, "positions");
    check_ptr(cos_tab, "cos_tab");
    check_ptr(sin_tab, "sin_tab");
    check_ptr(y, "y");
    check_ptr(rstd, "rstd");
    check_pos(rows, "rows");
    check_pos(seq_len, "seq_len");
    check_head_dim(head_dim);
    const xattn::IoType io = check_dtype(dtype);
    if (!(eps >= 0.f) || !std::isfinite(eps))
      fail(XATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!(theta > 0.0) || !std::isfinite(theta))
      fail(XATTN_ERR_INVALID_ARG, "theta must be positive and finite");
    const int64_t n = count4(rows, seq_len, head_dim, 1, "x");
    count4(seq_len, head_dim / 2, 1, 1, "rope table");
    const size_t xb = (size_t)n * io_size(io);
    const size_t tb = (size_t)seq_len * (head_dim / 2) * 4;
    check_no_overlap({{y, xb, "y"}, {rstd, (size_t)(rows * seq_len) * 4, "rstd"},
                      {cos_tab, tb, "cos_tab"}, {sin_tab, tb, "sin_tab"}},
                     {{x, xb, "x"}, {gamma, (size_t)head_dim * 4, "gamma"},
                      {positions, positions ? (size_t)seq_len * 4 : 0, "positions"}});
    hip_check(xattn::launch_qknorm_rope_fwd_table(io, (int)head_dim, x, gamma, positions, theta,
                                                  cos_tab, sin_tab, y, rstd, (int)rows,
                                                  (int)seq_len, eps, (hipStream_t)stream),
              "qknorm_rope_fwd_table launch");
  });
}

size_t xattn_qknorm_rope_bwd_workspace_bytes(int64_t rows, int64_t seq_len, int64_t head_dim) {
  if (rows <= 0 || seq_len <= 0 || head_dim <= 0) return 0;
  return (size_t)xattn::qknorm_rope_bwd_blocks(rows * seq_len) * (size_t)head_dim *
         sizeof(float);
}

xattn_status xattn_qknorm_rope_bwd(const void* dy, const void* x, const float* gamma,
                                   const float* rstd, const float* cos_tab,
                                   const float* sin_tab, void* dx, float* dgamma,
                                   void* workspace, size_t workspace_bytes, int64_t rows,
                                   int64_t seq_len, int64_t head_dim, int32_t dtype,
                                   void* stream) {
  return guarded([&] {
    check_ptr(dy, "dy");
    check_ptr(x, "x");
    check_ptr(gamma, "gamma");
    check_ptr(rstd, "rstd");
    check_ptr(cos_tab, "cos_tab");
    check_ptr(sin_tab, "sin_tab");
    check_ptr(dx, "dx");
    check_ptr(dgamma, "dgamma");
    check_ptr(workspace, "workspace");
    check_pos(rows, "rows");
    check_pos(seq_len, "seq_len");
    check_head_dim(head_dim);
    const xattn::IoType io = check_dtype(dtype);
    const int64_t n = count4(rows, seq_len, head_dim, 1, "x");
    const size_t need = xattn_qknorm_rope_bwd_workspace_bytes(rows, seq_len, head_dim);
    if (workspace_bytes < need)
      fail(XATTN_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    const size_t xb = (size_t)n * io_size(io);
    const size_t tb = (size_t)seq_len * (head_dim / 2) * 4;
    check_no_overlap({{dx, xb, "dx"}, {dgamma, (size_t)head_dim * 4, "dgamma"},
                      {workspace, need, "workspace"}},
                     {{dy, xb, "dy"}, {x, xb, "x"}, {gamma, (size_t)head_dim * 4, "gamma"},
                      {rstd, (size_t)(rows * seq_len) * 4, "rstd"}, {cos_tab, tb, "cos_tab"},
                      {sin_tab, tb, "sin_tab"}});
    hip_check(xattn::launch_qknorm_rope_bwd(io, io, (int)head_dim, dy, x, gamma, rstd, cos_tab,
                                            sin_tab, dx, dgamma, (float*)workspace,
                                            (int)(rows * seq_len), (int)seq_len,
                                            (hipStream_t)stream),
              "qknorm_rope_bwd launch");
  });
}

xattn_status xattn_fwd(const xattn_dims* dims, const void* q, const void* k, const void* v,
                       void* out, float* lse, void* stream) {
  return guarded([&] {
    const DimsChecked c = check_dims(dims);
    check_ptr(q, "q");
    check_ptr(k, "k");
    check_ptr(v, "v");
    check_ptr(out, "out");
    check_ptr(lse, "lse");
    const size_t qb = (size_t)c.q_elems * io_size(c.io), kb = (size_t)c.kv_elems * io_size(c.io);
    check_no_overlap({{out, qb, "out"}, {lse, (size_t)c.rows_q * 4, "lse"}},
                     {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, seg_lo_range(c),
                      seg_hi_range(c)});
    hip_check(xattn::launch_attn_fwd(c.io, c.s, q, k, v, out, lse, nullptr, (hipStream_t)stream),
              "attention forward launch");
  });
}

xattn_status xattn_fwd_qnorm(const xattn_dims* dims, const xattn_fwd_prologue* pro,
                             const void* k, const void* v, void* out, float* lse,
                             void* stream) {
  return guarded([&] {
    const DimsChecked c = check_dims(dims);
    if (pro == nullptr) fail(XATTN_ERR_INVALID_ARG, "pro is NULL");
    for (auto [p, name] : {std::pair<const void*, const char*>{pro->xq, "pro->xq"},
                           {pro->gamma_q, "pro->gamma_q"}, {pro->cos_tab, "pro->cos_tab"},
                           {pro->sin_tab, "pro->sin_tab"}, {pro->yq, "pro->yq"},
                           {pro->rstd_q, "pro->rstd_q"}, {k, "k"}, {v, "v"}, {out, "out"},
                           {lse, "lse"}})
      check_ptr(p, name);
    if (!(pro->eps >= 0.f) || !std::isfinite(pro->eps))
      fail(XATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const size_t qb = (size_t)c.q_elems * io_size(c.io), kb = (size_t)c.kv_elems * io_size(c.io);
    const size_t rb = (size_t)c.rows_q * 4, hdb = (size_t)c.s.head_dim * 4;
    const size_t tb = (size_t)c.s.seq_len * (c.s.head_dim / 2) * 4;
    check_no_overlap({{pro->yq, qb, "pro->yq"}, {pro->rstd_q, rb, "pro->rstd_q"}, {out, qb, "out"},
                      {lse, rb, "lse"}},
                     {{pro->xq, qb, "pro->xq"}, {pro->gamma_q, hdb, "pro->gamma_q"},
                      {pro->cos_tab, tb, "pro->cos_tab"}, {pro->sin_tab, tb, "pro->sin_tab"},
                      {k, kb, "k"}, {v, kb, "v"}, seg_lo_range(c), seg_hi_range(c)});
    xattn::QProFuse pf;  // one pass: the forward normalises and rotates its own Q rows
    pf.xq = pro->xq, pf.gamma_q = pro->gamma_q, pf.cos_tab = pro->cos_tab;
    pf.sin_tab = pro->sin_tab, pf.yq = pro->yq, pf.rstd_q = pro->rstd_q, pf.eps = pro->eps;
    hip_check(xattn::launch_attn_fwd(c.io, c.s, nullptr, k, v, out, lse, &pf,
                                     (hipStream_t)stream),
              "attention forward launch");
  });
}

size_t xattn_proj_workspace_bytes(const xattn_dims* dims, int64_t model_dim) {
  size_t n = 0;
  const xattn_status st = guarded([&] { n = proj_workspace(check_proj(dims, model_dim)); });
  return st == XATTN_OK ? n : 0;
}

xattn_status xattn_qkv_proj_fwd(const xattn_dims* dims, const xattn_proj* pr, const void* x,
                                void* xq, void* xk, void* v, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return guarded([&] {
    if (pr == nullptr) fail(XATTN_ERR_INVALID_ARG, "p is NULL");
    const ProjChecked p = check_proj(dims, pr->model_dim);
    for (auto [q, name] : {std::pair<const void*, const char*>{x, "x"}, {pr->wq, "p->wq"},
                           {pr->wk, "p->wk"}, {pr->wv, "p->wv"}, {xq, "xq"}, {xk, "xk"},
                           {v, "v"}})
      check_ptr(q, name);
    for (auto [q, name] : {std::pair<const void*, const char*>{pr->bq, "p->bq"},
                           {pr->bk, "p->bk"}, {pr->bv, "p->bv"}})
      if (q != nullptr) check_ptr(q, name);
    check_ws(workspace, workspace_bytes, proj_workspace(p));
    const size_t M = p.M;
    check_no_overlap({{xq, M * p.nq * p.io, "xq"}, {xk, M * p.nk * p.io, "xk"},
                      {v, M * p.nk * p.io, "v"}, {workspace, proj_workspace(p), "workspace"}},
                     {{x, M * p.d * p.io, "x"}, {pr->wq, (size_t)p.d * p.nq * p.io, "p->wq"},
                      {pr->wk, (size_t)p.d * p.nk * p.io, "p->wk"},
                      {pr->wv, (size_t)p.d * p.nk * p.io, "p->wv"},
                      {pr->bq, pr->bq ? (size_t)p.nq * 4 : 0, "p->bq"},
                      {pr->bk, pr->bk ? (size_t)p.nk * 4 : 0, "p->bk"},
                      {pr->bv, pr->bv ? (size_t)p.nk * 4 : 0, "p->bv"}});
    // one launch: x Wq, x Wk, x Wv, each split into heads with its bias
    const xattn::GemmMat xm = mat(x, p.M, p.d, p.io);
    const xattn::GemmJob jobs[3] = {
        job1(xm, mat(pr->wq, p.d, p.nq, p.io), p.d, p.M, p.nq, xq, 0, p.c.s.num_heads, pr->bq,
             nullptr),
        job1(xm, mat(pr->wk, p.d, p.nk, p.io), p.d, p.M, p.nk, xk, 0, p.c.s.num_kv_heads,
             pr->bk, nullptr),
        job1(xm, mat(pr->wv, p.d, p.nk, p.io), p.d, p.M, p.nk, v, 0, p.c.s.num_kv_heads,
             pr->bv, nullptr)};
    hip_check(xattn::launch_gemm(p.c.io, xattn::GEMM_NN, xattn::GEMM_OUT_IO_HEADS, jobs, 3,
                                 p.c.s.seq_len, p.c.s.head_dim, (hipStream_t)stream),
              "projection GEMM launch");
  });
}

xattn_status xattn_out_proj_fwd(const xattn_dims* dims, const xattn_proj* pr, const void* out,
                                void* y, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return guarded([&] {
    if (pr == nullptr) fail(XATTN_ERR_INVALID_ARG, "p is NULL");
    const ProjChecked p = check_proj(dims, pr->model_dim);
    check_ptr(out, "out");
    check_ptr(pr->wo, "p->wo");
    check_ptr(y, "y");
    if (pr->bo != nullptr) check_ptr(pr->bo, "p->bo");
    check_ws(workspace, workspace_bytes, proj_workspace(p));
    const size_t M = p.M;
    check_no_overlap({{y, M * p.d * p.io, "y"}, {workspace, proj_workspace(p), "workspace"}},
                     {{out, M * p.nq * p.io, "out"},
                      {pr->wo, (size_t)p.nq * p.d * p.io, "p->wo"},
                      {pr->bo, pr->bo ? (size_t)p.d * 4 : 0, "p->bo"}});
    const hipStream_t st = (hipStream_t)stream;
    Carver w{static_cast<char*>(workspace)};
    void* om = w.take<char>(M * p.nq * p.io);
    const bool direct = heads_in_place(p);
    if (!direct) {
      xattn::MergeJobs mj{{{out, om, p.M, p.nq}}, 1};
      hip_check(xattn::launch_merge_heads(p.c.io, mj, p.c.s.seq_len, p.c.s.head_dim, st),
                "merge_heads launch");
    }
    const xattn::GemmMat am = direct ? mat_heads(out, p.M, p.c.s.num_heads, p.c.s.head_dim, p.io)
                                     : mat(om, p.M, p.nq, p.io);
    const xattn::GemmJob j = job1(am, mat(pr->wo, p.nq, p.d, p.io), p.nq, p.M, p.d, y, p.d, 0,
                                  pr->bo, nullptr);
    hip_check(xattn::launch_gemm(p.c.io, xattn::GEMM_NN, xattn::GEMM_OUT_IO_ROWS, &j, 1,
                                 p.c.s.seq_len, p.c.s.head_dim, st),
              "projection GEMM launch");
  });
}

xattn_status xattn_out_proj_bwd(const xattn_dims* dims, const xattn_proj* pr, const void* out,
                                const void* dy, void* dout, float* dwo, float* dbo,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    if (pr == nullptr) fail(XATTN_ERR_INVALID_ARG, "p is NULL");
    const ProjChecked p = check_proj(dims, pr->model_dim);
    for (auto [q, name] : {std::pair<const void*, const char*>{out, "out"}, {dy, "dy"},
                           {pr->wo, "p->wo"}, {dout, "dout"}, {dwo, "dwo"}})
      check_ptr(q, name);
    if (dbo != nullptr) check_ptr(dbo, "dbo");
    check_ws(workspace, workspace_bytes, proj_workspace(p));
    const size_t M = p.M;
    check_no_overlap({{dout, M * p.nq * p.io, "dout"}, {dwo, (size_t)p.nq * p.d * 4, "dwo"},
                      {dbo, dbo ? (size_t)p.d * 4 : 0, "dbo"},
                      {workspace, proj_workspace(p), "workspace"}},
                     {{out, M * p.nq * p.io, "out"}, {dy, M * p.d * p.io, "dy"},
                      {pr->wo, (size_t)p.nq * p.d * p.io, "p->wo"}});
    const hipStream_t st = (hipStream_t)stream;
    Carver w{static_cast<char*>(workspace)};
    void* om = w.take<char>(M * p.nq * p.io);
    float* part = w.take<float>((size_t)xattn::colsum_parts(p.M) * p.d * 4);
    const bool direct = heads_in_place(p);
    xattn::GemmJob jw = direct ? dwo_job(p, out, dy, dwo, nullptr, p.c.s.num_heads)
                               : dwo_job(p, om, dy, dwo, nullptr);
    jw.part = w.take<float>(xattn::gemm_partial_floats(p.c.io, jw) * 4);
    // dout = split(dy Wo^T): Wo stored [nq, d] is B^T
    const xattn::GemmJob jd = job1(mat(dy, p.M, p.d, p.io), mat(pr->wo, p.nq, p.d, p.io), p.d,
                                   p.M, p.nq, dout, 0, p.c.s.num_heads, nullptr, nullptr);
    hip_check(xattn::launch_gemm(p.c.io, xattn::GEMM_NT, xattn::GEMM_OUT_IO_HEADS, &jd, 1,
                                 p.c.s.seq_len, p.c.s.head_dim, st),
              "projection GEMM launch");
    // dwo = merge(out)^T dy
    if (!direct) {
      xattn::MergeJobs mj{{{out, om, p.M, p.nq}}, 1};
      hip_check(xattn::launch_merge_heads(p.c.io, mj, p.c.s.seq_len, p.c.s.head_dim, st),
                "merge_heads launch");
    }
    hip_check(xattn::launch_gemm(p.c.io, xattn::GEMM_TN, xattn::GEMM_OUT_F32, &jw, 1,
                                 p.c.s.seq_len, p.c.s.head_dim, st),
              "projection GEMM launch");
    if (dbo != nullptr) {
      xattn::ColsumJobs cj{{{dy, part, dbo, p.M, p.d}}, 1};
      hip_check(xattn::launch_colsum(p.c.io, cj, st), "bias gradient launch");
    }
  });
}

xattn_status xattn_qkv_proj_bwd(const xattn_dims* dims, const xattn_proj* pr, const void* x,
                                const void* dxq, const void* dxk, const void* dv, void* dx,
                                float* dwq, float* dwk, float* dwv, float* dbq, float* dbk,
                                float* dbv, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return guarded([&] {
    if (pr == nullptr) fail(XATTN_ERR_INVALID_ARG, "p is NULL");
    const ProjChecked p = check_proj(dims, pr->model_dim);
    for (auto [q, name] : {std::pair<const void*, const char*>{x, "x"}, {dxq, "dxq"},
                           {dxk, "dxk"}, {dv, "dv"}, {pr->wq, "p->wq"}, {pr->wk, "p->wk"},
                           {pr->wv, "p->wv"}, {dx, "dx"}, {dwq, "dwq"}, {dwk, "dwk"},
                           {dwv, "dwv"}})
      check_ptr(q, name);
    for (auto [q, name] : {std::pair<const void*, const char*>{dbq, "dbq"}, {dbk, "dbk"},
                           {dbv, "dbv"}})
      if (q != nullptr) check_ptr(q, name);
    check_ws(workspace, workspace_bytes, proj_workspace(p));
    const size_t M = p.M;
    check_no_overlap(
        {{dx, M * p.d * p.io, "dx"}, {dwq, (size_t)p.d * p.nq * 4, "dwq"},
         {dwk, (size_t)p.d * p.nk * 4, "dwk"}, {dwv, (size_t)p.d * p.nk * 4, "dwv"},
         {dbq, dbq ? (size_t)p.nq * 4 : 0, "dbq"}, {dbk, dbk ? (size_t)p.nk * 4 : 0, "dbk"},
         {dbv, dbv ? (size_t)p.nk * 4 : 0, "dbv"}, {workspace, proj_workspace(p), "workspace"}},
        {{x, M * p.d * p.io, "x"}, {dxq, M * p.nq * p.io, "dxq"}, {dxk, M * p.nk * p.io, "dxk"},
         {dv, M * p.nk * p.io, "dv"}, {pr->wq, (size_t)p.d * p.nq * p.io, "p->wq"},
         {pr->wk, (size_t)p.d * p.nk * p.io, "p->wk"},
         {pr->wv, (size_t)p.d * p.nk * p.io, "p->wv"}});
    const hipStream_t st = (hipStream_t)stream;
    Carver w{static_cast<char*>(workspace)};
    void* gq = w.take<char>(M * p.nq * p.io);
    void* gk = w.take<char>(M * p.nk * p.io);
    void* gv = w.take<char>(M * p.nk * p.io);
    float* pq = w.take<float>((size_t)xattn::colsum_parts(p.M) * p.nq * 4);
    float* pk = w.take<float>((size_t)xattn::colsum_parts(p.M) * p.nk * 4);
    float* pv = w.take<float>((size_t)xattn::colsum_parts(p.M) * p.nk * 4);
    // the gradients as token rows: merged copies, or the head-major tensors read in place
    const bool direct = heads_in_place(p);
    const int hq = direct ? p.c.s.num_heads : 0, hk = direct ? p.c.s.num_kv_heads : 0;
    const void* rq = direct ? dxq : gq;
    const void* rk = direct ? dxk : gk;
    const void* rv = direct ? dv : gv;
    xattn::GemmJob jw[3] = {dw_job(p, x, rq, p.nq, dwq, nullptr, hq),
                            dw_job(p, x, rk, p.nk, dwk, nullptr, hk),
                            dw_job(p, x, rv, p.nk, dwv, nullptr, hk)};
    for (xattn::GemmJob& j : jw) j.part = w.take<float>(xattn::gemm_partial_floats(p.c.io, j) * 4);
    if (!direct) {
      xattn::MergeJobs mj{{{dxq, gq, p.M, p.nq}, {dxk, gk, p.M, p.nk}, {dv, gv, p.M, p.nk}}, 3};
      hip_check(xattn::launch_merge_heads(p.c.io, mj, p.c.s.seq_len, p.c.s.head_dim, st),
                "merge_heads launch");
    }
    const auto rows = [&](const void* t, int n, int heads) {
      return heads > 0 ? mat_heads(t, p.M, heads, p.c.s.head_dim, p.io) : mat(t, p.M, n, p.io);
    };
    // dx = gq Wq^T + gk Wk^T + gv Wv^T: one job, three K segments summed in fp32 (W stored
    // [d, n] is B^T)
    xattn::GemmJob jx{};
    jx.seg[0] = {rows(rq, p.nq, hq), mat(pr->wq, p.d, p.nq, p.io), p.nq};
    jx.seg[1] = {rows(rk, p.nk, hk), mat(pr->wk, p.d, p.nk, p.io), p.nk};
    jx.seg[2] = {rows(rv, p.nk, hk), mat(pr->wv, p.d, p.nk, p.io), p.nk};
    jx.nseg = 3;
    jx.m = p.M, jx.n = p.d, jx.c = dx, jx.ldc = p.d;
    hip_check(xattn::launch_gemm(p.c.io, xattn::GEMM_NT, xattn::GEMM_OUT_IO_ROWS, &jx, 1,
                                 p.c.s.seq_len, p.c.s.head_dim, st),
              "projection GEMM launch");
    // dW = x^T g for the three projections in one launch
    hip_check(xattn::launch_gemm(p.c.io, xattn::GEMM_TN, xattn::GEMM_OUT_F32, jw, 3,
                                 p.c.s.seq_len, p.c.s.head_dim, st),
              "projection GEMM launch");
    xattn::ColsumJobs cj{};
    if (dbq != nullptr) cj.job[cj.n++] = {rq, pq, dbq, p.M, p.nq, hq, p.c.s.seq_len};
    if (dbk != nullptr) cj.job[cj.n++] = {rk, pk, dbk, p.M, p.nk, hk, p.c.s.seq_len};
    if (dbv != nullptr) cj.job[cj.n++] = {rv, pv, dbv, p.M, p.nk, hk, p.c.s.seq_len};
    if (cj.n > 0) hip_check(xattn::launch_colsum(p.c.io, cj, st), "bias gradient launch");
  });
}

size_t xattn_decode_workspace_bytes(const xattn_decode_dims* dims) {
  size_t n = 0;
  const xattn_status st = guarded([&] { n = decode_workspace(check_decode_dims(dims, 0.f)).total; });
  return st == XATTN_OK ? n : 0;
}

xattn_status xattn_decode(const xattn_decode_dims* dims, const void* xq, const void* xk,
                          const void* v, const float* gamma_q, const float* gamma_k,
                          const float* cos_tab, const float* sin_tab, float eps, void* k_cache,
                          void* v_cache, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_impl(dims, nullptr, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, eps, k_cache,
                     v_cache, out, lse, workspace, workspace_bytes, stream);
}

xattn_status xattn_decode_varlen(const xattn_decode_dims* dims, const int32_t* cache_lens,
                                 const void* xq, const void* xk, const void* v,
                                 const float* gamma_q, const float* gamma_k,
                                 const float* cos_tab, const float* sin_tab, float eps,
                                 void* k_cache, void* v_cache, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (cache_lens == nullptr) {
    xattn::set_last_error("cache_lens is NULL");
    return XATTN_ERR_INVALID_ARG;
  }
  return decode_impl(dims, cache_lens, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, eps,
                     k_cache, v_cache, out, lse, workspace, workspace_bytes, stream);
}

size_t xattn_bwd_workspace_bytes(const xattn_dims* dims, int with_prologue) {
  size_t n = 0;
  const xattn_status st = guarded([&] { n = bwd_workspace(check_dims(dims), with_prologue != 0); });
  return st == XATTN_OK ? n : 0;
}

xattn_status xattn_bwd(const xattn_dims* dims, const void* q, const void* k, const void* v,
                       const void* out, const float* lse, const void* dout, void* dq,
                       void* dk, void* dv, const xattn_prologue* pro, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return guarded([&] {
    const DimsChecked c = check_dims(dims);
    for (auto [p, name] : {std::pair<const void*, const char*>{q, "q"}, {k, "k"}, {v, "v"},
                           {out, "out"}, {lse, "lse"}, {dout, "dout"}, {dq, "dq"}, {dk, "dk"},
                           {dv, "dv"}, {workspace, "workspace"}})
      check_ptr(p, name);
    const size_t need = bwd_workspace(c, pro != nullptr);
    if (workspace_bytes < need)
      fail(XATTN_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, need);
    const size_t es = io_size(c.io);
    const size_t qb = (size_t)c.q_elems * es, kb = (size_t)c.kv_elems * es;
    const size_t hdb = (size_t)c.s.head_dim * 4;
    const size_t tb = (size_t)c.s.seq_len * (c.s.head_dim / 2) * 4;
    const int64_t rows_k = (int64_t)c.s.batch * c.s.num_kv_heads * c.s.seq_len;
    if (pro != nullptr) {
      for (auto [p, name] :
           {std::pair<const void*, const char*>{pro->xq, "pro->xq"}, {pro->xk, "pro->xk"},
            {pro->gamma_q, "pro->gamma_q"}, {pro->gamma_k, "pro->gamma_k"},
            {pro->rstd_q, "pro->rstd_q"}, {pro->rstd_k, "pro->rstd_k"},
            {pro->cos_tab, "pro->cos_tab"}, {pro->sin_tab, "pro->sin_tab"},
            {pro->dgamma_q, "pro->dgamma_q"}, {pro->dgamma_k, "pro->dgamma_k"}})
        check_ptr(p, name);
      check_no_overlap(
          {{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {workspace, need, "workspace"},
           {pro->dgamma_q, hdb, "pro->dgamma_q"}, {pro->dgamma_k, hdb, "pro->dgamma_k"}},
          {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {out, qb, "out"},
           {lse, (size_t)c.rows_q * 4, "lse"}, {dout, qb, "dout"}, {pro->xq, qb, "pro->xq"},
           {pro->xk, kb, "pro->xk"}, {pro->gamma_q, hdb, "pro->gamma_q"},
           {pro->gamma_k, hdb, "pro->gamma_k"}, {pro->rstd_q, (size_t)c.rows_q * 4, "pro->rstd_q"},
           {pro->rstd_k, (size_t)rows_k * 4, "pro->rstd_k"}, {pro->cos_tab, tb, "pro->cos_tab"},
           {pro->sin_tab, tb, "pro->sin_tab"}, seg_lo_range(c), seg_hi_range(c)});
    } else {
      check_no_overlap({{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {workspace, need, "workspace"}},
                       {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {out, qb, "out"},
                        {lse, (size_t)c.rows_q * 4, "lse"}, {dout, qb, "dout"},
                        seg_lo_range(c), seg_hi_range(c)});
    }

    char* ws = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(ws);
    ws += align256((size_t)c.rows_q * sizeof(float));
    float* lse2 = reinterpret_cast<float*>(ws);
    ws += align256((size_t)c.rows_q * sizeof(float));
    const size_t npart = xattn::dkdv_partial_floats(c.io, c.s);
    float* dkdv_part = npart > 0 ? reinterpret_cast<float*>(ws) : nullptr;
    ws += align256(npart * sizeof(float));
    const hipStream_t st = (hipStream_t)stream;
    if (pro == nullptr) {
      hip_check(xattn::launch_attn_bwd(c.io, c.s, q, k, v, out, lse, dout, dq, dk, dv, delta,
                                       lse2, false, dkdv_part, nullptr, st),
                "attention backward launch");
      return;
    }
    xattn::ProFuse pf;
    pf.xq = pro->xq, pf.xk = pro->xk, pf.gamma_q = pro->gamma_q, pf.gamma_k = pro->gamma_k;
    pf.rstd_q = pro->rstd_q, pf.rstd_k = pro->rstd_k;
    pf.cos_tab = pro->cos_tab, pf.sin_tab = pro->sin_tab;
    pf.dgamma_q = pro->dgamma_q, pf.dgamma_k = pro->dgamma_k;
    if (fused_prologue_bwd(c)) {
      const int64_t hq = (int64_t)c.s.batch * c.s.num_heads;
      pf.partials_q = reinterpret_cast<float*>(ws);
      ws += align256((size_t)xattn::fused_pro_parts_q(hq, c.s.seq_len) * c.s.head_dim *
                     sizeof(float));
      pf.partials_k = reinterpret_cast<float*>(ws);
      hip_check(xattn::launch_attn_bwd_bf16_fast(c.s, q, k, v, out, lse, dout, dq, dk, dv,
                                                 delta, lse2, &pf, st),
                "attention backward launch");
      return;
    }
    if (int nq, nk; generic_fused_prologue_bwd(c, &nq, &nk)) {
      pf.partials_q = reinterpret_cast<float*>(ws);
      ws += align256((size_t)nq * c.s.head_dim * sizeof(float));
      pf.partials_k = reinterpret_cast<float*>(ws);
      hip_check(xattn::launch_attn_bwd(c.io, c.s, q, k, v, out, lse, dout, dq, dk, dv, delta,
                                       lse2, false, dkdv_part, &pf, st),
                "attention backward launch");
      return;
    }
    float* dyq = reinterpret_cast<float*>(ws);
    ws += align256((size_t)c.q_elems * sizeof(float));
    float* dyk = reinterpret_cast<float*>(ws);
    ws += align256((size_t)c.kv_elems * sizeof(float));
    float* part_q = reinterpret_cast<float*>(ws);
    ws += align256((size_t)xattn::qknorm_rope_bwd_blocks(c.rows_q) * c.s.head_dim * sizeof(float));
    float* part_k = reinterpret_cast<float*>(ws);
    hip_check(xattn::launch_attn_bwd(c.io, c.s, q, k, v, out, lse, dout, dyq, dyk, dv, delta,
                                     lse2, true, dkdv_part, nullptr, st),
              "attention backward launch");
    hip_check(xattn::launch_qknorm_rope_bwd_qk(
                  xattn::IO_F32, c.io, c.s.head_dim, dyq, pro->xq, pro->gamma_q, pro->rstd_q, dq,
                  pro->dgamma_q, part_q, (int)c.rows_q, dyk, pro->xk, pro->gamma_k, pro->rstd_k,
                  dk, pro->dgamma_k, part_k, (int)rows_k, pro->cos_tab, pro->sin_tab,
                  c.s.seq_len, st),
              "prologue backward launch");
  });
}

}  // extern "C"
