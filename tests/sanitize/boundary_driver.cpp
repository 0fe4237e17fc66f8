// Host-side driver for the sanitizer build of the C-ABI layer: calls every entry point of
// include/xattn.h with invalid arguments (and queries with valid ones) and checks the
// documented statuses.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code of xattn_api.cpp and profile.cpp (device code is not instrumented) and run on
// the CPU: no call here reaches a kernel launch.  Exit status 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "xattn.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL: %s (last error: '%s')\n", what, xattn_last_error());
    ++failures;
  }
}

void expect_status(xattn_status got, xattn_status want, const char* what, const char* msg) {
  expect(got == want, what);
  if (msg != nullptr) expect(std::strstr(xattn_last_error(), msg) != nullptr, msg);
}

// 16-byte aligned fake device addresses, never dereferenced (validation fails first)
void* at(uintptr_t mib) { return reinterpret_cast<void*>((uintptr_t)0x10000 + (mib << 20)); }
float* fat(uintptr_t mib) { return static_cast<float*>(at(mib)); }

xattn_dims dims(int64_t B, int64_t S, int64_t H, int64_t Hkv, int64_t hd, int32_t dt) {
  xattn_dims d;
  std::memset(&d, 0, sizeof d);
  d.batch = B, d.seq_len = S, d.num_heads = H, d.num_kv_heads = Hkv, d.head_dim = hd;
  d.dtype = dt;
  return d;
}

}  // namespace

int main() {
  for (int s = 0; s < 4; ++s) expect(xattn_status_string(s) != nullptr, "status");
  expect(std::strstr(xattn_status_string(99), "unknown") != nullptr, "unknown");
  expect(std::strstr(xattn_status_string(-1), "unknown") != nullptr, "unknown negative");
  expect(std::strstr(xattn_version(), "gfx950") != nullptr, "version");

  // attention forward: dims, pointers, overlap
  xattn_dims d = dims(2, 64, 8, 2, 64, XATTN_BF16);
  xattn_dims bad = dims(2, 64, 6, 4, 64, XATTN_BF16);
  expect_status(xattn_fwd(&bad, at(0), at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "H % Hkv", "multiple of num_kv_heads");
  bad = dims(2, 64, 8, 2, 48, XATTN_BF16);
  expect_status(xattn_fwd(&bad, at(0), at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_UNSUPPORTED, "head_dim 48", "not supported");
  bad = dims((int64_t)1 << 20, 4096, 8, 8, 128, XATTN_BF16);
  expect_status(xattn_fwd(&bad, at(0), at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "int32 overflow", "int32");
  expect_status(xattn_fwd(nullptr, at(0), at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "NULL dims", "dims");
  expect_status(xattn_fwd(&d, at(0), at(8), at(16), at(0), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "out aliases q", "overlaps input q");
  expect_status(xattn_fwd(&d, at(0), (char*)at(8) + 2, at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "misaligned k", "aligned");

  // backward: workspace size, prologue members
  const size_t w0 = xattn_bwd_workspace_bytes(&d, 0), w1 = xattn_bwd_workspace_bytes(&d, 1);
  expect(w0 > 0 && w1 > w0, "bwd workspace sizes");
  expect(xattn_bwd_workspace_bytes(&bad, 0) == 0, "bwd workspace of invalid dims");
  expect_status(xattn_bwd(&d, at(0), at(8), at(16), at(24), fat(32), at(40), at(48), at(56),
                          at(64), nullptr, at(72), w0 - 1, nullptr),
                XATTN_ERR_INVALID_ARG, "bwd workspace too small", "workspace too small");
  xattn_prologue pro;
  void** pp = reinterpret_cast<void**>(&pro);
  for (int i = 0; i < 10; ++i) pp[i] = at(80 + 8 * i);
  pro.rstd_k = nullptr;
  expect_status(xattn_bwd(&d, at(0), at(8), at(16), at(24), fat(32), at(40), at(48), at(56),
                          at(64), &pro, at(72), w1, nullptr),
                XATTN_ERR_INVALID_ARG, "bwd NULL prologue member", "rstd_k");
  expect_status(xattn_bwd_noalloc(&bad, at(0), at(8), at(16), at(24), fat(32), at(40), at(48),
                                  at(56), at(64), nullptr, nullptr),
                XATTN_ERR_INVALID_ARG, "noalloc invalid dims", "int32");
  xattn_dims big = dims(4, 16384, 64, 8, 128, XATTN_BF16);
  expect_status(xattn_bwd_noalloc(&big, at(0), at(8), at(16), at(24), fat(32), at(40), at(48),
                                  at(56), at(64), nullptr, nullptr),
                XATTN_ERR_UNSUPPORTED, "noalloc beyond its scratch", "static scratch");

  // prologue
  expect_status(xattn_qknorm_rope_fwd(at(0), fat(1), fat(2), fat(3), at(4), fat(5), 4, 16, 64,
                                      -1.f, XATTN_F32, nullptr),
                XATTN_ERR_INVALID_ARG, "prologue eps", "eps");
  expect_status(xattn_qknorm_rope_fwd(at(0), fat(1), fat(2), fat(3), at(4), fat(5), 4, 16, 64,
                                      NAN, XATTN_F32, nullptr),
                XATTN_ERR_INVALID_ARG, "prologue NaN eps", "eps");
  expect_status(xattn_qknorm_rope_fwd_table(at(0), fat(1), nullptr, 0.0, fat(2), fat(3), at(4),
                                            fat(5), 4, 16, 64, 1e-5f, XATTN_F32, nullptr),
                XATTN_ERR_INVALID_ARG, "table theta", "theta");
  const size_t pw = xattn_qknorm_rope_bwd_workspace_bytes(64, 64, 64);
  expect(pw > 0 && xattn_qknorm_rope_bwd_workspace_bytes(0, 1, 64) == 0, "prologue bwd ws");
  expect_status(xattn_qknorm_rope_bwd(at(0), at(8), fat(16), fat(17), fat(18), fat(19), at(24),
                                      fat(32), at(40), pw - 4, 64, 64, 64, XATTN_F32, nullptr),
                XATTN_ERR_INVALID_ARG, "prologue bwd workspace", "workspace too small");
  expect_status(xattn_rope_cache(fat(0), fat(0) + 4, 16, 64, 1e4, nullptr),
                XATTN_ERR_INVALID_ARG, "rope tables overlap", "overlap");
  expect_status(xattn_rope_cache_at(fat(0), fat(1), nullptr, 16, 64, 1e4, nullptr),
                XATTN_ERR_INVALID_ARG, "rope_cache_at NULL positions", "positions");
  expect_status(xattn_segments(nullptr, 2, 16, (int32_t*)at(1), (int32_t*)at(2), nullptr, nullptr),
                XATTN_ERR_INVALID_ARG, "segments NULL offsets", "cu_seqlens");

  // documents
  xattn_dims dd = d;
  dd.seg_lo = (const int32_t*)at(100);
  expect_status(xattn_fwd(&dd, at(0), at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "seg_lo without seg_hi", "both be set");

  // fused forward prologue
  xattn_fwd_prologue fp;
  std::memset(&fp, 0, sizeof fp);
  expect_status(xattn_fwd_qnorm(&d, &fp, at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "fwd_qnorm NULL members", "NULL");
  expect_status(xattn_fwd_qnorm(&d, nullptr, at(8), at(16), at(24), fat(32), nullptr),
                XATTN_ERR_INVALID_ARG, "fwd_qnorm NULL pro", "pro is NULL");

  // decode
  xattn_decode_dims dec{2, 8, 2, 64, XATTN_BF16, 3, 10, 64};
  expect_status(xattn_decode(&dec, at(0), at(1), at(2), fat(3), fat(4), fat(5), fat(6), 1e-5f,
                             at(7), at(8), at(9), fat(10), at(11), 16, nullptr),
                XATTN_ERR_INVALID_ARG, "decode rows in chunks, small workspace",
                "workspace too small");
  expect_status(xattn_decode_varlen(&dec, nullptr, at(0), at(1), at(2), fat(3), fat(4), fat(5),
                                    fat(6), 1e-5f, at(7), at(8), at(9), fat(10), at(11),
                                    1 << 20, nullptr),
                XATTN_ERR_INVALID_ARG, "decode_varlen NULL lengths", "cache_lens is NULL");
  dec.q_len = 1;
  const size_t dw = xattn_decode_workspace_bytes(&dec);
  expect(dw > 0, "decode workspace");
  expect_status(xattn_decode(&dec, at(0), at(1), at(2), fat(3), fat(4), fat(5), fat(6), 1e-5f,
                             at(7), at(8), at(9), fat(10), at(11), dw - 1, nullptr),
                XATTN_ERR_INVALID_ARG, "decode workspace", "workspace too small");
  dec.cache_len = 64;
  expect(xattn_decode_workspace_bytes(&dec) == 0, "decode past capacity");

  // projections
  const size_t jw = xattn_proj_workspace_bytes(&d, 128);
  expect(jw > 0 && xattn_proj_workspace_bytes(&d, 100) == 0, "projection workspace");
  xattn_proj pj;
  std::memset(&pj, 0, sizeof pj);
  pj.model_dim = 128, pj.wq = at(0), pj.wk = at(1), pj.wv = at(2), pj.wo = at(3);
  expect_status(xattn_qkv_proj_fwd(&d, &pj, at(4), at(8), at(12), at(16), at(32), jw - 1, nullptr),
                XATTN_ERR_INVALID_ARG, "projection workspace too small", "workspace too small");
  expect_status(xattn_qkv_proj_fwd(&d, nullptr, at(4), at(8), at(12), at(16), at(32), jw, nullptr),
                XATTN_ERR_INVALID_ARG, "projection NULL p", "p is NULL");
  expect_status(xattn_out_proj_bwd(&d, &pj, at(4), at(8), at(12), nullptr, nullptr, at(32), jw,
                                   nullptr),
                XATTN_ERR_INVALID_ARG, "projection NULL dwo", "dwo is NULL");
  expect_status(xattn_out_proj_fwd(&d, &pj, at(4), at(4), at(32), jw, nullptr),
                XATTN_ERR_INVALID_ARG, "projection y aliases out", "overlaps input");
  expect_status(xattn_qkv_proj_bwd(&d, &pj, at(4), at(8), at(12), at(16), at(20), fat(24),
                                   fat(28), fat(30), nullptr, nullptr, nullptr, at(32), 16, nullptr),
                XATTN_ERR_INVALID_ARG, "projection bwd workspace", "workspace too small");

  // instrumentation with nothing recorded
  int32_t n = -1;
  expect(xattn_profile_stop(nullptr, 4, &n) == XATTN_ERR_INVALID_ARG, "profile stop args");
  expect(xattn_profile_start() == XATTN_OK, "profile start");
  expect(xattn_profile_stop(nullptr, 0, &n) == XATTN_OK && n == 0, "profile empty session");

  std::printf("%d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
