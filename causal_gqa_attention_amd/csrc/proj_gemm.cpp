// Row-major GEMM for the projections around attention ("Phase T12: bf16 mixed precision",
// precision table: linear GEMMs take bf16 in / out with fp32 accumulation), on hipBLASLt:
// the projections are plain dense GEMMs, which the vendor library covers; what is
// specific to attention (the head split / merge layouts, bias, rounding, bias gradients)
// is in proj.hip.
//
// hipBLASLt is column-major.  A row-major [R, C] matrix with leading dimension ld is the
// column-major [C, R] matrix with the same ld, so row-major C = op(A) op(B) is
// column-major C^T = op(B)^T op(A)^T: the library's first operand is B, its second A,
// and the output is [N, M] with leading dimension ldc.
#include <hipblaslt/hipblaslt.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "xattn_internal.h"

namespace xattn {
namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool ok = false;
};

using Key = std::tuple<int, bool, bool, int, int, int, int, int, int, bool>;

std::mutex g_mu;
hipblasLtHandle_t g_handle = nullptr;
std::map<Key, Plan> g_plans;

bool make_plan(Plan& p, IoType io, bool ta, bool tb, int M, int N, int K, int lda, int ldb,
               int ldc, bool accumulate, char (*err)[160]) {
  const hipDataType in = io == IO_F32 ? HIP_R_32F : HIP_R_16BF;
  const hipblasOperation_t opa = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;  // library A = our B
  const hipblasOperation_t opb = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;  // library B = our A
  bool good = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa,
                                              sizeof(opa)) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb,
                                              sizeof(opb)) == HIPBLAS_STATUS_SUCCESS;
  // stored shapes in column-major terms
  good = good &&
         hipblasLtMatrixLayoutCreate(&p.la, in, tb ? K : N, tb ? N : K, ldb) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.lb, in, ta ? M : K, ta ? K : M, lda) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_32F, N, M, ldc) == HIPBLAS_STATUS_SUCCESS;
  if (!good) {
    std::snprintf(*err, sizeof(*err), "hipBLASLt descriptor setup failed");
    return false;
  }
  hipblasLtMatmulPreference_t pref = nullptr;
  hipblasLtMatmulPreferenceCreate(&pref);
  const uint64_t wsmax = kGemmWorkspace;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                        &wsmax, sizeof(wsmax));
  hipblasLtMatmulHeuristicResult_t res[1];
  int found = 0;
  const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(
      g_handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &found);
  hipblasLtMatmulPreferenceDestroy(pref);
  (void)accumulate;
  if (st != HIPBLAS_STATUS_SUCCESS || found < 1) {
    std::snprintf(*err, sizeof(*err),
                  "hipBLASLt has no algorithm for GEMM %dx%dx%d (ta=%d tb=%d, status %d)", M,
                  N, K, (int)ta, (int)tb, (int)st);
    return false;
  }
  p.algo = res[0].algo;
  p.ok = true;
  return true;
}

}  // namespace

bool gemm_rm(IoType io, bool ta, bool tb, int M, int N, int K, const void* A, int lda,
             const void* B, int ldb, float beta, float* C, int ldc, void* ws, size_t ws_bytes,
             hipStream_t stream, char (*err)[160]) {
  Plan* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_handle == nullptr && hipblasLtCreate(&g_handle) != HIPBLAS_STATUS_SUCCESS) {
      g_handle = nullptr;
      std::snprintf(*err, sizeof(*err), "hipblasLtCreate failed");
      return false;
    }
    const Key key{(int)io, ta, tb, M, N, K, lda, ldb, ldc, beta != 0.f};
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
      Plan fresh;
      if (!make_plan(fresh, io, ta, tb, M, N, K, lda, ldb, ldc, beta != 0.f, err)) return false;
      it = g_plans.emplace(key, fresh).first;
    }
    p = &it->second;
  }
  const float alpha = 1.f;
  ProfScope prof("proj_gemm", stream);
  const hipblasStatus_t st =
      hipblasLtMatmul(g_handle, p->desc, &alpha, B, p->la, A, p->lb, &beta, C, p->lc, C, p->lc,
                      &p->algo, ws, ws_bytes, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) {
    std::snprintf(*err, sizeof(*err), "hipblasLtMatmul failed (status %d)", (int)st);
    return false;
  }
  return true;
}

}  // namespace xattn
