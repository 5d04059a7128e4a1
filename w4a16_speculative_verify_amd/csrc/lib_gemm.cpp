// Plain fp16 GEMM through hipBLASLt: the half-precision linears of a partly
// quantised target (results page section 5: layers kept in fp16).  No W4A16
// call goes through it.
//
//   y[M x N] (row-major, ldy) = alpha * x[M x K] (row-major, ldx) @ wt[N x K]^T (ldw)
//
// In the library's column-major terms: D^T[N x M] = op_T(wt as K x N, ld ldw) x
// op_N(x as K x M, ld ldx), fp32 accumulation, fp32 alpha, fp16 in and out.
// One handle per device and one matmul plan per shape are created on first
// use and kept for the life of the process.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <mutex>
#include <vector>

#include "w4v_launch.h"

namespace w4v {

namespace {

struct Plan {
  int dev, M, N, K;
  int64_t ldx, ldy, ldw;
  hipblasLtMatmulDesc_t op;
  hipblasLtMatrixLayout_t la, lb, lc;
  hipblasLtMatmulAlgo_t algo;
  size_t ws;
};

std::mutex g_mu;
std::vector<std::pair<int, hipblasLtHandle_t>> g_handles;
std::vector<Plan> g_plans;

hipblasLtHandle_t handle_for(int dev) {
  for (auto& h : g_handles)
    if (h.first == dev) return h.second;
  hipblasLtHandle_t h = nullptr;
  if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  g_handles.emplace_back(dev, h);
  return h;
}

// The plan for a shape, made once (nullptr if the library offers none).
const Plan* plan_for(hipblasLtHandle_t h, int dev, int M, int N, int K, int64_t ldx, int64_t ldy,
                     int64_t ldw, size_t scratch_bytes) {
  for (auto& p : g_plans)
    if (p.dev == dev && p.M == M && p.N == N && p.K == K && p.ldx == ldx && p.ldy == ldy &&
        p.ldw == ldw && p.ws <= scratch_bytes)
      return &p;
  Plan p{};
  p.dev = dev; p.M = M; p.N = N; p.K = K; p.ldx = ldx; p.ldy = ldy; p.ldw = ldw;
  if (hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
    return nullptr;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
  hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
  bool ok = hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16F, (uint64_t)K, (uint64_t)N, ldw) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16F, (uint64_t)K, (uint64_t)M, ldx) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16F, (uint64_t)N, (uint64_t)M, ldy) ==
                HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    const uint64_t cap = scratch_bytes;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                          sizeof(cap));
    // the ranked candidates; the first whose scratch fits (the ranking does
    // not always honour the cap)
    hipblasLtMatmulHeuristicResult_t res[8];
    int n = 0;
    ok = hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.la, p.lb, p.lc, p.lc, pref, 8, res, &n) ==
         HIPBLAS_STATUS_SUCCESS;
    int pick = -1;
    for (int i = 0; ok && i < n && pick < 0; ++i)
      if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= scratch_bytes) pick = i;
    ok = ok && pick >= 0;
    if (ok) {
      p.algo = res[pick].algo;
      p.ws = res[pick].workspaceSize;
    }
  }
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (!ok) {
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
    hipblasLtMatmulDescDestroy(p.op);
    return nullptr;
  }
  g_plans.push_back(p);
  return &g_plans.back();
}

}  // namespace

bool lib_gemm_f16_tn(const _Float16* x, int64_t ldx, const _Float16* wt, int64_t ldw, _Float16* y,
                     int64_t ldy, int M, int N, int K, float alpha, void* scratch,
                     size_t scratch_bytes, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  hipblasLtHandle_t h = handle_for(dev);
  if (!h) return false;
  const Plan* p = plan_for(h, dev, M, N, K, ldx, ldy, ldw, scratch_bytes);
  if (!p) return false;
  const float beta = 0.f;
  return hipblasLtMatmul(h, p->op, &alpha, wt, p->la, x, p->lb, &beta, y, p->lc, y, p->lc,
                         &p->algo, p->ws ? scratch : nullptr, p->ws, stream) ==
         HIPBLAS_STATUS_SUCCESS;
}

}  // namespace w4v
