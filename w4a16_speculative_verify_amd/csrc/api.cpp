// C ABI of libw4v: host-side validation, launch planning and dispatch.
// Every argument check runs before any HIP call, so invalid requests return
// a status without touching the device (and without needing one).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "w4v.h"
#include "w4v_launch.h"

namespace {

// Launch plans are a function of the shape alone (sized for the 256 compute
// units of an MI355X), so workspace sizes are device-independent and results
// are bit-identical across devices.
constexpr int kPlanCUs = 256;
constexpr int kMaxGridYZ = 65535;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline bool ranges_overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

int gemm_check(const void* x, int64_t ldx, const int32_t* qweight, const void* scales,
               const int32_t* qzeros, const void* y, int64_t ldy, int M, int N, int K,
               int group_size) {
  if (M < 0 || N < 0 || K <= 0 || group_size <= 0) return W4V_ERR_INVALID_ARG;
  if (group_size != w4v::kGroup) return W4V_ERR_UNSUPPORTED;
  if (K % group_size != 0 || N % 8 != 0) return W4V_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return W4V_OK;
  if (!x || !qweight || !scales || !qzeros || !y) return W4V_ERR_INVALID_ARG;
  if (ldx < K || ldy < N) return W4V_ERR_INVALID_ARG;
  if (!aligned(x, 16) || (ldx % 8) != 0 || !aligned(qweight, 16) || !aligned(scales, 16) ||
      !aligned(qzeros, 4) || !aligned(y, 16) || (ldy % 8) != 0)
    return W4V_ERR_ALIGNMENT;
  const size_t xbytes = ((size_t)(M - 1) * (size_t)ldx + (size_t)K) * 2;
  const size_t ybytes = ((size_t)(M - 1) * (size_t)ldy + (size_t)N) * 2;
  if (ranges_overlap(x, xbytes, y, ybytes)) return W4V_ERR_INVALID_ARG;
  return W4V_OK;
}

int lmhead_check(const void* h, int64_t ldh, const int8_t* w, const void* scales,
                 const int32_t* target_ids, int M, int H, int V) {
  if (M < 0 || H <= 0 || V <= 0) return W4V_ERR_INVALID_ARG;
  if (H % 128 != 0) return W4V_ERR_INVALID_ARG;
  if (M == 0) return W4V_OK;
  if (!h || !w || !scales || !target_ids) return W4V_ERR_INVALID_ARG;
  if (ldh < H) return W4V_ERR_INVALID_ARG;
  if (!aligned(h, 16) || (ldh % 8) != 0 || !aligned(w, 16) || !aligned(scales, 2) ||
      !aligned(target_ids, 4))
    return W4V_ERR_ALIGNMENT;
  return W4V_OK;
}

int workspace_check(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return W4V_OK;
  if (!ws || ws_bytes < need) return W4V_ERR_WORKSPACE;
  if (!aligned(ws, w4v::kWorkspaceAlign)) return W4V_ERR_ALIGNMENT;
  return W4V_OK;
}

int run_lmhead(const void* h, int64_t ldh, const int8_t* w, const void* scales,
               int32_t* target_ids, float* max_logits, int M, int H, int V,
               const int32_t* draft_ids, int B, int K, int32_t* accepted_len,
               int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  const w4v::LmheadPlan p = w4v::plan_lmhead(M, H, V, kPlanCUs);
  if (p.mblocks > kMaxGridYZ) return W4V_ERR_UNSUPPORTED;
  int st = workspace_check(p.workspace_bytes(), workspace, workspace_bytes);
  if (st != W4V_OK) return st;
  w4v::LmheadArgs a{};
  a.h = static_cast<const _Float16*>(h);
  a.ldh = ldh;
  a.w = w;
  a.scales = static_cast<const _Float16*>(scales);
  a.target_ids = target_ids;
  a.max_logits = max_logits;
  a.M = M;
  a.H = H;
  a.V = V;
  a.draft_ids = draft_ids;
  a.B = B;
  a.K = K;
  a.accepted_len = accepted_len;
  a.out_tokens = out_tokens;
  hipError_t e = w4v::launch_lmhead_argmax(a, p, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

}  // namespace

extern "C" {

const char* w4v_status_string(int status) {
  switch (status) {
    case W4V_OK: return "ok";
    case W4V_ERR_INVALID_ARG: return "invalid argument (null pointer, size or stride)";
    case W4V_ERR_UNSUPPORTED: return "unsupported request (e.g. group_size other than 128)";
    case W4V_ERR_ALIGNMENT: return "pointer or stride breaks the required alignment";
    case W4V_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case W4V_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int w4v_abi_version(void) { return W4V_ABI_VERSION; }

size_t w4a16_gemm_workspace_size(int M, int N, int K, int group_size) {
  if (M <= 0 || N <= 0 || K <= 0 || group_size != w4v::kGroup || K % group_size != 0 ||
      N % 8 != 0)
    return 0;
  return w4v::plan_w4a16(M, N, K, kPlanCUs).workspace_bytes();
}

int w4a16_gemm(const void* x, int64_t ldx, const int32_t* qweight, const void* scales,
               const int32_t* qzeros, void* y, int64_t ldy, int M, int N, int K, int group_size,
               float alpha, void* workspace, size_t workspace_bytes, void* stream) {
  int st = gemm_check(x, ldx, qweight, scales, qzeros, y, ldy, M, N, K, group_size);
  if (st != W4V_OK || M == 0 || N == 0) return st;
  const w4v::GemmPlan p = w4v::plan_w4a16(M, N, K, kPlanCUs);
  if (p.mblocks > kMaxGridYZ || p.splits > kMaxGridYZ) return W4V_ERR_UNSUPPORTED;
  st = workspace_check(p.workspace_bytes(), workspace, workspace_bytes);
  if (st != W4V_OK) return st;
  w4v::GemmArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.ldx = ldx;
  a.qweight = reinterpret_cast<const uint32_t*>(qweight);
  a.scales = static_cast<const _Float16*>(scales);
  a.qzeros = reinterpret_cast<const uint32_t*>(qzeros);
  a.y = static_cast<_Float16*>(y);
  a.ldy = ldy;
  a.M = M;
  a.N = N;
  a.K = K;
  a.alpha = alpha;
  hipError_t e = w4v::launch_w4a16_skinny(a, p, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

size_t w8a16_lmhead_argmax_workspace_size(int M, int H, int V) {
  if (M <= 0 || H <= 0 || V <= 0 || H % 128 != 0) return 0;
  return w4v::plan_lmhead(M, H, V, kPlanCUs).workspace_bytes();
}

int w8a16_lmhead_argmax(const void* h, int64_t ldh, const int8_t* w, const void* scales,
                        int32_t* target_ids, float* max_logits, int M, int H, int V,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = lmhead_check(h, ldh, w, scales, target_ids, M, H, V);
  if (st != W4V_OK || M == 0) return st;
  if (max_logits && !aligned(max_logits, 4)) return W4V_ERR_ALIGNMENT;
  return run_lmhead(h, ldh, w, scales, target_ids, max_logits, M, H, V, nullptr, 0, 0, nullptr,
                    nullptr, workspace, workspace_bytes, stream);
}

int greedy_verify(const int32_t* target_ids, const int32_t* draft_ids, int B, int K, int V,
                  int32_t* accepted_len, int32_t* out_tokens, void* stream) {
  if (B < 0 || K < 0 || V <= 0) return W4V_ERR_INVALID_ARG;
  if (B == 0) return W4V_OK;
  if (!target_ids || !accepted_len || !out_tokens || (K > 0 && !draft_ids))
    return W4V_ERR_INVALID_ARG;
  if ((long long)B * (K + 1) > INT32_MAX) return W4V_ERR_INVALID_ARG;
  if (!aligned(target_ids, 4) || !aligned(accepted_len, 4) || !aligned(out_tokens, 4) ||
      (draft_ids && !aligned(draft_ids, 4)))
    return W4V_ERR_ALIGNMENT;
  hipError_t e = w4v::launch_greedy_verify(target_ids, draft_ids, B, K, V, accepted_len,
                                           out_tokens, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

int w8a16_lmhead_argmax_verify(const void* h, int64_t ldh, const int8_t* w, const void* scales,
                               int32_t* target_ids, float* max_logits, int H, int V,
                               const int32_t* draft_ids, int B, int K, int32_t* accepted_len,
                               int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (B < 0 || K < 0) return W4V_ERR_INVALID_ARG;
  if ((long long)B * (K + 1) > INT32_MAX) return W4V_ERR_INVALID_ARG;
  const int M = B * (K + 1);
  int st = lmhead_check(h, ldh, w, scales, target_ids, M, H, V);
  if (st != W4V_OK || M == 0) return st;
  if (!accepted_len || !out_tokens || (K > 0 && !draft_ids)) return W4V_ERR_INVALID_ARG;
  if ((max_logits && !aligned(max_logits, 4)) || !aligned(accepted_len, 4) ||
      !aligned(out_tokens, 4) || (draft_ids && !aligned(draft_ids, 4)))
    return W4V_ERR_ALIGNMENT;
  return run_lmhead(h, ldh, w, scales, target_ids, max_logits, M, H, V, draft_ids, B, K,
                    accepted_len, out_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"
