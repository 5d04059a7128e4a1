// C ABI of libw4v: host-side validation, launch planning and dispatch.
// Every argument check runs before any HIP call, so invalid requests return
// a status without touching the device (and without needing one).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <vector>

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
  if (group_size != w4v::kGroup && group_size != 32) return W4V_ERR_UNSUPPORTED;
  if (K % group_size != 0 || N % 8 != 0) return W4V_ERR_INVALID_ARG;
  if (K % w4v::kGroup != 0) return W4V_ERR_UNSUPPORTED;   // the kernels step 128 k at a time
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
  // buffer resources take 32-bit offsets below 2 GiB
  if ((size_t)V * (size_t)H >= (1ull << 31) || (size_t)M * (size_t)ldh * 2 >= (1ull << 31))
    return W4V_ERR_UNSUPPORTED;
  return W4V_OK;
}

int workspace_check(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return W4V_OK;
  if (!ws || ws_bytes < need) return W4V_ERR_WORKSPACE;
  if (!aligned(ws, w4v::kWorkspaceAlign)) return W4V_ERR_ALIGNMENT;
  return W4V_OK;
}

int run_lmhead(const void* h, int64_t ldh, const void* w, const void* scales, int f16,
               int32_t* target_ids, float* max_logits, int M, int H, int V,
               const int32_t* draft_ids, int B, int K, int32_t* accepted_len,
               int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  const w4v::LmheadPlan p = w4v::plan_lmhead(M, H, V, kPlanCUs);
  if (p.vblocks > kMaxGridYZ) return W4V_ERR_UNSUPPORTED;    // grid y
  int st = workspace_check(p.workspace_bytes(), workspace, workspace_bytes);
  if (st != W4V_OK) return st;
  w4v::LmheadArgs a{};
  a.h = static_cast<const _Float16*>(h);
  a.ldh = ldh;
  a.w = w;
  a.scales = static_cast<const _Float16*>(scales);
  a.f16 = f16;
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

// Unit shape of linear (K, N) for a grid of `blocks` blocks: wt 64-column
// tiles per column block and S K-splits, with cb * S <= blocks and every
// unit's activation slice fitting in LDS.  Among the shapes that fit, the one
// with the least estimated time: the slowest block's weight stream (at most
// one compute unit's share of the load bandwidth, and never faster than the
// whole linear at the HBM rate), its activation slice, and for S > 1 the
// round trips of the split hand-off plus the last split's read of the
// partials.  Returns false when no shape fits.
struct ChainShape { int wt, splits; };
bool chain_shape(int K, int N, int blocks, ChainShape* out) {
  constexpr double kCuBytesPerNs = 50.0;      // one CU streaming alone
  constexpr double kHbmBytesPerNs = 7000.0;   // the whole chip
  constexpr double kL2BytesPerNs = 100.0;     // one CU reading activations
  constexpr double kSplitNs = 1500.0;         // partial store, ticket, partial loads
  const int G = K / w4v::kGroup;
  const int T = (N + w4v::kColTile - 1) / w4v::kColTile;
  const double total = (double)K * N / 2;
  double best = 0;
  bool found = false;
  for (int wt = 1; wt <= 4; wt *= 2) {
    const int cb = (T + wt - 1) / wt;
    if (cb > blocks) continue;
    const int s_max = blocks / cb < G ? blocks / cb : G;
    for (int S = 1; S <= s_max; ++S) {
      const int glen = (G + S - 1) / S;
      if (glen > w4v::kChainMaxGroups) continue;
      const double wbytes = (double)glen * wt * w4v::kColTile * w4v::kGroup / 2;
      const double xbytes = (double)glen * 16 * w4v::kGroup * 2;
      double t = wbytes / kCuBytesPerNs;
      if (t < total / kHbmBytesPerNs) t = total / kHbmBytesPerNs;
      t += xbytes / kL2BytesPerNs;
      if (S > 1) t += kSplitNs + (double)S * wt * 16 * w4v::kColTile * 4 / kCuBytesPerNs;
      if (!found || t < best) {
        best = t;
        *out = ChainShape{wt, S};
        found = true;
      }
    }
  }
  return found;
}

// Workspace bytes of linear l's ready flags (one word per 64-column tile),
// split tickets, output (16 rows; none for the last linear) and split
// partials.
size_t chain_flag_bytes(int N) {
  const int T = (N + w4v::kColTile - 1) / w4v::kColTile;
  return w4v::align_up((size_t)T * sizeof(unsigned), 256);
}
size_t chain_out_bytes(int N) {
  const int T = (N + w4v::kColTile - 1) / w4v::kColTile;
  return w4v::align_up(16 * (size_t)T * w4v::kColTile * 2, 256);
}
size_t chain_ticket_bytes(int N, const ChainShape& sh) {
  const int T = (N + w4v::kColTile - 1) / w4v::kColTile;
  const int cb = (T + sh.wt - 1) / sh.wt;
  return sh.splits == 1 ? 0 : (size_t)cb * sh.wt * w4v::kChainSlot;
}
size_t chain_partial_bytes(int N, const ChainShape& sh) {
  const int T = (N + w4v::kColTile - 1) / w4v::kColTile;
  const int cb = (T + sh.wt - 1) / sh.wt;
  if (sh.splits == 1) return 0;
  return w4v::align_up((size_t)sh.splits * 16 * cb * sh.wt * w4v::kColTile * 4, 256);
}

// Checks the descriptors and lays out the workspace for a grid of `blocks`:
// header, descriptor table, ready flags and tickets (zeroed by prepare), then
// the intermediate outputs and split partials.  Host-only.
int chain_layout(const w4v_chain_linear* lins, int n, int M, int blocks, w4v::ChainLayout* lay) {
  if (!lins || n < 1 || n > 65535) return W4V_ERR_INVALID_ARG;
  if (M < 1) return W4V_ERR_INVALID_ARG;
  if (M > w4v::kChainMaxRows) return W4V_ERR_UNSUPPORTED;
  if (blocks < 1) return W4V_ERR_HIP;
  size_t off = sizeof(w4v::ChainHeader);
  lay->lin_offset = off;
  off += w4v::align_up((size_t)n * sizeof(w4v::ChainLinear), 256);
  ChainShape sh{};
  for (int l = 0; l < n; ++l) {
    const w4v_chain_linear& L = lins[l];
    if (L.K <= 0 || L.N <= 0 || L.K % w4v::kGroup != 0 || L.N % 8 != 0) return W4V_ERR_INVALID_ARG;
    if (l > 0 && L.K > lins[l - 1].N) return W4V_ERR_INVALID_ARG;
    if (!L.qweight || !L.scales || !L.qzeros) return W4V_ERR_INVALID_ARG;
    if (!aligned(L.qweight, 16) || !aligned(L.scales, 16) || !aligned(L.qzeros, 4))
      return W4V_ERR_ALIGNMENT;
    // buffer resources take 32-bit offsets below 2 GiB
    if ((size_t)L.K * L.N / 2 >= (1ull << 31)) return W4V_ERR_UNSUPPORTED;
    if (!chain_shape(L.K, L.N, blocks, &sh)) return W4V_ERR_UNSUPPORTED;
  }
  lay->counters_offset = off;
  for (int l = 0; l < n; ++l) {
    chain_shape(lins[l].K, lins[l].N, blocks, &sh);
    off += chain_flag_bytes(lins[l].N) + chain_ticket_bytes(lins[l].N, sh);
  }
  lay->buffers_offset = off;
  for (int l = 0; l < n; ++l) {
    chain_shape(lins[l].K, lins[l].N, blocks, &sh);
    if (l < n - 1) off += chain_out_bytes(lins[l].N);
    off += chain_partial_bytes(lins[l].N, sh);
  }
  lay->bytes = off;
  return W4V_OK;
}

int chain_blocks() {
  static int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached_cus = cus;
    cached_dev = dev;
  }
  return cached_cus;
}

}  // namespace

extern "C" {

const char* w4v_status_string(int status) {
  switch (status) {
    case W4V_OK: return "ok";
    case W4V_ERR_INVALID_ARG: return "invalid argument (null pointer, size or stride)";
    case W4V_ERR_UNSUPPORTED: return "unsupported request (e.g. group_size other than 128 or 32)";
    case W4V_ERR_ALIGNMENT: return "pointer or stride breaks the required alignment";
    case W4V_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case W4V_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int w4v_abi_version(void) { return W4V_ABI_VERSION; }

// Workspace of the library path (M >= kLibMinRows): the counter prefix and
// the split-K partials region are left alone (so one workspace still serves
// calls of every shape), then the transposed fp16 weights, then the library
// GEMM's scratch.
static size_t lib_offset() { return w4v::kTicketRegion + w4v::kPartialRegion; }
static size_t lib_weights_bytes(int N, int K) { return w4v::align_up((size_t)N * K * 2, 256); }
static size_t lib_workspace_bytes(int N, int K) {
  return lib_offset() + lib_weights_bytes(N, K) + w4v::kLibWorkspace;
}

size_t w4a16_gemm_workspace_size(int M, int N, int K, int group_size) {
  if (M <= 0 || N <= 0 || K <= 0 || (group_size != w4v::kGroup && group_size != 32) ||
      K % w4v::kGroup != 0 || N % 8 != 0)
    return 0;
  if (M >= w4v::kLibMinRows) return lib_workspace_bytes(N, K);
  return w4v::plan_w4a16(M, N, K, kPlanCUs).workspace_bytes();
}

int w4a16_gemm(const void* x, int64_t ldx, const int32_t* qweight, const void* scales,
               const int32_t* qzeros, void* y, int64_t ldy, int M, int N, int K, int group_size,
               float alpha, void* workspace, size_t workspace_bytes, void* stream) {
  int st = gemm_check(x, ldx, qweight, scales, qzeros, y, ldy, M, N, K, group_size);
  if (st != W4V_OK || M == 0 || N == 0) return st;
  // 33 rows and more: the library path with a workspace, the LDS-tiled
  // kernel (no workspace needed) when none is given at all
  const bool many = M >= w4v::kTiledMinRows;
  const bool lib = many && M >= w4v::kLibMinRows && !(workspace == nullptr && workspace_bytes == 0);
  const bool tiled = many;
  if (tiled && (M + 127) / 128 > kMaxGridYZ) return W4V_ERR_UNSUPPORTED;
  // buffer resources take 32-bit offsets below 2 GiB
  const bool big = (size_t)K * N / 2 >= (1ull << 31) || (size_t)M * ldx * 2 >= (1ull << 31) ||
                   (size_t)(K / group_size) * N * 2 >= (1ull << 31);
  if (tiled && !lib && big) return W4V_ERR_UNSUPPORTED;
  if (lib) {
    st = workspace_check(lib_workspace_bytes(N, K), workspace, workspace_bytes);
    if (st != W4V_OK) return st;
  }
  w4v::GemmPlan p{};
  if (!tiled) {
    p = w4v::plan_w4a16(M, N, K, kPlanCUs);
    if (big || p.mblocks > kMaxGridYZ || p.splits > kMaxGridYZ ||
        p.partial_bytes > w4v::kPartialRegion)
      return W4V_ERR_UNSUPPORTED;
    st = workspace_check(p.workspace_bytes(), workspace, workspace_bytes);
    if (st != W4V_OK) return st;
  }
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
  a.group_size = group_size;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (lib) {
    // weights to fp16 (our kernel), then the plain GEMM; if the library has
    // no plan for the shape (or the weights exceed the tiled kernel's range
    // anyway), the LDS-tiled kernel computes the same product
    char* base = static_cast<char*>(workspace) + lib_offset();
    _Float16* wt = reinterpret_cast<_Float16*>(base);
    hipError_t e = w4v::launch_dequant_w4_f16t(a.qweight, a.scales, a.qzeros, K, N, group_size,
                                               wt, s);
    if (e != hipSuccess) return W4V_ERR_HIP;
    if (w4v::lib_gemm_f16_tn(a.x, ldx, wt, K, a.y, ldy, M, N, K, alpha,
                             base + lib_weights_bytes(N, K), w4v::kLibWorkspace, s))
      return W4V_OK;
    if (big) return W4V_ERR_HIP;
  }
  hipError_t e = tiled ? w4v::launch_w4a16_tiled(a, s) : w4v::launch_w4a16_skinny(a, p, workspace, s);
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
  return run_lmhead(h, ldh, w, scales, 0, target_ids, max_logits, M, H, V, nullptr, 0, 0, nullptr,
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
  return run_lmhead(h, ldh, w, scales, 0, target_ids, max_logits, M, H, V, draft_ids, B, K,
                    accepted_len, out_tokens, workspace, workspace_bytes, stream);
}

size_t f16_lmhead_argmax_workspace_size(int M, int H, int V) {
  return w8a16_lmhead_argmax_workspace_size(M, H, V);
}

int f16_lmhead_argmax_verify(const void* h, int64_t ldh, const void* w, int32_t* target_ids,
                             float* max_logits, int M, int H, int V, const int32_t* draft_ids,
                             int B, int K, int32_t* accepted_len, int32_t* out_tokens,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || K < 0) return W4V_ERR_INVALID_ARG;
  if (B > 0 && (long long)B * (K + 1) != (long long)M) return W4V_ERR_INVALID_ARG;
  // the fp16 head reads no scales: any non-null, aligned pointer passes the shared check
  int st = lmhead_check(h, ldh, static_cast<const int8_t*>(w), w, target_ids, M, H, V);
  if (st != W4V_OK || M == 0) return st;
  if ((size_t)V * (size_t)H * 2 >= (1ull << 31)) return W4V_ERR_UNSUPPORTED;
  if (B > 0 && (!accepted_len || !out_tokens || (K > 0 && !draft_ids))) return W4V_ERR_INVALID_ARG;
  if ((max_logits && !aligned(max_logits, 4)) ||
      (B > 0 && (!aligned(accepted_len, 4) || !aligned(out_tokens, 4) ||
                 (draft_ids && !aligned(draft_ids, 4)))))
    return W4V_ERR_ALIGNMENT;
  return run_lmhead(h, ldh, w, nullptr, 1, target_ids, max_logits, M, H, V,
                    B > 0 ? draft_ids : nullptr, B, B > 0 ? K : 0, B > 0 ? accepted_len : nullptr,
                    B > 0 ? out_tokens : nullptr, workspace, workspace_bytes, stream);
}

// The library's scratch follows the counter prefix and the partials region,
// as for the W4A16 library path, so that one workspace serves both kinds of
// linear on a stream.
size_t f16_gemm_workspace_size(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return lib_offset() + w4v::kLibWorkspace;
}

int f16_gemm(const void* x, int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy, int M,
             int N, int K, float alpha, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K <= 0) return W4V_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return W4V_OK;
  if (!x || !w || !y) return W4V_ERR_INVALID_ARG;
  if (ldx < K || ldw < K || ldy < N) return W4V_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || ldx % 8 != 0 || ldw % 8 != 0 ||
      ldy % 8 != 0)
    return W4V_ERR_ALIGNMENT;
  const size_t xbytes = ((size_t)(M - 1) * (size_t)ldx + (size_t)K) * 2;
  const size_t ybytes = ((size_t)(M - 1) * (size_t)ldy + (size_t)N) * 2;
  const size_t wbytes = ((size_t)(N - 1) * (size_t)ldw + (size_t)K) * 2;
  if (ranges_overlap(x, xbytes, y, ybytes) || ranges_overlap(w, wbytes, y, ybytes))
    return W4V_ERR_INVALID_ARG;
  int st = workspace_check(f16_gemm_workspace_size(M, N, K), workspace, workspace_bytes);
  if (st != W4V_OK) return st;
  if (!w4v::lib_gemm_f16_tn(static_cast<const _Float16*>(x), ldx, static_cast<const _Float16*>(w),
                            ldw, static_cast<_Float16*>(y), ldy, M, N, K, alpha,
                            static_cast<char*>(workspace) + lib_offset(),
                            workspace_bytes - lib_offset(), static_cast<hipStream_t>(stream)))
    return W4V_ERR_UNSUPPORTED;
  return W4V_OK;
}

int gdn_state_commit(float* state, const float* k, const float* v, const float* alpha,
                     const float* beta, const int32_t* accepted_len, int B, int T, int H, int D,
                     void* stream) {
  if (B < 0 || T < 1 || H < 1 || D < 1) return W4V_ERR_INVALID_ARG;
  if (T > w4v::kGdnMaxT || (D != 64 && D != 128) || B > kMaxGridYZ) return W4V_ERR_UNSUPPORTED;
  if (B == 0) return W4V_OK;
  if (!state || !k || !v || !alpha || !beta || !accepted_len) return W4V_ERR_INVALID_ARG;
  if (!aligned(state, 16) || !aligned(k, 4) || !aligned(v, 4) || !aligned(alpha, 4) ||
      !aligned(beta, 4) || !aligned(accepted_len, 4))
    return W4V_ERR_ALIGNMENT;
  // keys and values are read through buffer resources with 32-bit offsets
  if ((size_t)B * T * H * D * 4 >= (1ull << 31)) return W4V_ERR_UNSUPPORTED;
  const size_t sbytes = (size_t)B * H * D * D * 4, kbytes = (size_t)B * T * H * D * 4;
  if (ranges_overlap(state, sbytes, k, kbytes) || ranges_overlap(state, sbytes, v, kbytes))
    return W4V_ERR_INVALID_ARG;
  hipError_t e = w4v::launch_gdn_commit(state, k, v, alpha, beta, accepted_len, B, T, H, D,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

int ngram_draft(const int32_t* history, int64_t ld, const int32_t* lengths, int B, int n_max,
                int n_min, int K, int32_t* drafts, void* stream) {
  if (B < 0 || ld < 1 || K < 1 || n_min < 1 || n_max < n_min) return W4V_ERR_INVALID_ARG;
  if (n_max > w4v::kNgramMaxN || ld >= (1ll << 31)) return W4V_ERR_UNSUPPORTED;
  if (B == 0) return W4V_OK;
  if (!history || !lengths || !drafts) return W4V_ERR_INVALID_ARG;
  if (!aligned(history, 4) || !aligned(lengths, 4) || !aligned(drafts, 4)) return W4V_ERR_ALIGNMENT;
  if (ranges_overlap(history, (size_t)B * ld * 4, drafts, (size_t)B * K * 4))
    return W4V_ERR_INVALID_ARG;
  hipError_t e = w4v::launch_ngram_draft(history, ld, lengths, B, n_max, n_min, K, drafts,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

int append_accepted(int32_t* history, int64_t ld, int32_t* lengths, int B, int K,
                    const int32_t* out_tokens, const int32_t* accepted_len, void* stream) {
  if (B < 0 || ld < 1 || K < 0) return W4V_ERR_INVALID_ARG;
  if (ld >= (1ll << 31)) return W4V_ERR_UNSUPPORTED;
  if (B == 0) return W4V_OK;
  if (!history || !lengths || !out_tokens || !accepted_len) return W4V_ERR_INVALID_ARG;
  if (!aligned(history, 4) || !aligned(lengths, 4) || !aligned(out_tokens, 4) ||
      !aligned(accepted_len, 4))
    return W4V_ERR_ALIGNMENT;
  hipError_t e = w4v::launch_append_accepted(history, ld, lengths, B, K, out_tokens, accepted_len,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

size_t w4a16_chain_workspace_size(const w4v_chain_linear* linears, int n_linears, int M) {
  w4v::ChainLayout lay{};
  if (chain_layout(linears, n_linears, M, chain_blocks(), &lay) != W4V_OK) return 0;
  return lay.bytes;
}

int w4a16_chain_prepare(const w4v_chain_linear* linears, int n_linears, int M, void* workspace,
                        size_t workspace_bytes) {
  const int blocks = chain_blocks();
  w4v::ChainLayout lay{};
  int st = chain_layout(linears, n_linears, M, blocks, &lay);
  if (st != W4V_OK) return st;
  if (!workspace || workspace_bytes < lay.bytes) return W4V_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return W4V_ERR_ALIGNMENT;
  char* base = static_cast<char*>(workspace);
  std::vector<char> img(lay.counters_offset, 0);
  w4v::ChainHeader* hdr = reinterpret_cast<w4v::ChainHeader*>(img.data());
  hdr->magic = w4v::kChainMagic;
  hdr->n_linears = (unsigned)n_linears;
  hdr->blocks = (unsigned)blocks;
  hdr->M = (unsigned)M;
  hdr->K0 = (unsigned)linears[0].K;
  hdr->N_last = (unsigned)linears[n_linears - 1].N;
  hdr->lin_offset = lay.lin_offset;
  w4v::ChainLinear* tab = reinterpret_cast<w4v::ChainLinear*>(img.data() + lay.lin_offset);
  size_t cnt_off = lay.counters_offset;
  size_t buf_off = lay.buffers_offset;
  for (int l = 0; l < n_linears; ++l) {
    const w4v_chain_linear& L = linears[l];
    w4v::ChainLinear& d = tab[l];
    const int T = (L.N + w4v::kColTile - 1) / w4v::kColTile;
    ChainShape sh{};
    chain_shape(L.K, L.N, blocks, &sh);
    const int cb = (T + sh.wt - 1) / sh.wt;
    d.qweight = reinterpret_cast<const uint32_t*>(L.qweight);
    d.scales = static_cast<const _Float16*>(L.scales);
    d.qzeros = reinterpret_cast<const uint32_t*>(L.qzeros);
    d.K = L.K;
    d.N = L.N;
    d.wt = sh.wt;
    d.cb = cb;
    d.splits = sh.splits;
    d.units = cb * sh.splits;
    d.alpha = L.alpha;
    d.ldo = T * w4v::kColTile;
    d.flags = reinterpret_cast<unsigned*>(base + cnt_off);
    cnt_off += chain_flag_bytes(L.N);
    d.tickets = reinterpret_cast<unsigned*>(base + cnt_off);
    cnt_off += chain_ticket_bytes(L.N, sh);
    d.out = nullptr;
    if (l < n_linears - 1) {
      d.out = reinterpret_cast<_Float16*>(base + buf_off);
      buf_off += chain_out_bytes(L.N);
    }
    d.partials = nullptr;
    if (sh.splits > 1) {
      d.partials = reinterpret_cast<float*>(base + buf_off);
      buf_off += chain_partial_bytes(L.N, sh);
    }
  }
  if (hipMemcpy(workspace, img.data(), img.size(), hipMemcpyHostToDevice) != hipSuccess)
    return W4V_ERR_HIP;
  if (hipMemset(base + lay.counters_offset, 0, lay.buffers_offset - lay.counters_offset) !=
      hipSuccess)
    return W4V_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return W4V_ERR_HIP;
  return W4V_OK;
}

int w4a16_chain(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int K0, int N_last,
                void* workspace, void* stream) {
  if (M < 1 || K0 <= 0 || N_last <= 0) return W4V_ERR_INVALID_ARG;
  if (M > w4v::kChainMaxRows) return W4V_ERR_UNSUPPORTED;
  if (!x || !y || !workspace) return W4V_ERR_INVALID_ARG;
  if (ldx < K0 || ldy < N_last) return W4V_ERR_INVALID_ARG;
  if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(y, 16) || ldy % 8 != 0 || !aligned(workspace, 256))
    return W4V_ERR_ALIGNMENT;
  const size_t xbytes = ((size_t)(M - 1) * (size_t)ldx + (size_t)K0) * 2;
  const size_t ybytes = ((size_t)(M - 1) * (size_t)ldy + (size_t)N_last) * 2;
  if (ranges_overlap(x, xbytes, y, ybytes)) return W4V_ERR_INVALID_ARG;
  const int blocks = chain_blocks();
  if (blocks <= 0) return W4V_ERR_HIP;
  hipError_t e = w4v::launch_w4a16_chain(static_cast<w4v::ChainHeader*>(workspace),
                                         static_cast<const _Float16*>(x), ldx,
                                         static_cast<_Float16*>(y), ldy, M, K0, N_last, blocks,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

}  // extern "C"
