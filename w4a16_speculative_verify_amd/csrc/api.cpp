// C ABI of libw4v: host-side validation, launch planning and dispatch.
// Every argument check runs before any HIP call, so invalid requests return
// a status without touching the device (and without needing one).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
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

// ---------------------------------------------------------------- chain plan
// Linear l's 16-column blocks are dealt to G groups of blocks (G = 8 when the
// block count allows: block b belongs to group b % G, the XCD the hardware
// deals it to), contiguously; inside a group, tiles of nb column blocks x S
// K-splits give one unit per block.  nb and S are chosen per linear by a small
// estimate of the slowest unit's time after its inputs are ready: its weights
// through dequantisation and MFMA (about 55 KB/us per CU), its activation rows
// from L2 (about 150 KB/us), and for S > 1 the split hand-off (about 0.8 us)
// plus the last split's read of the partials.
struct ChainPlan {
  int blocks = 0, G = 1, P = 0, n = 0;
  std::vector<w4v::ChainUnit> units;          // [n][blocks]
  std::vector<int> S, tiles, max_ng, N;
  std::vector<std::vector<int>> tile_c0;      // per linear: first column of each tile (+ end)
  std::vector<size_t> part_floats;            // per linear
  std::vector<uint64_t> stream_bytes;         // per block
  size_t lin_offset = 0, unit_offset = 0, stream_offset = 0, xcc_offset = 0;
  size_t counters_offset = 0, buffers_offset = 0, streams_base = 0, bytes = 0;
  std::vector<size_t> flag_off, sflag_off, out_off, part_off;
  std::vector<uint64_t> stream_off;
};

bool chain_shape(int Gk, int nbx_max, int P, int* nb_out, int* S_out) {
  constexpr double kComputeKBperUs = 55.0, kL2KBperUs = 150.0, kSplitUs = 0.8;
  const int ring_kb = w4v::kChainRingBytes / 1024;
  double best = 0;
  bool found = false;
  for (int nb = 1; nb <= w4v::kChainMaxNb; ++nb) {
    const int T = (nbx_max + nb - 1) / nb;
    for (int S = 1; S <= Gk && T * S <= P; ++S) {
      const int ngmax = (Gk + S - 1) / S;
      if (ngmax > w4v::kChainComputeWaves * w4v::kChainMaxWaveGroups) continue;
      const double unit_bytes = (double)ngmax * w4v::chain_group_bytes(nb);
      if ((1023.0 + unit_bytes) / 1024.0 > ring_kb) continue;
      double t = unit_bytes / 1024.0 / kComputeKBperUs + 4.0 * ngmax / kL2KBperUs;
      if (S > 1) t += kSplitUs + (double)S * nb / kL2KBperUs;
      if (!found || t < best - 1e-9) {
        best = t;
        *nb_out = nb;
        *S_out = S;
        found = true;
      }
    }
  }
  return found;
}

int chain_plan(const w4v_chain_linear* lins, int n, int M, int blocks, ChainPlan* p) {
  if (!lins || n < 1 || n > 65535) return W4V_ERR_INVALID_ARG;
  if (M < 1) return W4V_ERR_INVALID_ARG;
  if (M > w4v::kChainMaxRows) return W4V_ERR_UNSUPPORTED;
  if (blocks < 1) return W4V_ERR_HIP;
  p->blocks = blocks;
  p->G = blocks % w4v::kChainGroups == 0 ? w4v::kChainGroups : 1;
  p->P = blocks / p->G;
  p->n = n;
  p->units.assign((size_t)n * blocks, w4v::ChainUnit{-1, 0, 0, 0, 0, 1, 0, 0, 0, 0u, 0, 0u});
  p->S.assign(n, 1);
  p->tiles.assign(n, 0);
  p->max_ng.assign(n, 0);
  p->N.assign(n, 0);
  p->tile_c0.assign(n, {});
  p->part_floats.assign(n, 0);
  p->stream_bytes.assign(blocks, 0);
  for (int l = 0; l < n; ++l) {
    const w4v_chain_linear& L = lins[l];
    if (L.K <= 0 || L.N <= 0 || L.K % w4v::kGroup != 0 || L.N % 8 != 0) return W4V_ERR_INVALID_ARG;
    if (L.N % 16 != 0) return W4V_ERR_UNSUPPORTED;
    if (l > 0 && L.K > lins[l - 1].N) return W4V_ERR_INVALID_ARG;
    if (!L.qweight || !L.scales || !L.qzeros) return W4V_ERR_INVALID_ARG;
    if (!aligned(L.qweight, 4) || !aligned(L.scales, 2) || !aligned(L.qzeros, 4))
      return W4V_ERR_ALIGNMENT;
    const int Gk = L.K / w4v::kGroup, NB = L.N / 16;
    const int nbx_max = (NB + p->G - 1) / p->G;
    int nb = 0, S = 0;
    if (!chain_shape(Gk, nbx_max, p->P, &nb, &S)) return W4V_ERR_UNSUPPORTED;
    p->S[l] = S;
    p->N[l] = L.N;
    int tile = 0;
    size_t pf = 0;
    for (int x = 0; x < p->G; ++x) {
      const int cb_lo = (int)((long)NB * x / p->G), cb_hi = (int)((long)NB * (x + 1) / p->G);
      const int T = (cb_hi - cb_lo + nb - 1) / nb;
      for (int t = 0; t < T; ++t, ++tile) {
        const int c_lo = cb_lo + t * nb;
        const int nbt = std::min(nb, cb_hi - c_lo);
        p->tile_c0[l].push_back(c_lo * 16);
        for (int sp = 0; sp < S; ++sp) {
          const int b = x + p->G * (t * S + sp);
          w4v::ChainUnit& U = p->units[(size_t)l * blocks + b];
          U.col0 = c_lo * 16;
          U.nb = nbt;
          U.g0 = Gk * sp / S;
          U.ng = Gk * (sp + 1) / S - U.g0;
          U.split = sp;
          U.S = S;
          U.tile = tile;
          U.gbytes = w4v::chain_group_bytes(nbt);
          U.soff = (unsigned)p->stream_bytes[b];
          U.part_off = (int)pf;
          p->stream_bytes[b] += (uint64_t)U.ng * U.gbytes;
          if (p->stream_bytes[b] >= (1ull << 31)) return W4V_ERR_UNSUPPORTED;
          p->max_ng[l] = std::max(p->max_ng[l], U.ng);
        }
        if (S > 1) pf += (size_t)(S - 1) * 16 * nbt * 16;
      }
    }
    p->tile_c0[l].push_back(L.N);
    p->tiles[l] = tile;
    p->part_floats[l] = pf;
  }
  // the input tiles of every unit: tiles of linear l-1 whose columns meet the
  // unit's k-range
  for (int l = 1; l < n; ++l) {
    const std::vector<int>& c0 = p->tile_c0[l - 1];
    const int T = p->tiles[l - 1];
    for (int b = 0; b < blocks; ++b) {
      w4v::ChainUnit& U = p->units[(size_t)l * blocks + b];
      if (U.col0 < 0) continue;
      const int k0 = U.g0 * w4v::kGroup, k1 = (U.g0 + U.ng) * w4v::kGroup;
      int f0 = 0;
      while (f0 < T && c0[f0 + 1] <= k0) ++f0;
      int f1 = f0;
      while (f1 < T && c0[f1] < k1) ++f1;
      U.f0 = f0;
      U.nf = f1 - f0;
      if (U.nf > w4v::kChainMaxFlags) return W4V_ERR_UNSUPPORTED;
    }
  }
  // layout: header, tables, counters (zeroed by prepare), buffers, streams
  size_t off = sizeof(w4v::ChainHeader);
  p->lin_offset = off;
  off += w4v::align_up((size_t)n * sizeof(w4v::ChainLinear), 256);
  p->unit_offset = off;
  off += w4v::align_up((size_t)n * blocks * sizeof(w4v::ChainUnit), 256);
  p->stream_offset = off;
  off += w4v::align_up((size_t)blocks * sizeof(w4v::ChainStream), 256);
  p->counters_offset = off;
  p->xcc_offset = off;
  off += w4v::align_up((size_t)blocks * sizeof(unsigned), 256);
  p->flag_off.assign(n, 0);
  p->sflag_off.assign(n, 0);
  p->out_off.assign(n, 0);
  p->part_off.assign(n, 0);
  for (int l = 0; l < n; ++l) {
    p->flag_off[l] = off;
    off += w4v::align_up((size_t)p->tiles[l] * sizeof(unsigned), 256);
    if (p->S[l] > 1) {
      p->sflag_off[l] = off;
      off += w4v::align_up((size_t)p->tiles[l] * p->S[l] * sizeof(unsigned), 256);
    }
  }
  p->buffers_offset = off;
  for (int l = 0; l < n; ++l) {
    if (l < n - 1) {
      p->out_off[l] = off;
      off += w4v::align_up((size_t)16 * p->N[l] * 2, 256);
    }
    if (p->S[l] > 1) {
      p->part_off[l] = off;
      off += w4v::align_up(p->part_floats[l] * sizeof(float), 256);
    }
  }
  off = w4v::align_up(off, 1024);
  p->streams_base = off;
  p->stream_off.assign(blocks, 0);
  for (int b = 0; b < blocks; ++b) {
    p->stream_off[b] = off;
    off += w4v::align_up(p->stream_bytes[b], 1024);
  }
  p->bytes = off;
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

// ------------------------------------------------------------ static scratch
// Device memory of w4a16_gemm_noalloc: the layout of a w4a16_gemm workspace
// (split-K tickets, the skinny path's partials, the M >= 33 path's partials)
// in a file-scope device array.  Every GPU the library runs on holds its own
// copy from the time the library's code is loaded on it until the process
// ends.  Host code never uses the array's name as an address: each device's
// address comes from hipGetSymbolAddress (scratch_for_current_device).
static __device__ __attribute__((aligned(256))) unsigned char scratch[W4V_STATIC_SCRATCH_BYTES];

__global__ void w4v_zero_words(unsigned* p, unsigned n) {
  for (unsigned i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];     // per device: the array's device address
bool g_scratch_clear[kMaxScratchDevices];    // per device: tickets cleared by an eager call

// The scratch array's address on the current device.  Until a call that is
// not under stream capture has cleared the ticket region (with a fill kernel
// on the caller's stream, ordered before the GEMM), every call clears it, so
// that a graph captured before that carries its own clear.
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4V_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return W4V_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4V_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  if (!g_scratch_clear[dev]) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return W4V_ERR_HIP;
    const unsigned words = (unsigned)(w4v::kTicketRegion / sizeof(unsigned));
    hipLaunchKernelGGL(w4v_zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<unsigned*>(g_scratch_ptr[dev]), words);
    if (hipGetLastError() != hipSuccess) return W4V_ERR_HIP;
    if (cap == hipStreamCaptureStatusNone) g_scratch_clear[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return W4V_OK;
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

// Offset of everything after the split-K counter prefix and the skinny
// kernel's partials region: the fp32 partials of the M >= 33 path and the
// fp16 linear's library scratch start here, so one workspace serves calls of
// every shape ordered on one stream.
static size_t lib_offset() { return w4v::kTicketRegion + w4v::kPartialRegion; }

size_t w4a16_gemm_workspace_size(int M, int N, int K, int group_size) {
  if (M <= 0 || N <= 0 || K <= 0 || (group_size != w4v::kGroup && group_size != 32) ||
      K % w4v::kGroup != 0 || N % 8 != 0)
    return 0;
  if (M >= w4v::kMfmaMinRows) {
    const w4v::MfmaPlan p = w4v::plan_w4a16_mfma(M, N, K, kPlanCUs);
    return p.splits > 1 ? lib_offset() + p.partial_bytes : 0;
  }
  return w4v::plan_w4a16(M, N, K, kPlanCUs).workspace_bytes();
}

// w4a16_gemm; may_probe = false for the entry point that must not allocate
static int gemm_impl(const void* x, int64_t ldx, const int32_t* qweight, const void* scales,
                     const int32_t* qzeros, void* y, int64_t ldy, int M, int N, int K,
                     int group_size, float alpha, void* workspace, size_t workspace_bytes,
                     void* stream, bool may_probe) {
  int st = gemm_check(x, ldx, qweight, scales, qzeros, y, ldy, M, N, K, group_size);
  if (st != W4V_OK || M == 0 || N == 0) return st;
  // buffer resources take 32-bit offsets below 2 GiB
  if ((size_t)K * N / 2 >= (1ull << 31) || (size_t)M * ldx * 2 >= (1ull << 31) ||
      (size_t)(K / group_size) * N * 2 >= (1ull << 31))
    return W4V_ERR_UNSUPPORTED;
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
  if (M >= w4v::kMfmaMinRows) {
    // one path for every call of this shape: the plan depends on the shape
    // alone, and a plan with K-splits requires its workspace
    const w4v::MfmaPlan p = w4v::plan_w4a16_mfma(M, N, K, kPlanCUs);
    if (p.mblocks * p.nblocks > INT32_MAX / 64 || p.splits > kMaxGridYZ) return W4V_ERR_UNSUPPORTED;
    float* partials = nullptr;
    if (p.splits > 1) {
      st = workspace_check(lib_offset() + p.partial_bytes, workspace, workspace_bytes);
      if (st != W4V_OK) return st;
      partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + lib_offset());
    }
    hipError_t e = w4v::launch_w4a16_mfma(a, p, partials, s);
    return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
  }
  const w4v::GemmPlan p = w4v::plan_w4a16(M, N, K, kPlanCUs);
  if (p.mblocks > kMaxGridYZ || p.splits > kMaxGridYZ || p.partial_bytes > w4v::kPartialRegion)
    return W4V_ERR_UNSUPPORTED;
  st = workspace_check(p.workspace_bytes(), workspace, workspace_bytes);
  if (st != W4V_OK) return st;
  hipError_t e = w4v::launch_w4a16_skinny(a, p, workspace, s, may_probe);
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
}

int w4a16_gemm(const void* x, int64_t ldx, const int32_t* qweight, const void* scales,
               const int32_t* qzeros, void* y, int64_t ldy, int M, int N, int K, int group_size,
               float alpha, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(x, ldx, qweight, scales, qzeros, y, ldy, M, N, K, group_size, alpha, workspace,
                   workspace_bytes, stream, true);
}

int w4a16_gemm_noalloc(const void* x, int64_t ldx, const int32_t* qweight, const void* scales,
                       const int32_t* qzeros, void* y, int64_t ldy, int M, int N, int K,
                       int group_size, float alpha, void* stream) {
  int st = gemm_check(x, ldx, qweight, scales, qzeros, y, ldy, M, N, K, group_size);
  if (st != W4V_OK || M == 0 || N == 0) return st;
  const size_t need = w4a16_gemm_workspace_size(M, N, K, group_size);
  if (need > W4V_STATIC_SCRATCH_BYTES) return W4V_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
    if (st != W4V_OK) return st;
  }
  return gemm_impl(x, ldx, qweight, scales, qzeros, y, ldy, M, N, K, group_size, alpha, ws,
                   ws ? (size_t)W4V_STATIC_SCRATCH_BYTES : 0, stream, false);
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

int w4v_read_probe_blocks(void) { return w4v::kReadProbeBlocks; }

int w4v_read_probe(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0) return W4V_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(out, 4)) return W4V_ERR_ALIGNMENT;
  hipError_t e = w4v::launch_read_probe(src, bytes, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4V_OK : W4V_ERR_HIP;
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
  ChainPlan p;
  if (chain_plan(linears, n_linears, M, chain_blocks(), &p) != W4V_OK) return 0;
  return p.bytes;
}

int w4a16_chain_prepare(const w4v_chain_linear* linears, int n_linears, int M, void* workspace,
                        size_t workspace_bytes) {
  const int blocks = chain_blocks();
  ChainPlan p;
  int st = chain_plan(linears, n_linears, M, blocks, &p);
  if (st != W4V_OK) return st;
  if (!workspace || workspace_bytes < p.bytes) return W4V_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return W4V_ERR_ALIGNMENT;
  char* base = static_cast<char*>(workspace);
  std::vector<char> img(p.counters_offset, 0);
  w4v::ChainHeader* hdr = reinterpret_cast<w4v::ChainHeader*>(img.data());
  hdr->magic = w4v::kChainMagic;
  hdr->n_linears = (unsigned)n_linears;
  hdr->blocks = (unsigned)blocks;
  hdr->M = (unsigned)M;
  hdr->K0 = (unsigned)linears[0].K;
  hdr->N_last = (unsigned)linears[n_linears - 1].N;
  hdr->groups = (unsigned)p.G;
  hdr->group_blocks = (unsigned)p.P;
  hdr->lin_offset = p.lin_offset;
  hdr->unit_offset = p.unit_offset;
  hdr->stream_offset = p.stream_offset;
  hdr->xcc_offset = p.xcc_offset;
  w4v::ChainLinear* tab = reinterpret_cast<w4v::ChainLinear*>(img.data() + p.lin_offset);
  for (int l = 0; l < n_linears; ++l) {
    w4v::ChainLinear& d = tab[l];
    d.out = l < n_linears - 1 ? reinterpret_cast<_Float16*>(base + p.out_off[l]) : nullptr;
    d.flags = reinterpret_cast<unsigned*>(base + p.flag_off[l]);
    d.sflags = p.S[l] > 1 ? reinterpret_cast<unsigned*>(base + p.sflag_off[l]) : nullptr;
    d.partials = p.S[l] > 1 ? reinterpret_cast<float*>(base + p.part_off[l]) : nullptr;
    d.K = linears[l].K;
    d.N = linears[l].N;
    d.ld_out = linears[l].N;
    d.alpha = linears[l].alpha;
    d.S = p.S[l];
    d.tiles = p.tiles[l];
  }
  memcpy(img.data() + p.unit_offset, p.units.data(), p.units.size() * sizeof(w4v::ChainUnit));
  w4v::ChainStream* sts = reinterpret_cast<w4v::ChainStream*>(img.data() + p.stream_offset);
  for (int b = 0; b < blocks; ++b) {
    sts[b].offset = p.stream_off[b];
    sts[b].kb = (unsigned)(w4v::align_up(p.stream_bytes[b], 1024) / 1024);
    sts[b].pad = 0;
  }
  if (hipMemcpy(workspace, img.data(), img.size(), hipMemcpyHostToDevice) != hipSuccess)
    return W4V_ERR_HIP;
  if (hipMemset(base + p.counters_offset, 0, p.buffers_offset - p.counters_offset) != hipSuccess)
    return W4V_ERR_HIP;
  // the streams' tails past the last unit are never computed on; zero them
  // anyway so that every byte the loader copies is defined
  if (hipMemset(base + p.streams_base, 0, p.bytes - p.streams_base) != hipSuccess)
    return W4V_ERR_HIP;
  for (int l = 0; l < n_linears; ++l) {
    if (p.max_ng[l] == 0) continue;
    hipError_t e = w4v::launch_w4a16_chain_prepack(
        reinterpret_cast<const w4v::ChainUnit*>(base + p.unit_offset) + (size_t)l * blocks,
        reinterpret_cast<const w4v::ChainStream*>(base + p.stream_offset), blocks, p.max_ng[l],
        reinterpret_cast<const uint32_t*>(linears[l].qweight),
        static_cast<const _Float16*>(linears[l].scales),
        reinterpret_cast<const uint32_t*>(linears[l].qzeros), linears[l].N, base, nullptr);
    if (e != hipSuccess) return W4V_ERR_HIP;
  }
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
  if ((size_t)M * (size_t)ldx * 2 >= (1ull << 31) || (size_t)M * (size_t)ldy * 2 >= (1ull << 31))
    return W4V_ERR_UNSUPPORTED;
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
