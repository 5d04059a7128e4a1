// Prompt-lookup (n-gram) drafting and appending the verify's accepted tokens,
// gfx950.  Section 3 of the organisers' results page (Table 3 and the
// paragraph on n-gram drafting): the drafter needs no model and copies spans
// from the prompt; its K is fixed (K = 23 for the team that used it).
//
// ngram_draft: one block per sequence.  A candidate end position e (e <= L-2,
// so at least one token follows) scores the length of the common suffix of
// history[0..e] and history[0..L-1], capped at n_max; the block keeps the
// lexicographic maximum of (score, e) over scores >= n_min: the longest n
// that has an earlier occurrence, then its most recent occurrence.  The
// drafts are the up-to-K tokens after e, padded with -1.
// The history is staged through LDS in tiles of kTile candidates, newest
// first, each with the kHalo tokens before it that a match can reach back
// into: one coalesced pass over HBM per tile, then every comparison from LDS.
// Once a tile holds a match of the longest possible n, older tiles cannot win
// (their candidates are older at best the same score) and the scan stops.
// append_accepted: one thread per sequence appends out_tokens[b][0..a_b].
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kDraftThreads = 512;
constexpr int kTile = 8192;                 // candidates per LDS tile
constexpr int kHalo = kNgramMaxN;           // look-back tokens staged before a tile
constexpr int kStageRounds = (kTile + kHalo + kDraftThreads - 1) / kDraftThreads;

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)(v & 0xffffffffu), mask, 64);
    const unsigned hi = __shfl_xor((unsigned)(v >> 32), mask, 64);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(kDraftThreads) void ngram_draft_kernel(
    const int32_t* __restrict__ history, int64_t ld, const int32_t* __restrict__ lengths, int n_max,
    int n_min, int K, int32_t* __restrict__ drafts) {
  __shared__ int32_t s_tok[kHalo + kTile];  // s_tok[i] = history[base + i]
  __shared__ int32_t s_suf[kNgramMaxN];     // s_suf[m] = history[L - 1 - m]
  __shared__ unsigned long long s_best[kDraftThreads / 64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int32_t* h = history + (size_t)b * ld;
  int L = lengths[b];
  L = L < 0 ? 0 : (L > ld ? (int)ld : L);
  const int nh = n_max < L - 1 ? n_max : L - 1;   // longest n with room for an earlier occurrence
  // key (score << 32) | e; 0 = no match (a match has score >= n_min >= 1)
  unsigned long long best = 0;
  int lo = 0, hi = -1, base = 0;                  // the tile held in LDS: candidates lo..hi
  if (nh >= n_min) {
    if (tid < nh) s_suf[tid] = h[L - 1 - tid];
    for (int top = L - 2; top >= n_min - 1 && (int)(best >> 32) < nh; top = lo - 1) {
      __syncthreads();                            // the previous tile is no longer read
      hi = top;
      lo = hi - kTile + 1 > n_min - 1 ? hi - kTile + 1 : n_min - 1;
      base = lo - kHalo;
      const int count = hi - base + 1;
      int32_t v[kStageRounds];
#pragma unroll
      for (int r = 0; r < kStageRounds; ++r) {
        const int i = tid + r * kDraftThreads, p = base + i;
        v[r] = (i < count && p >= 0) ? h[p] : 0;
      }
#pragma unroll
      for (int r = 0; r < kStageRounds; ++r) {
        const int i = tid + r * kDraftThreads;
        if (i < count) s_tok[i] = v[r];
      }
      __syncthreads();
      const int32_t last = s_suf[0];
      unsigned long long tb = 0;
      for (int e = hi - tid; e >= lo; e -= kDraftThreads) {
        const int i = e - base;
        if (s_tok[i] != last) continue;
        const int lim = nh < e + 1 ? nh : e + 1;  // i - m >= kHalo - 63 > 0 for every m < lim
        int m = 1;
        while (m < lim && s_tok[i - m] == s_suf[m]) ++m;
        if (m >= n_min) {
          const unsigned long long key = ((unsigned long long)m << 32) | (unsigned)e;
          tb = key > tb ? key : tb;
        }
      }
      tb = wave_max_u64(tb);
      if ((tid & 63) == 0) s_best[tid >> 6] = tb;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kDraftThreads / 64; ++w) best = s_best[w] > best ? s_best[w] : best;
    }
  }
  const int e = best ? (int)(best & 0xffffffffu) : -1;
  int32_t* d = drafts + (size_t)b * K;
  for (int j = tid; j < K; j += kDraftThreads) {
    const int p = e + 1 + j;
    int32_t t = -1;
    if (e >= 0 && p < L) {
      if (p == L - 1) t = s_suf[0];
      else if (e >= lo && p <= hi) t = s_tok[p - base];
      else t = h[p];
    }
    d[j] = t;
  }
}

__global__ __launch_bounds__(256) void append_accepted_kernel(
    int32_t* __restrict__ history, int64_t ld, int32_t* __restrict__ lengths, int B, int K,
    const int32_t* __restrict__ out_tokens, const int32_t* __restrict__ accepted_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int L = lengths[b];
  L = L < 0 ? 0 : (L > ld ? (int)ld : L);
  int a = accepted_len[b];
  a = a < 0 ? 0 : (a > K ? K : a);
  const int room = (int)(ld - L);
  const int cnt = a + 1 < room ? a + 1 : room;
  int32_t* h = history + (size_t)b * ld + L;
  const int32_t* o = out_tokens + (size_t)b * (K + 1);
  for (int j = 0; j < cnt; ++j) h[j] = o[j];
  lengths[b] = L + cnt;
}

}  // namespace

hipError_t launch_ngram_draft(const int32_t* history, int64_t ld, const int32_t* lengths, int B,
                              int n_max, int n_min, int K, int32_t* drafts, hipStream_t stream) {
  hipLaunchKernelGGL(ngram_draft_kernel, dim3(B), dim3(kDraftThreads), 0, stream, history, ld,
                     lengths, n_max, n_min, K, drafts);
  return hipGetLastError();
}

hipError_t launch_append_accepted(int32_t* history, int64_t ld, int32_t* lengths, int B, int K,
                                  const int32_t* out_tokens, const int32_t* accepted_len,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(append_accepted_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, history,
                     ld, lengths, B, K, out_tokens, accepted_len);
  return hipGetLastError();
}

}  // namespace w4v
