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
// append_accepted: one thread per sequence appends out_tokens[b][0..a_b].
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kDraftThreads = 256;

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
  const int b = blockIdx.x;
  const int32_t* h = history + (size_t)b * ld;
  int L = lengths[b];
  L = L < 0 ? 0 : (L > ld ? (int)ld : L);
  const int nh = n_max < L - 1 ? n_max : L - 1;   // longest n with room for an earlier occurrence
  // key (score << 32) | e; 0 = no match (a match has score >= n_min >= 1)
  unsigned long long best = 0;
  if (nh >= n_min) {
    const int32_t last = h[L - 1];
    for (int e = L - 2 - (int)threadIdx.x; e >= n_min - 1; e -= kDraftThreads) {
      if (h[e] != last) continue;
      const int lim = nh < e + 1 ? nh : e + 1;
      int m = 1;
      while (m < lim && h[e - m] == h[L - 1 - m]) ++m;
      if (m >= n_min) {
        const unsigned long long key = ((unsigned long long)m << 32) | (unsigned)e;
        best = key > best ? key : best;
      }
    }
  }
  __shared__ unsigned long long s_best[kDraftThreads / 64];
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kDraftThreads / 64; ++w) best = s_best[w] > best ? s_best[w] : best;
  const int e = best ? (int)(best & 0xffffffffu) : -1;
  int32_t* d = drafts + (size_t)b * K;
  for (int j = threadIdx.x; j < K; j += kDraftThreads)
    d[j] = (e >= 0 && e + 1 + j < L) ? h[e + 1 + j] : -1;
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
