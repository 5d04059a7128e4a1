// Greedy prefix acceptance ("Efficient LLM Challenge Results", section 3:
// drafts are kept only as far as each one equals the token the target picks
// greedily after the drafts before it; -1 padding can never equal a
// vocabulary id, so padding never extends the accepted run).  One thread per
// sequence; the scan stops at the first draft that is out of [0, V) or
// differs from the target's token.
#include "w4v_launch.h"

namespace w4v {

namespace {

__global__ __launch_bounds__(256) void greedy_verify_kernel(const int32_t* __restrict__ target_ids,
                                                            const int32_t* __restrict__ draft_ids,
                                                            int B, int K, int V,
                                                            int32_t* __restrict__ accepted_len,
                                                            int32_t* __restrict__ out_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* t = target_ids + (size_t)b * (K + 1);
  const int32_t* d = draft_ids + (size_t)b * K;
  int a = 0;
  while (a < K) {
    const int dv = d[a];
    if (dv < 0 || dv >= V || dv != t[a]) break;
    ++a;
  }
  accepted_len[b] = a;
  int32_t* o = out_tokens + (size_t)b * (K + 1);
  for (int j = 0; j <= K; ++j) o[j] = (j <= a) ? t[j] : -1;
}

}  // namespace

hipError_t launch_greedy_verify(const int32_t* target_ids, const int32_t* draft_ids, int B, int K,
                                int V, int32_t* accepted_len, int32_t* out_tokens,
                                hipStream_t stream) {
  const int threads = 256;
  const int blocks = (B + threads - 1) / threads;
  hipLaunchKernelGGL(greedy_verify_kernel, dim3(blocks), dim3(threads), 0, stream, target_ids,
                     draft_ids, B, K, V, accepted_len, out_tokens);
  return hipGetLastError();
}

}  // namespace w4v
