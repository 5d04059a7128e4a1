// Committing a Gated DeltaNet state to the accepted prefix of a verify block,
// gfx950.  The results page (hazards list; section 3 on the runner-up's fix)
// traces wrong answers to recurrent state that rejected speculative drafts
// left behind.  Here the state committed before the block is updated only by
// the positions the verify accepted: position 0 (the last committed token)
// and the a_b accepted drafts, a_b + 1 steps of the gated delta rule (the
// update of the Gated DeltaNet paper the pages cite):
//
//   S <- alpha_t * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
//      = alpha_t * S + (beta_t v_t - alpha_t beta_t (S k_t)) k_t^T
//
// One block of 256 threads per (sequence, head).  The fp32 state [dv x dk]
// (dv = dk = D) stays in registers for all the steps: thread t owns row
// t / TPR and CPT consecutive columns of it.  The block's keys, values and
// gates for up to kGdnMaxT positions are staged in LDS first (one batch of
// masked loads per thread, so the steps wait for memory once); each step then
// forms S k_t with a partial dot product per thread and a shuffle across the
// row's TPR threads, and applies the rank-one update.  Every lane of a wave
// reads the same few key addresses from LDS (broadcast).  HBM-bound: the
// state is read and written once, 8 D^2 bytes per head.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void gdn_commit_kernel(
    float* __restrict__ state, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ accepted_len, int T, int H) {
  constexpr int TPR = kThreads / D;                 // threads per state row
  constexpr int CPT = D / TPR;                      // columns per thread
  constexpr int kStage = D * kGdnMaxT / kThreads;   // staged floats per thread, keys and values each
  __shared__ __attribute__((aligned(16))) float sk[kGdnMaxT][D];
  __shared__ float sv[kGdnMaxT][D];
  __shared__ float sa[kGdnMaxT], sb[kGdnMaxT];

  const int tid = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  int a = accepted_len[b];
  a = a < 0 ? 0 : (a > T - 1 ? T - 1 : a);
  const int n = a + 1;                              // steps to apply

  // ---- the state rows of this thread, then keys, values and gates of the n
  // positions: every load issued before the first wait, positions past n
  // masked off (no load under a branch)
  const int row = tid / TPR, c0 = (tid % TPR) * CPT;
  float* srow = state + (((size_t)b * H + h) * D + row) * D + c0;
  f32x4 sq[CPT / 4];
#pragma unroll
  for (int j = 0; j < CPT / 4; ++j) sq[j] = *reinterpret_cast<const f32x4*>(srow + 4 * j);
  const rsrc_t rk = make_rsrc(k), rv = make_rsrc(v), ra = make_rsrc(alpha), rb = make_rsrc(beta);
  float stk[kStage], stv[kStage];
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int e = tid + u * kThreads;               // element e of [pos][D]
    const int pos = e / D, c = e % D;
    const uint32_t off = (((uint32_t)((b * T + pos) * H + h) * D + c) * 4) |
                         ((uint32_t)(pos >= n) << 31);
    stk[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rk, off, 0, 0));
    stv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0));
  }
  const int gp = tid % kGdnMaxT;
  const uint32_t goff = (((uint32_t)((b * T + gp) * H + h)) * 4) | ((uint32_t)(gp >= n) << 31);
  const float ga = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, goff, 0, 0));
  const float gb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, goff, 0, 0));

  float s[CPT];
#pragma unroll
  for (int j = 0; j < CPT / 4; ++j) {
    s[4 * j] = sq[j][0]; s[4 * j + 1] = sq[j][1]; s[4 * j + 2] = sq[j][2]; s[4 * j + 3] = sq[j][3];
  }
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int e = tid + u * kThreads;
    sk[e / D][e % D] = stk[u];
    sv[e / D][e % D] = stv[u];
  }
  if (tid < kGdnMaxT) {
    sa[tid] = ga;
    sb[tid] = gb;
  }
  __syncthreads();

  // ---- the n steps of the gated delta rule
  for (int t = 0; t < n; ++t) {                     // block-uniform trip count
    const float* kt = &sk[t][c0];
    float kv[CPT];
#pragma unroll
    for (int j = 0; j < CPT; j += 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(kt + j);
      kv[j] = q[0]; kv[j + 1] = q[1]; kv[j + 2] = q[2]; kv[j + 3] = q[3];
    }
    float u = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) u = __builtin_fmaf(s[j], kv[j], u);
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) u += __shfl_xor(u, m, 64);
    const float al = sa[t], be = sb[t];
    const float cf = be * sv[t][row] - al * be * u;
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = __builtin_fmaf(al, s[j], cf * kv[j]);
  }

#pragma unroll
  for (int j = 0; j < CPT; j += 4)
    *reinterpret_cast<f32x4*>(srow + j) = f32x4{s[j], s[j + 1], s[j + 2], s[j + 3]};
}

}  // namespace

hipError_t launch_gdn_commit(float* state, const float* k, const float* v, const float* alpha,
                             const float* beta, const int32_t* accepted_len, int B, int T, int H,
                             int D, hipStream_t stream) {
  const dim3 grid(H, B);
  if (D == 128)
    hipLaunchKernelGGL(gdn_commit_kernel<128>, grid, dim3(kThreads), 0, stream, state, k, v, alpha,
                       beta, accepted_len, T, H);
  else if (D == 64)
    hipLaunchKernelGGL(gdn_commit_kernel<64>, grid, dim3(kThreads), 0, stream, state, k, v, alpha,
                       beta, accepted_len, T, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace w4v
