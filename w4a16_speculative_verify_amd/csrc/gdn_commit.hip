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
// The update of a state row needs only that row and k_t (u_i = S_i . k_t):
// one block per (sequence, head) with 8 threads per state row (1,024 threads
// at dv = dk = D = 128), the fp32 state in registers for all the steps.  A
// thread holds every 8th 16-byte chunk of its row, so the 8 threads of a row
// read and write one whole 128-byte line per instruction (a thread owning a
// contiguous half of its row made each instruction touch 64 lines, and the
// kernel 1.5x slower).  The block's keys, values and gates for up to
// kGdnMaxT positions are staged in LDS first (one batch of masked loads per
// thread, so the steps wait for memory once); each step then forms S k_t
// with a partial dot product per thread and a 3-level shuffle across the
// row's threads, and applies the rank-one update.  HBM-bound: the state is
// read and written once, 8 D^2 bytes per head.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kTPR = 8;                            // threads per state row

template <int D>
__global__ __launch_bounds__(D * kTPR) void gdn_commit_kernel(
    float* __restrict__ state, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ accepted_len, int T, int H) {
  constexpr int NT = D * kTPR;                      // threads per block
  constexpr int CPT = D / kTPR;                     // columns per thread
  constexpr int NC = CPT / 4;                       // 16-byte chunks per thread
  constexpr int kStage = D * kGdnMaxT / NT;         // staged floats per thread, keys and values each
  __shared__ __attribute__((aligned(16))) float sk[kGdnMaxT][D];
  __shared__ float sv[kGdnMaxT][D];
  __shared__ float sa[kGdnMaxT], sb[kGdnMaxT];

  const int tid = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  int a = accepted_len[b];
  a = a < 0 ? 0 : (a > T - 1 ? T - 1 : a);
  const int n = a + 1;                              // steps to apply

  // ---- the state chunks of this thread, then keys, values and gates of the n
  // positions: every load issued before the first wait, positions past n
  // masked off (no load under a branch).  Chunk j of the thread holds columns
  // 4 (j kTPR + r) .. + 3, r = tid % kTPR: the kTPR threads of a row read one
  // whole 128-byte line per instruction.
  const int row = tid / kTPR, r = tid % kTPR;
  float* srow = state + (((size_t)b * H + h) * D + row) * D + 4 * r;
  f32x4 sq[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) sq[j] = *reinterpret_cast<const f32x4*>(srow + 4 * kTPR * j);
  const rsrc_t rk = make_rsrc(k), rv = make_rsrc(v), ra = make_rsrc(alpha), rb = make_rsrc(beta);
  float stk[kStage], stv[kStage];
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int e = tid + u * NT;                     // element e of [pos][D]
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
  for (int j = 0; j < NC; ++j) {
    s[4 * j] = sq[j][0]; s[4 * j + 1] = sq[j][1]; s[4 * j + 2] = sq[j][2]; s[4 * j + 3] = sq[j][3];
  }
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int e = tid + u * NT;
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
    float kv[CPT];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(&sk[t][4 * (j * kTPR + r)]);
      kv[4 * j] = q[0]; kv[4 * j + 1] = q[1]; kv[4 * j + 2] = q[2]; kv[4 * j + 3] = q[3];
    }
    float u = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) u = __builtin_fmaf(s[j], kv[j], u);
#pragma unroll
    for (int m = 1; m < kTPR; m <<= 1) u += __shfl_xor(u, m, 64);
    const float al = sa[t], be = sb[t];
    const float cf = be * sv[t][row] - al * be * u;
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = __builtin_fmaf(al, s[j], cf * kv[j]);
  }

#pragma unroll
  for (int j = 0; j < NC; ++j)
    *reinterpret_cast<f32x4*>(srow + 4 * kTPR * j) =
        f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
}

}  // namespace

hipError_t launch_gdn_commit(float* state, const float* k, const float* v, const float* alpha,
                             const float* beta, const int32_t* accepted_len, int B, int T, int H,
                             int D, hipStream_t stream) {
  const dim3 grid(H, B);
  if (D == 128)
    hipLaunchKernelGGL(gdn_commit_kernel<128>, grid, dim3(128 * kTPR), 0, stream, state, k, v,
                       alpha, beta, accepted_len, T, H);
  else if (D == 64)
    hipLaunchKernelGGL(gdn_commit_kernel<64>, grid, dim3(64 * kTPR), 0, stream, state, k, v,
                       alpha, beta, accepted_len, T, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace w4v
