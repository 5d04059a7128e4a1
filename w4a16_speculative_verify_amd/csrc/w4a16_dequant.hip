// W4A16 weights expanded to fp16 for the linear at 33 rows and more (the
// batched verify block, prefill shapes), gfx950.  Section 4 of the
// organisers' results page puts long prompts in prefill compute: there the
// product is a dense contraction bound by the matrix cores, and a plain fp16
// GEMM on dequantised weights runs it at about twice the rate of the fused
// in-register kernel; at the batched verify block (M = 168) the pair is also
// twice as fast as that kernel, which has too few blocks (measured on MI355X).
//
//   wt[n, k] = fp16_rne( float(s[k/gs, n]) * (q[k, n] - z[k/gs, n]) ),  gs = 128 or 32
//
// written transposed (row n holds all K values of column n), the layout in
// which both GEMM operands are contiguous along k.  The product in fp32 is
// exact (an 11-bit scale times a 5-bit integer), so each weight is rounded
// once.  HBM-bound: K*N/2 + scales + zeros read, 2*K*N written.
//
// A block expands 128 k of 64 columns (one group, or four of 32 k: wave w's
// four packed rows then form group 4 * step + w): its 16 x 64 packed words are
// read row by row (each wave instruction covers 256 contiguous bytes), the
// 64 x 128 fp16 values are transposed through LDS, and each output row's 256
// bytes are written by 16 adjacent lanes.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kCols = 64;                   // columns per block (one per lane)
constexpr int kRowHalves = kGroup + 8;      // LDS row: 128 k + 16 bytes of padding

__global__ __launch_bounds__(256) void dequant_w4_f16t_kernel(
    const uint32_t* __restrict__ qweight, const _Float16* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int K, int N, int q4, _Float16* __restrict__ wt) {
  __shared__ _Float16 tile[kCols * kRowHalves];
  const int t = threadIdx.x;
  const int g = blockIdx.y;
  const int n0 = blockIdx.x * kCols;
  const int nl = t & (kCols - 1), wave = t >> 6;
  const int n = n0 + nl;
  if (n < N) {
    const int qg = q4 ? 4 * g + wave : g;           // quantisation group of this wave's rows
    const float s = (float)scales[(size_t)qg * N + n];
    const int z = (int)((qzeros[(size_t)qg * (N >> 3) + (n >> 3)] >> (4 * (n & 7))) & 0xFu);
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = qweight[(size_t)(g * 16 + wave * 4 + r) * N + n];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t h[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int q0 = (int)((w[r] >> (8 * p)) & 0xFu), q1 = (int)((w[r] >> (8 * p + 4)) & 0xFu);
        const f16x2 v = {(_Float16)(s * (float)(q0 - z)), (_Float16)(s * (float)(q1 - z))};
        h[p] = __builtin_bit_cast(uint32_t, v);
      }
      *reinterpret_cast<u32x4*>(tile + nl * kRowHalves + (wave * 4 + r) * 8) = u32x4{h[0], h[1], h[2], h[3]};
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = t + 256 * p;                      // 16-byte chunk c of the 64 x 256-byte tile
    const int row = c >> 4, part = c & 15;
    if (n0 + row < N)
      *reinterpret_cast<u32x4*>(wt + (size_t)(n0 + row) * K + (size_t)g * kGroup + part * 8) =
          *reinterpret_cast<const u32x4*>(tile + row * kRowHalves + part * 8);
  }
}

}  // namespace

hipError_t launch_dequant_w4_f16t(const uint32_t* qweight, const _Float16* scales,
                                  const uint32_t* qzeros, int K, int N, int group_size,
                                  _Float16* wt, hipStream_t stream) {
  const dim3 grid((N + kCols - 1) / kCols, K / kGroup);
  hipLaunchKernelGGL(dequant_w4_f16t_kernel, grid, dim3(256), 0, stream, qweight,
                     scales, qzeros, K, N, group_size == 32 ? 1 : 0, wt);
  return hipGetLastError();
}

}  // namespace w4v
