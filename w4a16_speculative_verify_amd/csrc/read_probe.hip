// HBM read-bandwidth probe (a measurement helper, no step of the verify
// path): every byte of the source is read once with 16-byte non-temporal
// loads, four in flight per thread, and each block writes the XOR of what it
// read, so that no load can be dropped.  Timed around, it gives the read
// bandwidth the device reaches, the practical ceiling beside the 8 TB/s peak
// for the HBM-bound kernels.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kProbeThreads = 512;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src,
                                                                   size_t n16, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) ^ (b[0] ^ b[1] ^ b[2] ^ b[3]) ^ (c[0] ^ c[1] ^ c[2] ^ c[3]) ^
         (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace w4v
