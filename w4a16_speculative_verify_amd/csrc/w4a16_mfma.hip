// W4A16 linear for many activation rows (the batched verify block of several
// sequences, prefill-shaped blocks), gfx950: a dense contraction bound by the
// matrix cores ("Efficient LLM Challenge Results", section 4: the long
// bucket's cost is prefill compute), so the 4-bit weights are dequantised
// once per block tile into LDS and shared by all of the tile's rows.
//
// Block tile 256 rows x 256 columns, 64 k per stage, two LDS stages:
//   A  the activations, copied global -> LDS by LDS DMA (buffer_load_dwordx4
//      ... lds, no registers), 16-byte chunks of 8 k placed at
//      slot = row * 8 + (chunk ^ (row % 8)) so that the MFMA A reads of 8
//      consecutive rows fall in different banks;
//   B  the packed words of the stage (8 packed rows x 256 columns), loaded
//      into registers, dequantised in natural k order to
//      fp16(s * (q - z)) -- q - z exact, one rounding for the scale, the
//      fp32 accumulation unchanged -- and stored as 8 k per 16-byte chunk at
//      slot = n * 8 + (chunk ^ ((n / 4) % 8)).
// 8 waves as 2 (rows) x 4 (columns), each 128 x 64: 8 x 4 v_mfma_f32_16x16x32_f16
// tiles with fp32 accumulators.  MFMA column j of the wave's column tile c is
// output column 4 j + c, so every lane ends up with 4 adjacent columns of each
// row it holds and stores them as one 8-byte write.  While a stage's MFMAs
// run, the next stage's A is in flight to the other LDS buffer and its packed
// words to registers; they are dequantised into LDS after the MFMAs.
// Blocks are ordered in groups of 8 row blocks, so that the blocks running
// together share their activation rows and packed weights in L2.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupM = 8;                          // row blocks per raster group
constexpr int kAStage = BM * BK * 2;                // 32 KiB
constexpr int kBStage = BN * BK * 2;                // 32 KiB

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4s dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// 16 bytes per lane global -> LDS at M0 + 16 * lane (M0 saved and restored);
// from inline assembly so that the compiler does not wait for these copies
// before every LDS access of the other stage (the kernel waits itself)
__device__ __forceinline__ void dma16(uint32_t lds_addr, u32x4s src, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(off), "s"(src)
      : "memory");
}

// packed word (8 consecutive k of one column) -> 8 fp16 s * (q - z) in natural
// k order: bytes of w and w >> 4 interleaved by v_perm so that pair p holds
// nibbles 2p and 2p + 1, each OR-ed under 1024.0 (exact 1024 + q), then
// - (1024 + z) exact, then * s rounded once
__device__ __forceinline__ u32x4 dequant_natural(uint32_t w, f16x2 z1024, f16x2 s, uint32_t magic) {
  const uint32_t w4 = w >> 4;
  const uint32_t p0 = (__builtin_amdgcn_perm(w4, w, 0x0c040c00u) & 0x000F000Fu) | magic;
  const uint32_t p1 = (__builtin_amdgcn_perm(w4, w, 0x0c050c01u) & 0x000F000Fu) | magic;
  const uint32_t p2 = (__builtin_amdgcn_perm(w4, w, 0x0c060c02u) & 0x000F000Fu) | magic;
  const uint32_t p3 = (__builtin_amdgcn_perm(w4, w, 0x0c070c03u) & 0x000F000Fu) | magic;
  auto f = [&](uint32_t p) {
    return __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, p) - z1024) * s);
  };
  return u32x4{f(p0), f(p1), f(p2), f(p3)};
}

// Split-K: block (tile, split) computes stages [stages * split / S, stages *
// (split + 1) / S); with S > 1 it stores fp32 partials [split][M][N] and a
// second kernel adds them in split order.
template <int Q>    // 1: group size 128, 4: group size 32
__global__ __launch_bounds__(kThreads) void w4a16_mfma_kernel(GemmArgs a, int mblocks, int nblocks,
                                                              int S, float* partials) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * (kAStage + kBStage)];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;          // 2 x 4 waves
  const int l16 = lane & 15, kb = lane >> 4;

  // raster: groups of kGroupM row blocks, column blocks inside a group
  const int bid = blockIdx.x;
  const int per_group = kGroupM * nblocks;
  const int grp = bid / per_group;
  const int m_first = grp * kGroupM;
  const int gm = mblocks - m_first < kGroupM ? mblocks - m_first : kGroupM;
  const int mblk = m_first + (bid % per_group) % gm;
  const int nblk = (bid % per_group) / gm;
  const int m0 = mblk * BM, n0 = nblk * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int split = blockIdx.y;
  const int s_lo = (K / BK) * split / S, s_hi = (K / BK) * (split + 1) / S;

  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)lds);
  auto a_lds = [&](int s) { return lds_base + (uint32_t)(s & 1) * (kAStage + kBStage); };
  auto a_ptr = [&](int s) { return lds + (s & 1) * (kAStage + kBStage); };
  auto b_ptr = [&](int s) { return a_ptr(s) + kAStage; };

  // ---- A copy: wave w moves rows 32 w .. 32 w + 31 (4 instructions of 8 rows)
  //      lane l of instruction i: LDS slot 64 i + l = row 8 i + l / 8, stored
  //      chunk l % 8 holding logical chunk (l % 8) ^ (row % 8)
  const u32x4s rx = dma_rsrc(a.x, 0x7fffffffu);
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int m = m0 + r < M ? m0 + r : M - 1;      // rows past M: read a valid row, never stored
    const int chunk = (lane & 7) ^ (r & 7);
    a_off[i] = ((uint32_t)m * (uint32_t)a.ldx + (uint32_t)chunk * 8) * 2;
  }
  auto copy_a = [&](int s) {
    const uint32_t base = a_lds(s) + (uint32_t)wave * 32 * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(base + i * 1024, rx, a_off[i] + (uint32_t)s * BK * 2);
  };

  // ---- B: thread t dequantises column n_t, chunks 4 h .. 4 h + 3 (32 k) of a
  //      stage, h = t / 256; lanes 8 j .. 8 j + 7 take columns whose n / 4
  //      differ, so that their LDS stores fall in different banks
  const int h = t >> 8;
  const int tn = t & 255;
  const int ncol = (tn & ~31) + ((tn & 7) << 2) + ((tn >> 3) & 3);
  const int gcol_raw = n0 + ncol;
  const bool col_ok = gcol_raw < N;
  const int gcol = col_ok ? gcol_raw : N - 1;
  const rsrc_t rw = make_rsrc(a.qweight), rs = make_rsrc(a.scales), rz = make_rsrc(a.qzeros);
  const uint32_t Nu = (uint32_t)N;
  auto load_b = [&](int s, uint32_t (&w)[4], uint32_t& zw, uint32_t& sv) {
    const uint32_t prow = (uint32_t)(s * BK / 8 + h * 4);         // first packed row
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = ld_x1(rw, ((prow + j) * Nu + (uint32_t)gcol) * 4);
    const uint32_t g = (uint32_t)((s * BK + h * 32) / (128 / Q));  // quantisation group
    zw = ld_x1(rz, (g * (Nu >> 3) + ((uint32_t)gcol >> 3)) * 4);
    sv = ld_x1(rs, (g * Nu + (uint32_t)gcol) * 2 & ~3u);          // the dword holding the scale
  };
  const uint32_t magic = in_vgpr(0x64006400u);
  auto store_b = [&](int s, const uint32_t (&w)[4], uint32_t zw, uint32_t sv) {
    const uint32_t z = (zw >> (4 * (gcol & 7))) & 0xFu;
    const f16x2 z1024 = __builtin_bit_cast(f16x2, (0x6400u | z) * 0x00010001u);
    const uint32_t sbits = (gcol & 1) ? (sv >> 16) : (sv & 0xffffu);
    const f16x2 sc = __builtin_bit_cast(f16x2, sbits * 0x00010001u);
    unsigned char* bp = b_ptr(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = h * 4 + j;
      const int slot = ncol * 8 + (chunk ^ ((ncol >> 2) & 7));
      *reinterpret_cast<u32x4*>(bp + slot * 16) = dequant_natural(w[j], z1024, sc, magic);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: the first stage in LDS
  uint32_t wr[4], zw, sv;
  copy_a(s_lo);
  load_b(s_lo, wr, zw, sv);
  store_b(s_lo, wr, zw, sv);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // MFMA A rows of this wave: 128 wm + 16 mt + l16; B columns: 64 wn + 4 j + c
  for (int s = s_lo; s < s_hi; ++s) {
    const bool more = s + 1 < s_hi;
    if (more) {
      copy_a(s + 1);
      load_b(s + 1, wr, zw, sv);
    }
    const unsigned char* ap = a_ptr(s);
    const unsigned char* bp = b_ptr(s);
#pragma unroll
    for (int it = 0; it < 2; ++it) {                // two 32-k slabs
      const int chunk = it * 4 + kb;
      f16x8 av[8], bv[4];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int r = wm * 128 + mt * 16 + l16;
        av[mt] = *reinterpret_cast<const f16x8*>(ap + (r * 8 + (chunk ^ (r & 7))) * 16);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = wn * 64 + 4 * l16 + c;
        bv[c] = *reinterpret_cast<const f16x8*>(bp + (n * 8 + (chunk ^ ((n >> 2) & 7))) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[mt][c] = mfma16x16x32(av[mt], bv[c], acc[mt][c]);
    }
    if (more) store_b(s + 1, wr, zw, sv);
    __builtin_amdgcn_s_waitcnt(0);                  // the next stage's A copies have landed
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 16 mt + 4 kb + e, columns 4 l16 .. + 3 of its tile
  const int col = n0 + wn * 64 + 4 * l16;
  if (col >= N) return;                             // N % 8 == 0: 4 columns all in or all out
  if (S > 1) {
    float* pp = partials + (size_t)split * M * N;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 128 + mt * 16 + 4 * kb + e;
        if (m < M) {
          const f32x4 v = {acc[mt][0][e], acc[mt][1][e], acc[mt][2][e], acc[mt][3][e]};
          *reinterpret_cast<f32x4*>(pp + (size_t)m * N + col) = v;
        }
      }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + wm * 128 + mt * 16 + 4 * kb + e;
      if (m < M) {
        const f16x2 lo = {(_Float16)(a.alpha * acc[mt][0][e]), (_Float16)(a.alpha * acc[mt][1][e])};
        const f16x2 hi = {(_Float16)(a.alpha * acc[mt][2][e]), (_Float16)(a.alpha * acc[mt][3][e])};
        const u32x2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<u32x2*>(a.y + (size_t)m * a.ldy + col) = v;
      }
    }
}

// y = fp16(alpha * sum of the S partials in split order), 4 columns per thread
__global__ __launch_bounds__(256) void w4a16_mfma_reduce_kernel(const float* __restrict__ partials,
                                                                int S, int M, int N, float alpha,
                                                                _Float16* __restrict__ y,
                                                                int64_t ldy) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const size_t total = (size_t)M * N;
  if (i >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(partials + i);
  for (int k = 1; k < S; ++k) s += *reinterpret_cast<const f32x4*>(partials + (size_t)k * total + i);
  const size_t m = i / N, n = i - m * N;
  const f16x2 lo = {(_Float16)(alpha * s[0]), (_Float16)(alpha * s[1])};
  const f16x2 hi = {(_Float16)(alpha * s[2]), (_Float16)(alpha * s[3])};
  *reinterpret_cast<u32x2*>(y + m * ldy + n) = u32x2{__builtin_bit_cast(uint32_t, lo),
                                                     __builtin_bit_cast(uint32_t, hi)};
}

}  // namespace

MfmaPlan plan_w4a16_mfma(int M, int N, int K, int num_cus) {
  MfmaPlan p{};
  p.mblocks = (M + BM - 1) / BM;
  p.nblocks = (N + BN - 1) / BN;
  const int tiles = p.mblocks * p.nblocks;
  const int stages = K / BK;
  // time ~ rounds of blocks (one block per CU) x stages per block, plus for
  // S > 1 the partials written and read again (2 S M N fp32 at ~5 TB/s, in
  // stage units of ~1 us) and the reduce launch
  double best = 0;
  p.splits = 1;
  for (int S = 1; S <= 32 && stages / S >= 4; ++S) {
    const double rounds = (double)((tiles * S + num_cus - 1) / num_cus);
    double t = rounds * ((stages + S - 1) / S);
    if (S > 1) t += 2.0 * S * M * (double)N * 4 / 5e6 + 3.0;
    if (S == 1 || t < best - 1e-9) {
      best = t;
      p.splits = S;
    }
  }
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
  return p;
}

hipError_t launch_w4a16_mfma(const GemmArgs& a, const MfmaPlan& p, float* partials,
                             hipStream_t stream) {
  const dim3 grid(p.mblocks * p.nblocks, p.splits);
  if (a.group_size == 32)
    hipLaunchKernelGGL(w4a16_mfma_kernel<4>, grid, dim3(kThreads), 0, stream, a, p.mblocks,
                       p.nblocks, p.splits, partials);
  else
    hipLaunchKernelGGL(w4a16_mfma_kernel<1>, grid, dim3(kThreads), 0, stream, a, p.mblocks,
                       p.nblocks, p.splits, partials);
  if (p.splits > 1) {
    const size_t quads = ((size_t)a.M * a.N + 3) / 4;
    hipLaunchKernelGGL(w4a16_mfma_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256),
                       0, stream, partials, p.splits, a.M, a.N, a.alpha, a.y, a.ldy);
  }
  return hipGetLastError();
}

}  // namespace w4v
