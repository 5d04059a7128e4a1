// W4A16 linear for many activation rows without a workspace (prefill-shaped,
// the batched verify block of several sequences; with a workspace the
// library expands the weights to fp16 and runs a plain GEMM instead, and
// this kernel is its fallback when no plan exists), gfx950: an LDS-tiled
// MFMA GEMM with the exact in-register dequantisation.
// Section 4 of the organisers' results page puts the long-prompt cost in
// prefill compute; at M = 2,048-8,192 rows the W4A16 linear is a dense
// contraction bound by the matrix cores, not by HBM.
//
// Block tile 128 (rows) x 128 (columns), 128 k per K-step, 4 waves as 2 x 2 sub-tiles of 64 x 64 (4 x 4 MFMA 16x16x32 tiles).
//   A (activations): the block's 128 x 128 fp16 slice goes through LDS,
//     double-buffered, with the k order inside each 8-element block permuted
//     to match the dequantised nibbles; rows are padded by 16 bytes so the 16
//     rows of one MFMA operand read fall in different banks.
//   B (weights): every lane loads its own packed words straight from global
//     memory (4 columns x 8 k per 128-bit load, the lane layout of the MFMA B
//     operand), dequantises them in registers exactly (fp16 q - z), and each
//     quantisation group's fp16 scale multiplies the fp32 sum of the group
//     once (group size 128, or 32: four groups per K-step).
//   Weights run two groups ahead in a three-deep register ring, the next
//   group's activations are requested before the current group's MFMAs; the
//   per-group barrier orders LDS only, so loads stay in flight across it.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kRowBytes = BK * 2 + 16;            // padded LDS row of A
constexpr int kRowWords = kRowBytes / 4;
constexpr int DB = 3;                             // weight groups in flight per lane

// Q quantisation groups per 128-k step (1: group size 128; 4: group size 32)
template <int Q>
struct BFrag {
  u32x4 w[4];       // 4 quads of packed rows, 4 columns each
  uint32_t zw[Q];   // the zero-point words (the lane's 4 columns at zshift)
  u32x2 s[Q];       // 4 fp16 scales per quantisation group
};

// Lane byte offsets of step 0's loads; the weight stride per 128-k step, the
// zero-point and scale strides per quantisation group.
struct BLanes {
  uint32_t w, wq, gw, z, gz, s, gs;
};

// Group g's packed words, zero-point word and scales; a group past the last
// one reads zeros without touching memory (offset pushed past the resource).
template <int Q>
__device__ __forceinline__ void load_b(BFrag<Q>& f, const rsrc_t& rw, const rsrc_t& rz,
                                       const rsrc_t& rs, const BLanes& o, int g, int G) {
  const uint32_t gg = (uint32_t)(g < G ? g : 0);
  const uint32_t skip = g < G ? 0u : kNoLoad;
#pragma unroll
  for (int it = 0; it < 4; ++it) f.w[it] = ld_x4<kNT>(rw, (o.w + it * o.wq + gg * o.gw) | skip);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    f.zw[q] = ld_x1(rz, (o.z + (gg * Q + q) * o.gz) | skip);
    f.s[q] = ld_x2(rs, (o.s + (gg * Q + q) * o.gs) | skip);
  }
}

// A tile loads: thread t moves 8 consecutive k (16 bytes) of rows t/16 + 16 j.
struct AFrag {
  u32x4 v[8];
};

__device__ __forceinline__ void load_a(AFrag& f, const rsrc_t& rx, const uint32_t (&oa)[8], int g,
                                       int G) {
  const uint32_t skip = g < G ? (uint32_t)g * BK * 2 : kNoLoad;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = ld_x4(rx, oa[j] + skip);
}

__device__ __forceinline__ void store_a(uint32_t* lds, const AFrag& f, int rows_ok, int t) {
  const int chunk = t & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (t >> 4) + 16 * j;
    const f16x8 p = permute_for_int4(r < rows_ok ? f.v[j] : u32x4{0u, 0u, 0u, 0u});
    *reinterpret_cast<u32x4*>(lds + r * kRowWords + chunk * 4) = __builtin_bit_cast(u32x4, p);
  }
}

template <int Q>
__global__ __launch_bounds__(kThreads) void w4a16_tiled_kernel(GemmArgs a) {
  __shared__ uint32_t As[2][BM * kRowWords];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int kb = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = a.K / BK;
  const int rows_ok = a.M - m0;                     // rows of this tile that exist

  const int col_raw = n0 + wn * 64 + 4 * (lane & 15);
  const bool colok = col_raw < a.N;
  const int col = colok ? col_raw : a.N - 4;        // columns past N read valid words
  const int zshift = (col & 4) * 4;
  const uint32_t magic = in_vgpr(0x64006400u);

  const rsrc_t rw = make_rsrc(a.qweight), rz = make_rsrc(a.qzeros), rs = make_rsrc(a.scales);
  const rsrc_t rx = make_rsrc(a.x);
  const uint32_t N = (uint32_t)a.N;
  BLanes ob;
  ob.w = ((uint32_t)kb * N + col) * 4;
  ob.wq = 16 * N;
  ob.gw = 64 * N;
  ob.z = (uint32_t)(col >> 3) * 4;
  ob.gz = (N >> 3) * 4;
  ob.s = (uint32_t)col * 2;
  ob.gs = N * 2;
  uint32_t oa[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + (t >> 4) + 16 * j;
    const int mm = m < a.M ? m : a.M - 1;           // rows past M read a valid row, zeroed on store
    oa[j] = ((uint32_t)mm * (uint32_t)a.ldx + (t & 15) * 8) * 2;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue in the loop's order: weights of groups 0 .. DB-1, then A of group 0
  BFrag<Q> bf[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    load_b(bf[i], rw, rz, rs, ob, i, G);
    __builtin_amdgcn_sched_barrier(0);
  }
  AFrag af;
  load_a(af, rx, oa, 0, G);
  store_a(As[0], af, rows_ok, t);
  lds_barrier();

  // steps padded to a multiple of DB: a padding step loads and computes
  // nothing, so no load sits under a branch
  const int gsteps = (G + DB - 1) / DB * DB;
  for (int g0 = 0; g0 < gsteps; g0 += DB) {
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      const int g = g0 + i;
      // the next group's activations, staged into the other LDS buffer below
      load_a(af, rx, oa, g + 1, G);
      if (g < G) {                                  // block-uniform
        const uint32_t* as = As[g & 1];
        // per quantisation group: exact fp16 (q - z) operands, the group's
        // fp32 sum over its 128 / Q k, then its scale once
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          ZeroPair zz[4];
          {
            const uint32_t zw = bf[i].zw[q] >> zshift;
#pragma unroll
            for (int c = 0; c < 4; ++c) zz[c] = zero_pair((zw >> (4 * c)) & 0xFu);
          }
          f32x4 tmp[4][4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) tmp[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int it = q * (4 / Q); it < (q + 1) * (4 / Q); ++it) {
            f16x8 av[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = wm * 64 + r * 16 + (lane & 15);
              av[r] = __builtin_bit_cast(
                  f16x8, *reinterpret_cast<const u32x4*>(as + row * kRowWords + it * 16 + kb * 4));
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const f16x8 bv = dequant_int4_word(bf[i].w[it][c], zz[c], magic);
#pragma unroll
              for (int r = 0; r < 4; ++r) tmp[r][c] = mfma16x16x32(av[r], bv, tmp[r][c]);
            }
          }
          // copy the vector elements to scalars before the bit casts: a bit
          // cast of an ext-vector element expression reads element 0 with
          // this compiler
          const uint32_t s_lo = bf[i].s[q].x, s_hi = bf[i].s[q].y;
          const f16x2 s01 = __builtin_bit_cast(f16x2, s_lo);
          const f16x2 s23 = __builtin_bit_cast(f16x2, s_hi);
          const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[r][c][e] = __builtin_fmaf(sc[c], tmp[r][c][e], acc[r][c][e]);
        }
      }
      load_b(bf[i], rw, rz, rs, ob, g + DB, G);
      store_a(As[(g + 1) & 1], af, rows_ok, t);
      lds_barrier();
    }
  }

  // epilogue: lane holds rows 4*(l/16)+e of each m-tile, columns col..col+3
  if (!colok) return;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + wm * 64 + r * 16 + 4 * kb + e;
      if (m < a.M) {
        const f16x2 lo = {(_Float16)(a.alpha * acc[r][0][e]), (_Float16)(a.alpha * acc[r][1][e])};
        const f16x2 hi = {(_Float16)(a.alpha * acc[r][2][e]), (_Float16)(a.alpha * acc[r][3][e])};
        const u32x2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<u32x2*>(a.y + (size_t)m * a.ldy + col_raw) = v;
      }
    }
}

}  // namespace

hipError_t launch_w4a16_tiled(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  if (a.group_size == 32)
    hipLaunchKernelGGL(w4a16_tiled_kernel<4>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(w4a16_tiled_kernel<1>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace w4v
