// W4A16 linear for a skinny block of activation rows (the verify block of
// K+1 rows, section 3 of the organisers' results page), gfx950.
//
// Work decomposition
//   block  = 4 waves on one 64-column tile and one K-split; the waves divide
//            the split's groups (128 k each) between them, at most GW each.
//   lane l = columns col..col+3 with col = tile*64 + 4*(l % 16), packed row
//            4*it + l/16 of every 4-row quad; one 128-bit load brings 4 words
//            = 4 columns x 8 k, the B operands of 4 MFMAs (one per column).
//   A      = the activation rows, read straight from global memory (the block
//            of rows is small and stays in L2), reordered in registers to the
//            k order of the dequantised nibbles.
// A wave issues the loads of all its groups (weights, zero-points, scales and
// activations) before it computes anything, so the whole weight matrix is in
// flight at once when the grid covers it: the skinny linear is bound by HBM
// latency and bandwidth, not by arithmetic.
// Per group the int4 words become exact fp16 (q - z); four 16x16x32 MFMAs per
// column accumulate X * (q - z) over the group's 128 k in fp32, and the
// group's fp16 scale is applied once to that fp32 sum (exact algebra: the
// scale is constant over the group).  Waves of a block then add their fp32
// results in fixed order through LDS; with split-K > 1 the blocks of a tile
// publish fp32 partials and the last block to arrive adds them in split
// order, so the output does not depend on arrival order.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int MT>
struct GroupFrag {
  u32x4 w[4];        // 4 quads of packed rows, 4 columns each
  uint32_t zw;       // zero-point nibbles of the lane's 4 columns (low 16 bits)
  u32x2 s;           // 4 fp16 scales
  u32x4 a[MT][4];    // activations: per m-tile, per quad, 8 consecutive k
};

template <int MT>
__device__ __forceinline__ void load_group(GroupFrag<MT>& f, int g, const GemmArgs& a, int col,
                                           bool colok, int kb, int row0) {
  const int N = a.N;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (colok) {
      f.w[it] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(a.qweight + (size_t)(g * 16 + it * 4 + kb) * N + col));
    } else {
      f.w[it] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  if (colok) {
    f.zw = a.qzeros[(size_t)g * (N >> 3) + (col >> 3)] >> ((col & 4) * 4);
    f.s = *reinterpret_cast<const u32x2*>(a.scales + (size_t)g * N + col);
  } else {
    f.zw = 0u;
    f.s = u32x2{0u, 0u};
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = row0 + mt * 16;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (m < a.M) {
        f.a[mt][it] = *reinterpret_cast<const u32x4*>(a.x + (size_t)m * a.ldx + g * kGroup +
                                                        it * 32 + kb * 8);
      } else {
        f.a[mt][it] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

template <int MT>
__device__ __forceinline__ void compute_group(const GroupFrag<MT>& f, f32x4 (&acc)[MT][4],
                                              uint32_t magic) {
  ZeroPair zz[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) zz[c] = zero_pair((f.zw >> (4 * c)) & 0xFu);
  f32x4 tmp[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) tmp[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    f16x8 av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) av[mt] = permute_for_int4(f.a[mt][it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x8 b = dequant_int4_word(f.w[it][c], zz[c], magic);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) tmp[mt][c] = mfma16x16x32(av[mt], b, tmp[mt][c]);
    }
  }
  // copy the vector elements to scalars before the bit casts: a bit cast of
  // an ext-vector element expression reads element 0 with this compiler
  const uint32_t s_lo = f.s.x, s_hi = f.s.y;
  const f16x2 s01 = __builtin_bit_cast(f16x2, s_lo);
  const f16x2 s23 = __builtin_bit_cast(f16x2, s_hi);
  const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][c][r] = __builtin_fmaf(sc[c], tmp[mt][c][r], acc[mt][c][r]);
}

__device__ __forceinline__ void store_row4(_Float16* dst, float a0, float a1, float a2, float a3) {
  const f16x2 lo = {(_Float16)a0, (_Float16)a1};
  const f16x2 hi = {(_Float16)a2, (_Float16)a3};
  const u32x2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  *reinterpret_cast<u32x2*>(dst) = v;
}

template <int MT, int GW>
__global__ __launch_bounds__(kThreads) void w4a16_skinny_kernel(GemmArgs a, int splits,
                                                                unsigned* tickets, float* partials) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int mblk = blockIdx.z;
  const int G = a.K / kGroup;

  // groups of this split, then of this wave
  const int gs0 = (int)((long long)G * split / splits);
  const int gs1 = (int)((long long)G * (split + 1) / splits);
  const int glen = gs1 - gs0;
  const int g0 = gs0 + glen * wave / kWaves;
  const int g1 = gs0 + glen * (wave + 1) / kWaves;

  const int col = tile * kColTile + 4 * (lane & 15);
  const bool colok = col < a.N;                    // N % 8 == 0: 4 columns all valid or none
  const int kb = lane >> 4;
  const int mbase = mblk * 16 * MT;
  const int row_a = mbase + (lane & 15);           // A-operand row of this lane (m-tile 0)

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t magic = in_vgpr(0x64006400u);
  // batches of up to GW groups: all loads of a batch first, then the math
  for (int gb = g0; gb < g1; gb += GW) {
    GroupFrag<MT> f[GW];
#pragma unroll
    for (int i = 0; i < GW; ++i)
      if (gb + i < g1) load_group<MT>(f[i], gb + i, a, col, colok, kb, row_a);
#pragma unroll
    for (int i = 0; i < GW; ++i)
      if (gb + i < g1) compute_group<MT>(f[i], acc, magic);
  }

  // ---- combine the 4 waves in fixed order through LDS
  // element e = (mt*4 + r)*4 + c of lane l sits at red[wave][e][l]
  constexpr int E = MT * 16;
  __shared__ float red[kWaves][E][64];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[wave][(mt * 4 + r) * 4 + c][lane] = acc[mt][c][r];
  __syncthreads();

  // wave w finishes rows (mt, r = w): MT rows per lane, 4 columns each
  float out[MT][4];
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int mr = j * 4 + wave;      // (mt*4 + r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float s = red[0][mr * 4 + c][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s += red[w][mr * 4 + c][lane];
      out[j][c] = s;
    }
  }

  const int ntiles = gridDim.x;
  auto row_of = [&](int j) {
    const int mr = j * 4 + wave;
    const int mt = mr >> 2, r = mr & 3;
    return mbase + mt * 16 + 4 * (lane >> 4) + r;
  };

  if (splits == 1) {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int m = row_of(j);
      if (colok && m < a.M)
        store_row4(a.y + (size_t)m * a.ldy + col, a.alpha * out[j][0], a.alpha * out[j][1],
                   a.alpha * out[j][2], a.alpha * out[j][3]);
    }
    return;
  }

  // ---- split-K: publish this block's partial, the last block of the tile reduces
  // partials layout: [mblk][split][16*MT rows][ntiles*64 cols]
  const size_t ncols = (size_t)ntiles * kColTile;
  const size_t rows_blk = 16 * MT;
  float* pbase = partials + (size_t)mblk * splits * rows_blk * ncols;
  const rsrc_t pr = make_rsrc(pbase);
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int mloc = row_of(j) - mbase;
    const f32x4 v = {out[j][0], out[j][1], out[j][2], out[j][3]};
    st_agent_x4(pr, (uint32_t)((((size_t)split * rows_blk + mloc) * ncols + col) * 4),
                __builtin_bit_cast(u32x4, v));
  }
  if (!arrive_last(tickets + (size_t)mblk * ntiles + tile, (unsigned)splits)) return;

#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = row_of(j);
    const int mloc = m - mbase;
    f32x4 s = __builtin_bit_cast(f32x4, ld_agent_x4(pr, (uint32_t)(((size_t)mloc * ncols + col) * 4)));
    for (int sp = 1; sp < splits; ++sp)
      s += __builtin_bit_cast(
          f32x4, ld_agent_x4(pr, (uint32_t)((((size_t)sp * rows_blk + mloc) * ncols + col) * 4)));
    if (colok && m < a.M)
      store_row4(a.y + (size_t)m * a.ldy + col, a.alpha * s[0], a.alpha * s[1], a.alpha * s[2],
                 a.alpha * s[3]);
  }
}

template <int MT, int GW>
void launch_t(const GemmArgs& a, const GemmPlan& p, unsigned* tickets, float* partials,
              hipStream_t stream) {
  hipLaunchKernelGGL((w4a16_skinny_kernel<MT, GW>), dim3(p.col_tiles, p.splits, p.mblocks),
                     dim3(kThreads), 0, stream, a, p.splits, tickets, partials);
}

}  // namespace

GemmPlan plan_w4a16(int M, int N, int K, int num_cus) {
  GemmPlan p{};
  p.mt = (M <= 16) ? 1 : 2;
  const int rows_blk = 16 * p.mt;
  p.mblocks = (M + rows_blk - 1) / rows_blk;
  p.col_tiles = (N + kColTile - 1) / kColTile;
  const int G = K / kGroup;
  const int gw_max = (p.mt == 1) ? 4 : 2;
  int splits = 1;
  if (p.mblocks == 1 && (size_t)p.col_tiles <= kMaxTickets) {
    // Enough splits that a wave holds at most gw_max groups.  Beyond that,
    // about five splits measured best on MI355X for the 4B-class layer at
    // M = 16 (QKV, O, gate+up and down all within 10% of their best), as long
    // as every wave keeps at least one group.
    splits = (G + 4 * gw_max - 1) / (4 * gw_max);
    const int pref = G / 4 < 5 ? G / 4 : 5;
    if (pref > splits) splits = pref;
    const long target = (long)num_cus / 2;
    while ((long)p.col_tiles * splits < target && G >= 4 * (splits + 1)) ++splits;
  }
  p.splits = splits;
  const int groups_per_block = (G + splits - 1) / splits;
  const int per_wave = (groups_per_block + kWaves - 1) / kWaves;
  p.gw = per_wave < gw_max ? per_wave : gw_max;
  if (p.gw < 1) p.gw = 1;
  if (splits > 1) {
    p.ticket_bytes = kTicketRegion;
    p.partial_bytes = (size_t)p.mblocks * splits * rows_blk * p.col_tiles * kColTile * sizeof(float);
  }
  return p;
}

hipError_t launch_w4a16_skinny(const GemmArgs& a, const GemmPlan& p, void* workspace,
                               hipStream_t stream) {
  unsigned* tickets = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    tickets = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ticket_bytes);
  }
  if (p.mt == 1) {
    switch (p.gw) {
      case 1: launch_t<1, 1>(a, p, tickets, partials, stream); break;
      case 2: launch_t<1, 2>(a, p, tickets, partials, stream); break;
      case 3: launch_t<1, 3>(a, p, tickets, partials, stream); break;
      default: launch_t<1, 4>(a, p, tickets, partials, stream); break;
    }
  } else {
    if (p.gw == 1) launch_t<2, 1>(a, p, tickets, partials, stream);
    else launch_t<2, 2>(a, p, tickets, partials, stream);
  }
  return hipGetLastError();
}

}  // namespace w4v
