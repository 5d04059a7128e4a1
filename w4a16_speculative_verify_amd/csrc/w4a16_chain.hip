// A chain of W4A16 linears (the target's layers during one verify pass,
// section 3 of the organisers' results page) in ONE persistent launch, gfx950.
//
// Why one launch: at M <= 16 rows a linear moves 5-27 MB, 1-4 us of HBM time,
// while a launch in a graph costs about 2.5 us on its own and every linear
// also pays the ramp of a new grid and its split-K tail.  Here one block per
// CU stays resident for all linears, the weights of the block's next unit are
// requested before it waits for the previous linear to finish, and linears
// are separated by a grid barrier instead of a kernel boundary.
//
// Work units.  Linear l is cut into cb column blocks of 4 tiles (256
// columns) and S K-splits, cb * S <= blocks, and block b owns unit b of every
// linear (a block with no unit in a linear only prefetches and waits).
//
// A unit, 8 waves = 4 tiles x 2 k-slices:
//   1. after the barrier, the unit's activation slice (16 rows x the split's
//      groups) is loaded once, reordered to the nibble k order and stored in
//      LDS, where all 8 waves read their MFMA A operands;
//   2. each wave streams the packed weights of its tile and k-slice through a
//      ring of 3 groups in flight (masked buffer loads, no branch around
//      them), dequantises exactly and runs 16x16x32 MFMAs, the group scale
//      applied once per group to the fp32 sum;
//   3. the two k-slices of a tile are added through LDS; with one split the
//      block writes the tile's fp16 output, otherwise it publishes an fp32
//      partial and the last split to arrive (one ticket per tile) adds the
//      partials in split order and writes the output.
// Intermediate outputs go to buffers of the workspace with agent-scope (sc1)
// stores; each linear writes a buffer of its own that nothing read earlier
// in the launch, so the next linear may read it through the L2.
// Grid barrier: after its stores have completed, a block adds itself to the
// arrival counter of its group (16 groups); the last of a group re-arms that
// counter and adds the group to the counter of finished groups; the last
// group re-arms that one and writes the new generation to 16 copies, each
// polled by one group's blocks with agent-scope loads.  Every counter and
// copy has a 256-byte slot of its own: atomics and polls on one cache line
// serialise at the memory side, which made a single-counter barrier take
// several microseconds.  A poll that exceeds its bound sets the error and
// abort words; every poller also watches its abort copy, so all blocks leave
// instead of hanging.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int WT = kChainTiles;
constexpr int WK = kChainSlices;
constexpr int kWaves = WT * WK;
constexpr int kThreads = kChainThreads;
constexpr int D = 3;                                // groups in flight per wave
constexpr unsigned kSpinLimit = 1u << 20;
// LDS row of one group's activations: 128 fp16 + 16 bytes of padding (8 lanes
// reading one 16-byte column hit distinct banks)
constexpr int kXRowWords = (kGroup * 2 + 16) / 4;
constexpr int kXGroupWords = 16 * kXRowWords;
constexpr int kXWords = kChainMaxGroups * kXGroupWords;
constexpr int kRedWords = kWaves * 16 * 64;         // one fp32 accumulator set per wave
constexpr int kLdsWords = kXWords > kRedWords ? kXWords : kRedWords;

struct WFrag {
  u32x4 w[4];        // 4 quads of packed rows, 4 columns each
  uint32_t zw;       // zero-point word holding the lane's 4 columns at bit (l & 1) * 16
  u32x2 s;           // 4 fp16 scales
};

// One unit as a block sees it.
struct UnitPlan {
  bool valid;
  int cb, split, gs0, glen;       // column block, split, its groups
  int g0, n;                      // this wave's groups (k-slice)
  int col;                        // the column this lane reads (clamped below N)
  bool colok;
  uint32_t ow, oz, os;            // lane byte offsets for group 0
  uint32_t gw, gz, gs;            // per-group strides
};

__device__ __forceinline__ UnitPlan plan_unit(const ChainLinear& L, int b, int wt, int wk, int lane) {
  UnitPlan u{};
  u.valid = b < L.units;
  const int bb = u.valid ? b : 0;
  u.cb = bb / L.splits;
  u.split = bb - u.cb * L.splits;
  const int G = L.K / kGroup;
  u.gs0 = (int)((unsigned)(G * u.split) / (unsigned)L.splits);
  u.glen = (int)((unsigned)(G * (u.split + 1)) / (unsigned)L.splits) - u.gs0;
  u.g0 = u.gs0 + u.glen * wk / WK;
  u.n = u.gs0 + u.glen * (wk + 1) / WK - u.g0;
  if (!u.valid) u.n = 0;
  const int T = (L.N + kColTile - 1) / kColTile;
  const int tile = u.cb * WT + wt;
  const int col_raw = tile * kColTile + 4 * (lane & 15);
  u.colok = u.valid && tile < T && col_raw < L.N;
  u.col = u.colok ? col_raw : L.N - 4;
  const uint32_t N = (uint32_t)L.N;
  u.ow = ((uint32_t)(lane >> 4) * N + u.col) * 4;
  u.gw = 64 * N;
  u.oz = (uint32_t)(u.col >> 3) * 4;
  u.gz = (N >> 3) * 4;
  u.os = (uint32_t)u.col * 2;
  u.gs = N * 2;
  return u;
}

// Weights, zero-points and scales of local group j of the wave (masked past n).
__device__ __forceinline__ void load_w(WFrag& f, const rsrc_t& rw, const rsrc_t& rz,
                                       const rsrc_t& rs, const UnitPlan& u, int j) {
  const uint32_t g = (uint32_t)(u.g0 + (j < u.n ? j : 0));
  const uint32_t skip = j < u.n ? 0u : kNoLoad;
#pragma unroll
  for (int it = 0; it < 4; ++it)
    f.w[it] = ld_x4<kNT>(rw, (u.ow + it * (u.gw >> 2) + g * u.gw) | skip);
  f.zw = ld_x1(rz, (u.oz + g * u.gz) | skip);
  f.s = ld_x2(rs, (u.os + g * u.gs) | skip);
}

__device__ __forceinline__ void st_agent_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__global__ __launch_bounds__(kThreads) void w4a16_chain_kernel(ChainHeader* hdr,
                                                               const _Float16* __restrict__ x,
                                                               int64_t ldx, _Float16* y,
                                                               int64_t ldy, int M_arg, int K0,
                                                               int N_last) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wt = wave % WT, wk = wave / WT;
  const int kb = lane >> 4, chunk = lane & 15;
  const int b = blockIdx.x;

  // a workspace that was not prepared for this call: report and touch nothing else
  if (hdr->magic != kChainMagic || (int)hdr->M != M_arg || (int)hdr->K0 != K0 ||
      (int)hdr->N_last != N_last || hdr->blocks != gridDim.x || hdr->abort != 0u) {
    if (threadIdx.x == 0 && b == 0) st_agent_u32(&hdr->error, 2u);
    return;
  }
  const ChainLinear* lins =
      reinterpret_cast<const ChainLinear*>(reinterpret_cast<const char*>(hdr) + hdr->lin_offset);
  const int nlin = (int)hdr->n_linears;
  const int M = (int)hdr->M;
  const unsigned nblk = gridDim.x;

  __shared__ uint32_t lds[kLdsWords];
  __shared__ unsigned s_flag[WT + 1];
  __shared__ unsigned s_gen0;
  // barrier slots: group counters, finished-group counter, generation copies
  char* const bar = reinterpret_cast<char*>(hdr) + sizeof(ChainHeader);
  auto slot = [&](int i) { return reinterpret_cast<unsigned*>(bar + (size_t)i * kChainSlot); };
  const int ngroups = (int)nblk < kChainBarGroups ? (int)nblk : kChainBarGroups;
  const int grp = b % kChainBarGroups;
  unsigned* const my_gen = slot(kChainBarGroups + 1 + grp);
  if (threadIdx.x == 0) {
    s_gen0 = __hip_atomic_load(my_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[WT] = 0u;
  }
  __syncthreads();
  const unsigned gen0 = s_gen0;

  const uint32_t magic = in_vgpr(0x64006400u);
  const int zshift = (lane & 1) * 16;

  // weights of linear 0 in flight before anything else
  ChainLinear L = lins[0];
  UnitPlan u = plan_unit(L, b, wt, wk, lane);
  rsrc_t rw = make_rsrc(L.qweight), rz = make_rsrc(L.qzeros), rs = make_rsrc(L.scales);
  WFrag f[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    load_w(f[i], rw, rz, rs, u, i);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int l = 0; l < nlin; ++l) {
    const _Float16* xin = l == 0 ? x : lins[l - 1].out;
    const int64_t ldin = l == 0 ? ldx : lins[l - 1].ldo;
    const bool last_lin = l == nlin - 1;

    // ---- wait for linear l-1 (grid barrier l-1), unless this block released it
    if (l > 0) {
      if (threadIdx.x == 0 && s_flag[WT] == 0u) {
        const unsigned target = gen0 + (unsigned)l;
        const rsrc_t rh = make_rsrc(my_gen);
        unsigned spins = 0;
        while (true) {
          const u32x2 g = __builtin_amdgcn_raw_buffer_load_b64(rh, 0, 0, kSC1);   // generation, abort
          if (g.x == target) break;
          if (g.y != 0u) { s_flag[WT] = 2u; break; }
          if (++spins > kSpinLimit) {
            st_agent_u32(&hdr->error, 1u);
            st_agent_u32(&hdr->abort, 1u);
            for (int c = 0; c < kChainBarGroups; ++c) st_agent_u32(slot(kChainBarGroups + 1 + c) + 1, 1u);
            s_flag[WT] = 2u;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      lds_barrier();
      if (s_flag[WT] == 2u) return;                 // a wait gave up somewhere: leave
    }

    if (u.valid) {
      // ---- the unit's activation slice into LDS: rows x groups x 16 chunks of 8 k
      {
        const rsrc_t rx = make_rsrc(xin);
        const int nchunks = 16 * u.glen * 16;
        constexpr int kMaxPer = kChainMaxGroups * 256 / kThreads;
        u32x4 v[kMaxPer];
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
          const int c = (int)threadIdx.x + i * kThreads;
          const int gl = c >> 8, row = (c >> 4) & 15, ch = c & 15;
          const int m = row < M ? row : M - 1;
          const uint32_t off = ((uint32_t)m * (uint32_t)ldin + (u.gs0 + gl) * kGroup + ch * 8) * 2;
          v[i] = ld_x4(rx, c < nchunks ? off : kNoLoad);
        }
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
          const int c = (int)threadIdx.x + i * kThreads;
          if (c < nchunks) {
            const int gl = c >> 8, row = (c >> 4) & 15, ch = c & 15;
            *reinterpret_cast<f16x8*>(lds + gl * kXGroupWords + row * kXRowWords + ch * 4) =
                permute_for_int4(v[i]);
          }
        }
      }
      lds_barrier();

      // ---- this wave's groups: weights through the ring, activations from LDS
      f32x4 acc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int nsteps = (u.n + D - 1) / D * D;
      for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int j = j0 + i;
          if (j < u.n) {
            const uint32_t* xt = lds + (u.g0 - u.gs0 + j) * kXGroupWords;
            ZeroPair zz[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) zz[c] = zero_pair((f[i].zw >> (zshift + 4 * c)) & 0xFu);
            f32x4 tmp[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) tmp[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < 4; ++it) {
              const f16x8 av = *reinterpret_cast<const f16x8*>(xt + chunk * kXRowWords + (it * 4 + kb) * 4);
#pragma unroll
              for (int c = 0; c < 4; ++c)
                tmp[c] = mfma16x16x32(av, dequant_int4_word(f[i].w[it][c], zz[c], magic), tmp[c]);
            }
            // copy the vector elements to scalars before the bit casts: a bit
            // cast of an ext-vector element expression reads element 0 with
            // this compiler
            const uint32_t s_lo = f[i].s.x, s_hi = f[i].s.y;
            const f16x2 s01 = __builtin_bit_cast(f16x2, s_lo);
            const f16x2 s23 = __builtin_bit_cast(f16x2, s_hi);
            const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[c][r] = __builtin_fmaf(sc[c], tmp[c][r], acc[c][r]);
          }
          load_w(f[i], rw, rz, rs, u, j + D);
        }
      }

      // ---- the two k-slices of each tile, in fixed order through LDS
      float* red = reinterpret_cast<float*>(lds);
      lds_barrier();                                // activation slice no longer read
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[(wave * 16 + r * 4 + c) * 64 + lane] = acc[c][r];
      lds_barrier();
      // wave (wt, wk) finishes rows r = 2 j + wk (j = 0, 1) of its tile: 4 kb + r
      float out[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 2 * j + wk;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float v = red[((0 * WT + wt) * 16 + r * 4 + c) * 64 + lane];
#pragma unroll
          for (int k = 1; k < WK; ++k) v += red[((k * WT + wt) * 16 + r * 4 + c) * 64 + lane];
          out[j][c] = v;
        }
      }
      _Float16* dst = last_lin ? y : L.out;
      const int64_t ldd = last_lin ? ldy : L.ldo;
      const rsrc_t rd = make_rsrc(dst);
      auto store_out = [&](int m, float a0, float a1, float a2, float a3) {
        const u32x2 v = {pack_f16x2(L.alpha * a0, L.alpha * a1), pack_f16x2(L.alpha * a2, L.alpha * a3)};
        const uint32_t off = (uint32_t)(((size_t)m * ldd + u.col) * 2);
        if (last_lin) __builtin_amdgcn_raw_buffer_store_b64(v, rd, off, 0, 0);
        else st_agent_x2(rd, off, v);
      };
      if (L.splits == 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int m = 4 * kb + 2 * j + wk;
          if (u.colok && m < M) store_out(m, out[j][0], out[j][1], out[j][2], out[j][3]);
        }
      } else {
        // partials [split][16 rows][cb * 4 * 64 columns]
        const size_t ncols = (size_t)L.cb * WT * kColTile;
        const rsrc_t pr = make_rsrc(L.partials);
        const int pcol = (u.cb * WT + wt) * kColTile + 4 * chunk;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int m = 4 * kb + 2 * j + wk;
          const f32x4 v = {out[j][0], out[j][1], out[j][2], out[j][3]};
          st_agent_x4(pr, (uint32_t)((((size_t)u.split * 16 + m) * ncols + pcol) * 4),
                      __builtin_bit_cast(u32x4, v));
        }
        __builtin_amdgcn_s_waitcnt(0);              // this thread's partial stores are complete
        lds_barrier();
        if (threadIdx.x < WT) {
          const int t = u.cb * WT + (int)threadIdx.x;
          const int T = (L.N + kColTile - 1) / kColTile;
          unsigned last = 0u;
          if (t < T) {
            unsigned* tk = L.tickets + (size_t)t * (kChainSlot / sizeof(unsigned));
            const unsigned prev =
                __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (prev == (unsigned)L.splits - 1) {
              __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              last = 1u;
            }
          }
          s_flag[threadIdx.x] = last;
        }
        lds_barrier();
        if (s_flag[wt]) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int m = 4 * kb + 2 * j + wk;
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
            for (int sp0 = 0; sp0 < L.splits; sp0 += 8) {
              u32x4 v[8];
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const int sp = sp0 + q < L.splits ? sp0 + q : L.splits - 1;
                v[q] = ld_agent_x4(pr, (uint32_t)((((size_t)sp * 16 + m) * ncols + pcol) * 4));
              }
#pragma unroll
              for (int q = 0; q < 8; ++q)
                if (sp0 + q < L.splits) sum += __builtin_bit_cast(f32x4, v[q]);
            }
            if (u.colok && m < M) store_out(m, sum[0], sum[1], sum[2], sum[3]);
          }
        }
      }
    }
    if (last_lin) break;

    // ---- arrive at barrier l once every store of the block has completed,
    //      then request the next linear's weights while waiting
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (wave == 0) {
      unsigned released = 0u;
      if (lane == 0) {
        const unsigned gsize = (nblk - (unsigned)grp + kChainBarGroups - 1) / kChainBarGroups;
        const unsigned prev =
            __hip_atomic_fetch_add(slot(grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gsize - 1) {
          st_agent_u32(slot(grp), 0u);
          __builtin_amdgcn_s_waitcnt(0);            // re-armed before the group counts as done
          const unsigned done = __hip_atomic_fetch_add(slot(kChainBarGroups), 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
          if (done == (unsigned)ngroups - 1) {
            st_agent_u32(slot(kChainBarGroups), 0u);
            __builtin_amdgcn_s_waitcnt(0);          // re-armed before anyone is released
            released = 1u;
          }
        }
        s_flag[WT] = released;
      }
      released = __shfl(released, 0, 64);
      if (released && lane < kChainBarGroups)
        st_agent_u32(slot(kChainBarGroups + 1 + lane), gen0 + (unsigned)l + 1u);
    }
    L = lins[l + 1];
    u = plan_unit(L, b, wt, wk, lane);
    rw = make_rsrc(L.qweight);
    rz = make_rsrc(L.qzeros);
    rs = make_rsrc(L.scales);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      load_w(f[i], rw, rz, rs, u, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace

hipError_t launch_w4a16_chain(ChainHeader* hdr, const _Float16* x, int64_t ldx, _Float16* y,
                              int64_t ldy, int M, int K0, int N_last, int blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(w4a16_chain_kernel, dim3(blocks), dim3(kThreads), 0, stream, hdr, x, ldx, y,
                     ldy, M, K0, N_last);
  return hipGetLastError();
}

}  // namespace w4v
