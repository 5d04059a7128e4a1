// W4A16 linear for a skinny block of activation rows (the verify block of
// K+1 rows, section 3 of the organisers' results page), gfx950.
//
// Work decomposition
//   block  = WT x WK waves: WT adjacent 64-column tiles x WK k-slices, on
//            one K-split of the quantisation groups (128 k each).  The WT
//            waves of a k-slice walk the same groups, so the activations of a
//            group are loaded once per block and shared through LDS: on
//            MI355X a CU's load throughput is the limit, and activations
//            loaded per wave cost as much of it as the weights themselves.
//   lane l = columns col..col+3 with col = tile*64 + 4*(l % 16), packed row
//            4*it + l/16 of every 4-row quad; one 128-bit load brings 4 words
//            = 4 columns x 8 k, the B operands of 4 MFMAs (one per column).
//   A      = the group's 16 activation rows x 128 k: the k-slice's waves load
//            it row-contiguous (4 rows x 256 bytes per instruction, 4/WT
//            instructions each), reorder each 8-k chunk to the k order of the
//            dequantised nibbles and store it in a double-buffered LDS tile,
//            from which every wave reads the MFMA A layout.  With one tile
//            per block no other wave reads a k-slice's tile, so the step
//            takes no block barrier (a wave's LDS accesses complete in
//            order).  A single activation row (DX) skips LDS: each lane loads
//            its A fragments straight from memory (four distinct 16-byte
//            pieces per instruction, all lanes reading row 0) and reorders
//            them in registers.  Measured per 144-linear step: the barrier
//            dropped for one-tile blocks, 1,173 -> 1,150 us at M = 16; direct
//            fragments at M = 1, 1,081 -> 1,060 us (at M = 16 they touch 16
//            rows per instruction and were slower, 1,179 us).
// Loads run D groups ahead of the math (a ring of register sets; the plans
// use D = 2, which beat 3 at every shape on MI355X: a third slot mostly
// issues empty loads ahead of the first step and holds registers), and every
// load is unconditional (a missing group reads zeros from outside its buffer
// resource), because a load under a branch makes the compiler wait for all
// loads in flight.
// Per group the int4 words become exact fp16 (q - z); four 16x16x32 MFMAs per
// column accumulate X * (q - z) over the group's 128 k in fp32, and the
// group's fp16 scale is applied once to that fp32 sum (exact algebra: the
// scale is constant over the group).  The k-slices of a tile are added in
// fixed order through LDS; with split-K > 1 the blocks of a tile publish fp32
// partials and the last block to arrive adds them in split order, so the
// output does not depend on arrival order.  The hand-off goes through the
// memory side (agent scope: the eight XCDs' L2 caches are not coherent with
// each other) unless all splits of a tile are known to run on one XCD: the
// hardware deals a launch's blocks over the XCDs round-robin by block id, so
// with a multiple of 8 column blocks the splits of a tile (ids equal mod 8)
// share an XCD, and then the partials stay in its L2 (per launch over 36
// weight copies: QKV 6.92 -> 6.75 us, O 6.33 -> 6.06, down 8.33 -> 8.02; the
// ticket atomics are the same instruction either way).
// A probe launch, once per device (the first split call outside stream
// capture), records the offsets (XCC_ID - block id) mod 8 it observes; the
// launcher passes the L2 path in only if that offset was constant.
#include <mutex>
#include <type_traits>

#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

struct Resources {
  rsrc_t w, z, s, x;
};

// One bit per observed (XCC_ID - block id) mod 8 of the probe launch: a single
// bit set means block i runs on XCD (i + c) mod 8 for a constant c.  Read back
// by the host once per device; no kernel reads it.
__device__ unsigned g_xcd_offsets;

__global__ __launch_bounds__(64) void xcd_probe_kernel() {
  if (threadIdx.x == 0) {
    const unsigned x = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 15u;   // HW_REG_XCC_ID[3:0]
    __hip_atomic_fetch_or(&g_xcd_offsets, 1u << ((x - blockIdx.x) & 7u), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  }
}

// LDS tile of one group's activations: 16*MT rows of 128 fp16, padded by 16
// bytes so that 8 lanes reading one 16-byte column hit distinct banks
constexpr int kXRowWords = (kGroup * 2 + 16) / 4;

// One 128-k step holds Q quantisation groups (Q = 1: group size 128; Q = 4:
// group size 32, one per 32-k MFMA slab).
template <int MT, int WT, int Q>
struct Frag {
  static constexpr int kXLoads = 4 * MT / WT;   // activation loads of this wave per step
  u32x4 w[4];            // 4 quads of packed rows, 4 columns each
  uint32_t zw[Q];        // zero-point words holding the lane's 4 columns at bit (l & 1) * 16
  u32x2 s[Q];            // 4 fp16 scales per quantisation group
  u32x4 x[kXLoads];      // this wave's share of the step's activation rows
};

// Byte offsets of one lane's loads for group 0; group g adds g times the
// per-group strides.  A group that does not exist gets 2 GiB added instead,
// which puts every load outside its buffer resource (reads zeros, no memory
// access): no load ever sits under a branch, because a load under a branch
// makes the compiler wait for all loads in flight.
template <int MT, int WT>
struct Lanes {
  uint32_t w, z, s;                     // weights (quad 0), zero-point word, scales
  uint32_t x[4 * MT / WT];              // activation chunks
  uint32_t wq;                          // weight offset step between quads (4 packed rows)
  uint32_t gw;                          // weight stride per 128-k step
  uint32_t gz, gs;                      // zero-point and scale strides per quantisation group
};

// activation load i of the group (i = 0 .. 4*MT-1): rows 4 i + l/16, k = 8 (l % 16) .. + 7
__device__ __forceinline__ int xrow_of(int i, int lane) { return 4 * i + (lane >> 4); }

template <int MT, int WT, int Q>
__device__ __forceinline__ void load_weights(Frag<MT, WT, Q>& f, const Resources& rs,
                                             const Lanes<MT, WT>& o, int g, bool valid) {
  const uint32_t gg = (uint32_t)g;
#pragma unroll
  for (int it = 0; it < 4; ++it)
    f.w[it] = ld_x4<kNT>(rs.w, o.w + it * o.wq + (valid ? gg * o.gw : kNoLoad));
}

// the rest of a group: zero-points, scales, activations (issued after its weights)
template <int MT, int WT, int Q>
__device__ __forceinline__ void load_rest(Frag<MT, WT, Q>& f, const Resources& rs,
                                          const Lanes<MT, WT>& o, int g, bool valid) {
  const uint32_t gg = (uint32_t)g;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    f.zw[q] = ld_x1(rs.z, o.z + (valid ? (gg * Q + q) * o.gz : kNoLoad));
    f.s[q] = ld_x2(rs.s, o.s + (valid ? (gg * Q + q) * o.gs : kNoLoad));
  }
#pragma unroll
  for (int q = 0; q < Frag<MT, WT, Q>::kXLoads; ++q)
    f.x[q] = ld_x4(rs.x, o.x[q] + (valid ? gg * (uint32_t)(kGroup * 2) : kNoLoad));
}

template <int MT, int WT, int Q>
__device__ __forceinline__ void load_group(Frag<MT, WT, Q>& f, const Resources& rs,
                                           const Lanes<MT, WT>& o, int g, bool valid) {
  load_weights<MT, WT, Q>(f, rs, o, g, valid);
  load_rest<MT, WT, Q>(f, rs, o, g, valid);
}

__device__ __forceinline__ void store_row4(_Float16* dst, float a0, float a1, float a2, float a3) {
  const f16x2 lo = {(_Float16)a0, (_Float16)a1};
  const f16x2 hi = {(_Float16)a2, (_Float16)a3};
  const u32x2 v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  *reinterpret_cast<u32x2*>(dst) = v;
}

// SB: split-K partials the last block of a tile loads per batch (one round
// trip to memory per batch; loads past the last split are masked off)
// Everything the first group step needs comes first, as scalars (pointers to
// the weights, scales, zero-points and activations, N, M, the activation row
// stride, the split parameters): the library builds this kernel with those 14
// dwords preloaded into SGPRs, so the prologue's loads issue without waiting
// for argument loads; the rest of GemmArgs is needed only by the epilogue.
template <int MT, int WT, int WK, int D, int SB, int Q, int DX>
__global__ __launch_bounds__(64 * WT * WK) void w4a16_skinny_kernel(
    const uint32_t* pqw, const _Float16* psc, const uint32_t* pqz, const _Float16* px, int pN,
    int pM, int pldx, int splits, int gbase, int grem, GemmArgs a, unsigned* tickets,
    float* partials) {
  static_assert(!DX || (MT == 1 && WT == 1), "direct fragments: one row tile, one tile");
  static_assert(D == 2 || D == 3, "the step loop unrolls rings of two or three groups");
  constexpr int NW = WT * WK;                       // waves per block
  constexpr int kXWords = MT * 16 * kXRowWords;     // one group's activation tile
  const int lane = threadIdx.x & 63;
  // the wave index is the same in every lane: read it into a scalar register,
  // so that the wave's group range, its step count and the load masks derived
  // from them are scalars (a per-lane value put the prologue's zero-point load
  // under an exec-masked branch and every step's test on the vector ALU)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wt = wave % WT, wk = wave / WT;
  const int cb = blockIdx.x;
  const int split = blockIdx.y;
  const int mblk = blockIdx.z;
  const int T = (pN + kColTile - 1) / kColTile;
  const int tile = cb * WT + wt;
  const int kb = lane >> 4, chunk = lane & 15;
  const int mbase = mblk * 16 * MT;

  // groups of this split, then of this k-slice: the first grem splits take
  // gbase + 1 groups, the others gbase (G / splits and G % splits, from the
  // host: a division here would put some fifty dependent instructions in
  // front of the first load)
  const int gs0 = split * gbase + (split < grem ? split : grem);
  const int glen = gbase + (split < grem ? 1 : 0);
  const int g0 = gs0 + glen * wk / WK;
  const int n = gs0 + glen * (wk + 1) / WK - g0;   // groups of this wave
  const int nmax = (glen + WK - 1) / WK;            // steps of the block

  const int col_raw = tile * kColTile + 4 * chunk;
  const bool colok = tile < T && col_raw < pN;      // N % 8 == 0: 4 columns all valid or none
  const int col = colok ? col_raw : pN - 4;         // the column this lane reads

  constexpr int E = MT * 16;                        // accumulator floats per lane
  constexpr int kTileWords = DX ? 0 : 2 * WK * kXWords;   // double-buffered activation tiles
  constexpr int kRedWords = (WK > 1) ? NW * E * 64 : 0;
  __shared__ uint32_t lds[kTileWords > kRedWords ? kTileWords : kRedWords];
  auto xtile = [&](int buf, int slice) { return lds + (buf * WK + slice) * kXWords; };

  // The first group's weights are requested before any other set-up: a
  // freshly launched kernel fetches its instructions from L2, so every
  // instruction ahead of a load delays it.
  Resources rs;
  rs.w = make_rsrc(pqw);
  const uint32_t N = (uint32_t)pN;
  Lanes<MT, WT> o;
  o.w = ((uint32_t)kb * N + col) * 4;
  o.wq = 16 * N;                                    // 4 packed rows
  o.gw = 64 * N;                                    // 16 packed rows
  Frag<MT, WT, Q> f[D];
  auto group_of = [&](int j) { return g0 + (j < n ? j : (n > 0 ? n - 1 : 0)); };
  load_weights<MT, WT, Q>(f[0], rs, o, group_of(0), 0 < n);
  __builtin_amdgcn_sched_barrier(0);

  rs.z = make_rsrc(pqz);
  rs.s = make_rsrc(psc);
  rs.x = make_rsrc(px);
  o.z = (uint32_t)(col >> 3) * 4;
  o.gz = (N >> 3) * 4;
  o.s = (uint32_t)col * 2;
  o.gs = N * 2;
#pragma unroll
  for (int q = 0; q < Frag<MT, WT, Q>::kXLoads; ++q) {
    if constexpr (DX) {
      // A fragment q = it: row l % 16 (row 0 when M = 1), k = 32 it + 8 (l / 16) .. + 7
      int m = mbase + chunk;
      m = m < pM ? m : pM - 1;                      // rows past M: never stored
      o.x[q] = ((uint32_t)m * (uint32_t)pldx + q * 32 + kb * 8) * 2;
    } else {
      int m = mbase + xrow_of(q * WT + wt, lane);
      m = m < pM ? m : pM - 1;                      // rows past M: never stored
      o.x[q] = ((uint32_t)m * (uint32_t)pldx + chunk * 8) * 2;
    }
  }
  // prologue loads in the loop's order (f[0] complete, then f[1], ...): the
  // wait counts at the loop head are then the same on entry and on the back edge
  load_rest<MT, WT, Q>(f[0], rs, o, group_of(0), 0 < n);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 1; i < D; ++i) {
    load_group<MT, WT, Q>(f[i], rs, o, group_of(i), i < n);
    __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t magic = in_vgpr(0x64006400u);
  const int zshift = (lane & 1) * 16;

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step per group: ring slot i (a compile-time index) is computed and
  // then refilled D groups ahead.  The loop body runs whole rounds of D
  // steps with no branch around loads or barriers (a branch there would make
  // the compiler drain the loads at every iteration); the last nmax % D steps
  // follow the loop, where draining costs nothing.  Steps past a wave's own
  // groups (k-slices of unequal length) load nothing and compute nothing but
  // still take the block barrier.
  auto step = [&](auto slot, const int j) __attribute__((always_inline)) {
    constexpr int i = decltype(slot)::value;
    // share the group's activations: this wave's chunks, reordered to the
    // k order of the dequantised nibbles, into the LDS tile (the waves of
    // both tiles of a k-slice read it: a block barrier with two tiles)
    uint32_t* xt = xtile(j & 1, wk);
    if constexpr (!DX) {
#pragma unroll
      for (int q = 0; q < Frag<MT, WT, Q>::kXLoads; ++q)
        *reinterpret_cast<f16x8*>(xt + xrow_of(q * WT + wt, lane) * kXRowWords + chunk * 4) =
            permute_for_int4(f[i].x[q]);
      if constexpr (WT > 1) lds_barrier();
    }
    if (j < n) {                                  // wave-uniform
      // per quantisation group: exact fp16 (q - z) operands, the group's
      // fp32 sum over its 128 / Q k, then its scale once
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        ZeroPair zz[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) zz[c] = zero_pair((f[i].zw[q] >> (zshift + 4 * c)) & 0xFu);
        f32x4 tmp[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int c = 0; c < 4; ++c) tmp[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int it = q * (4 / Q); it < (q + 1) * (4 / Q); ++it) {
          // A layout: row l % 16, k = 32 it + 8 (l / 16) .. + 7
          f16x8 av[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if constexpr (DX)
              av[mt] = permute_for_int4(f[i].x[it]);
            else
              av[mt] = *reinterpret_cast<const f16x8*>(xt + (mt * 16 + chunk) * kXRowWords +
                                                       (it * 4 + kb) * 4);
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f16x8 b = dequant_int4_word(f[i].w[it][c], zz[c], magic);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) tmp[mt][c] = mfma16x16x32(av[mt], b, tmp[mt][c]);
          }
        }
        // copy the vector elements to scalars before the bit casts: a bit
        // cast of an ext-vector element expression reads element 0 with
        // this compiler
        const uint32_t s_lo = f[i].s[q].x, s_hi = f[i].s[q].y;
        const f16x2 s01 = __builtin_bit_cast(f16x2, s_lo);
        const f16x2 s23 = __builtin_bit_cast(f16x2, s_hi);
        const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][c][r] = __builtin_fmaf(sc[c], tmp[mt][c][r], acc[mt][c][r]);
      }
    }
    load_group<MT, WT, Q>(f[i], rs, o, group_of(j + D), j + D < n);
  };
  int j0 = 0;
  for (; j0 + D <= nmax; j0 += D) {
    step(std::integral_constant<int, 0>{}, j0);
    step(std::integral_constant<int, 1>{}, j0 + 1);
    if constexpr (D > 2) step(std::integral_constant<int, 2>{}, j0 + 2);
  }
  if (j0 < nmax) step(std::integral_constant<int, 0>{}, j0);                 // block-uniform
  if constexpr (D > 2) {
    if (j0 + 1 < nmax) step(std::integral_constant<int, 1>{}, j0 + 1);
  }

  // ---- add the k-slices of each tile in fixed order through LDS
  // element e = (mt*4 + r)*4 + c of lane l of wave w sits at red[(w*E + e)*64 + l]
  constexpr int kSlots = MT * 4;                    // (mt, r) row slots of a lane
  constexpr int kMine = (kSlots + WK - 1) / WK;     // row slots this wave finishes (at most)
  float* red = reinterpret_cast<float*>(lds);
  float out[kMine][4];
  if (WK == 1) {
#pragma unroll
    for (int j = 0; j < kMine; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) out[j][c] = acc[j >> 2][c][j & 3];
  } else {
    __syncthreads();                                // LDS tiles no longer read
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[(wave * E + (mt * 4 + r) * 4 + c) * 64 + lane] = acc[mt][c][r];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int mr = j * WK + wk < kSlots ? j * WK + wk : kSlots - 1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v = red[((0 * WT + wt) * E + mr * 4 + c) * 64 + lane];
#pragma unroll
        for (int k = 1; k < WK; ++k) v += red[((k * WT + wt) * E + mr * 4 + c) * 64 + lane];
        out[j][c] = v;
      }
    }
  }
  // row slot j of this wave, or -1 when the k-slices outnumber the slots
  auto slot_of = [&](int j) { return (WK == 1) ? j : (j * WK + wk < kSlots ? j * WK + wk : -1); };
  auto row_of = [&](int mr) { return mbase + (mr >> 2) * 16 + 4 * kb + (mr & 3); };

  if (splits == 1) {
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int mr = slot_of(j);
      const int m = row_of(mr);
      if (mr >= 0 && colok && m < a.M)
        store_row4(a.y + (size_t)m * a.ldy + col, a.alpha * out[j][0], a.alpha * out[j][1],
                   a.alpha * out[j][2], a.alpha * out[j][3]);
    }
    return;
  }

  // ---- split-K: publish this block's partials, the last block of a tile adds them
  // partials layout: [mblk][split][16*MT rows][col_blocks*WT*64 cols]
  const size_t ncols = (size_t)gridDim.x * WT * kColTile;
  const size_t rows_blk = 16 * MT;
  float* pbase = partials + (size_t)mblk * splits * rows_blk * ncols;
  const rsrc_t pr = make_rsrc(pbase);
  const int pcol = tile * kColTile + 4 * chunk;     // column in the partial rows (< ncols)
  // all splits of this tile on one XCD: a multiple of 8 column blocks, and the
  // probe saw a constant block-to-XCD offset
  const bool local = a.xcd_local != 0 && (gridDim.x & 7u) == 0u;
  auto publish = [&](auto aux) __attribute__((always_inline)) {
    constexpr int kAux = decltype(aux)::value;
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int mr = slot_of(j);
      if (mr < 0) continue;
      const int mloc = row_of(mr) - mbase;
      const f32x4 v = {out[j][0], out[j][1], out[j][2], out[j][3]};
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, v), pr,
          (uint32_t)((((size_t)split * rows_blk + mloc) * ncols + pcol) * 4), 0, kAux);
    }
  };
  if (local) publish(std::integral_constant<int, 0>{});     // written through L1 into this XCD's L2
  else publish(std::integral_constant<int, kSC1>{});
  // one ticket per tile of the block, taken after every partial store completed
  __shared__ unsigned s_last[WT];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < WT) {
    const int t = cb * WT + (int)threadIdx.x;
    unsigned last = 0u;
    if (t < T) {                                    // tiles past N take no ticket
      unsigned* tk = tickets + ((size_t)mblk * T + t) * kTicketStride;
      const unsigned prev = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (unsigned)splits - 1) {
        __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = 1u;
      }
    }
    s_last[threadIdx.x] = last;
  }
  __syncthreads();
  if (!s_last[wt]) return;

  // the last block: partials in split order, SB loads in flight per batch
  // (one loop per cache policy, so that no load sits under a branch)
  auto finish = [&](auto aux) __attribute__((always_inline)) {
    constexpr int kAux = decltype(aux)::value;
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int mr = slot_of(j);
      if (mr < 0) continue;
      const int m = row_of(mr);
      const int mloc = m - mbase;
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      for (int sp0 = 0; sp0 < splits; sp0 += SB) {
        u32x4 v[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u)
          v[u] = __builtin_amdgcn_raw_buffer_load_b128(
              pr,
              sp0 + u < splits ? (uint32_t)((((size_t)(sp0 + u) * rows_blk + mloc) * ncols + pcol) * 4)
                               : kNoLoad,
              0, kAux);
#pragma unroll
        for (int u = 0; u < SB; ++u)
          if (sp0 + u < splits) sum += __builtin_bit_cast(f32x4, v[u]);
      }
      if (colok && m < a.M)
        store_row4(a.y + (size_t)m * a.ldy + col, a.alpha * sum[0], a.alpha * sum[1],
                   a.alpha * sum[2], a.alpha * sum[3]);
    }
  };
  if (local) finish(std::integral_constant<int, kSC0>{});
  else finish(std::integral_constant<int, kSC1>{});
}

template <int MT, int WT, int WK, int D, int SB, int Q, int DX>
void launch_t(const GemmArgs& a, const GemmPlan& p, unsigned* tickets, float* partials,
              hipStream_t stream) {
  const int G = a.K / kGroup;
  hipLaunchKernelGGL((w4a16_skinny_kernel<MT, WT, WK, D, SB, Q, DX>),
                     dim3(p.col_blocks, p.splits, p.mblocks), dim3(64 * WT * WK), 0, stream,
                     a.qweight, a.scales, a.qzeros, a.x, a.N, a.M, (int)a.ldx, p.splits,
                     G / p.splits, G % p.splits, a, tickets, partials);
}

// Four k-slices per block, one or two tiles, two groups in flight per wave;
// one batch of partial loads up to 8 splits, batches of 16 beyond.
template <int MT, int WT, int Q, int DX>
void launch_w(const GemmArgs& a, const GemmPlan& p, unsigned* tickets, float* partials,
              hipStream_t stream) {
  if (p.splits <= 8) launch_t<MT, WT, 4, 2, 8, Q, DX>(a, p, tickets, partials, stream);
  else launch_t<MT, WT, 4, 2, 16, Q, DX>(a, p, tickets, partials, stream);
}

// a single activation row on one-tile blocks takes its A fragments directly
template <int MT, int Q>
void launch_q(const GemmArgs& a, const GemmPlan& p, unsigned* tickets, float* partials,
              hipStream_t stream) {
  if (p.wt == 1) {
    if constexpr (MT == 1) {
      if (a.M == 1) {
        launch_w<1, 1, Q, 1>(a, p, tickets, partials, stream);
        return;
      }
    }
    launch_w<MT, 1, Q, 0>(a, p, tickets, partials, stream);
  } else {
    launch_w<MT, 2, Q, 0>(a, p, tickets, partials, stream);
  }
}

}  // namespace

GemmPlan plan_w4a16(int M, int N, int K, int num_cus) {
  GemmPlan p{};
  p.mt = (M <= 16) ? 1 : 2;
  const int rows_blk = 16 * p.mt;
  p.mblocks = (M + rows_blk - 1) / rows_blk;
  p.tiles = (N + kColTile - 1) / kColTile;
  const int G = K / kGroup;
  // Four k-slices per block (added through LDS); one or two 64-column tiles
  // per block, and a split-K factor, chosen to minimise the steps of the
  // longest wave times its rounds (blocks per CU, times waves per SIMD within a
  // block), one tile and the fewest splits on ties.  Measured on MI355X for the
  // 4B-class verify shapes:
  //   - 16-row blocks: one tile, at most two blocks per CU once split (QKV 5
  //     splits, O 4, down 5);
  //   - 32-row blocks (the group-32 target at M = 24): at most one block per
  //     CU, and two tiles may share a block, so that a tile pair shares its
  //     twice-as-large activation tile (QKV 12.7 -> 10.3 us with two tiles x
  //     5 splits);
  //   - tiles outnumbering the CUs (gate+up, 304 tiles): two tiles per block
  //     and no split (15.2 us at 3 splits against 10.8 us unsplit).
  p.wk = 4;
  const bool wide = (long)p.tiles * p.mblocks > num_cus;
  const long max_blocks = (p.mt == 1 ? 2L : 1L) * num_cus;
  const int smax = (!wide && (size_t)p.tiles * p.mblocks <= kMaxTickets) ? G : 1;
  int splits = 1;
  long best = -1;
  for (int wt = 1; wt <= 2; ++wt) {
    if ((wt == 1 && wide) || (wt == 2 && !wide && p.mt == 1)) continue;
    const int cb = (p.tiles + wt - 1) / wt;
    const size_t part_per_split =
        (size_t)p.mblocks * rows_blk * cb * wt * kColTile * sizeof(float);
    for (int s = 1; s <= smax; ++s) {
      const long blocks = (long)cb * p.mblocks * s;
      if (s > 1 && (blocks > max_blocks || part_per_split * s > kPartialRegion)) break;
      const long steps = ((G + s - 1) / s + p.wk - 1) / p.wk;   // of the longest wave
      const long rounds = ((blocks + num_cus - 1) / num_cus) * ((wt * p.wk + 3) / 4);
      const long cost = steps * rounds;
      if (best < 0 || cost < best) {
        best = cost;
        splits = s;
        p.wt = wt;
      }
    }
  }
  // two groups in flight per wave: against three, on MI355X at M = 16 per
  // launch QKV 6.77 -> 6.10 us, O 6.03 -> 5.69, down 8.07 -> 7.34, gate+up
  // 11.15 -> 10.65, and the 144 linears at M = 1 1,061 -> 1,012 us (deeper
  // rings were slower still; two k-slices per block instead of four were
  // slower at every shape with two groups in flight)
  p.depth = 2;
  p.col_blocks = (p.tiles + p.wt - 1) / p.wt;
  p.splits = splits;
  if (splits > 1) {
    p.ticket_bytes = kTicketRegion;
    p.partial_bytes = (size_t)p.mblocks * rows_blk * p.col_blocks * p.wt * kColTile *
                      sizeof(float) * splits;
  }
  return p;
}

namespace {
std::mutex g_probe_mu;
// per device: 0 not probed, 1 probe in flight, 2 round-robin placement, 3 not
// (or the probe could not run)
int g_xcd_state[64];
hipEvent_t g_xcd_event[64];
unsigned* g_xcd_host[64];    // pinned word the probe's result is copied to
}  // namespace

// Whether blocks with ids equal mod 8 share an XCD on the current device.  The
// first call outside stream capture enqueues the probe, a copy of its result
// to pinned host memory and an event on `stream`, and never waits for them; a
// later call outside capture that finds the event complete reads the result.
// Until then, and under capture, the answer is no (the memory-side hand-off,
// same result bits).  may_probe = false (callers that must not allocate: the
// probe's host word is pinned memory) only reads a result another call started.
static bool xcd_round_robin(hipStream_t stream, bool may_probe) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  std::lock_guard<std::mutex> lock(g_probe_mu);
  int& st = g_xcd_state[dev];
  if (st == 0 && !may_probe) return false;
  if (st == 0 || st == 1) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
      return false;
  }
  if (st == 0) {
    void* sym = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&g_xcd_host[dev]), sizeof(unsigned),
                      hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&g_xcd_event[dev], hipEventDisableTiming) != hipSuccess ||
        hipGetSymbolAddress(&sym, HIP_SYMBOL(g_xcd_offsets)) != hipSuccess) {
      st = 3;
      return false;
    }
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(256), dim3(64), 0, stream);
    if (hipGetLastError() != hipSuccess ||
        hipMemcpyAsync(g_xcd_host[dev], sym, sizeof(unsigned), hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipEventRecord(g_xcd_event[dev], stream) != hipSuccess) {
      st = 3;
      return false;
    }
    st = 1;
    return false;
  }
  if (st == 1) {
    const hipError_t q = hipEventQuery(g_xcd_event[dev]);
    if (q == hipErrorNotReady) return false;
    if (q != hipSuccess) {
      st = 3;
      return false;
    }
    const unsigned mask = *g_xcd_host[dev];
    st = (mask != 0u && (mask & (mask - 1u)) == 0u) ? 2 : 3;
  }
  return st == 2;
}

hipError_t launch_w4a16_skinny(const GemmArgs& a, const GemmPlan& p, void* workspace,
                               hipStream_t stream, bool may_probe) {
  unsigned* tickets = nullptr;
  float* partials = nullptr;
  GemmArgs la = a;
  la.xcd_local = 0;
  if (p.splits > 1) {
    la.xcd_local = xcd_round_robin(stream, may_probe) ? 1 : 0;
    tickets = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ticket_bytes);
  }
  if ((p.wt != 1 && p.wt != 2) || p.wk != 4 || p.depth != 2 ||
      (a.group_size != 128 && a.group_size != 32))
    return hipErrorInvalidValue;
  const bool g32 = a.group_size == 32;
  if (p.mt == 1) {
    if (g32) launch_q<1, 4>(la, p, tickets, partials, stream);
    else launch_q<1, 1>(la, p, tickets, partials, stream);
  } else {
    if (g32) launch_q<2, 4>(la, p, tickets, partials, stream);
    else launch_q<2, 1>(la, p, tickets, partials, stream);
  }
  return hipGetLastError();
}

}  // namespace w4v
