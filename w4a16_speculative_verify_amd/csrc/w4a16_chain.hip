// A chain of W4A16 linears (the target's layers during one verify pass,
// section 3 of the organisers' results page) in ONE persistent launch, gfx950.
//
// Why one launch: at M <= 16 rows a linear moves 5-27 MB, 1-4 us of HBM time,
// while a launch in a graph costs about 2.5 us on its own and every linear
// also pays the ramp of a new grid and its split-K tail: 144 launches cannot
// come near the HBM bound.  Here one block per CU stays resident for all
// linears and starts streaming its next unit's weights while the current
// unit is reduced and published.
//
// Work units.  Linear l is cut into cb column blocks of wt 64-column tiles
// (wt = 1, 2 or 4, chosen per linear) and S K-splits, cb * S <= blocks, and
// block b owns unit b of every linear (a block with no unit in a linear
// skips it).
//
// Ordering.  Every dependent step between blocks costs a memory round trip of
// a microsecond or more, so the chain keeps them few:
//   outputs   the block that completes an output tile raises the tile's ready
//             flag (epoch + 1) once its stores have landed; a reader waits for
//             the flags of the tiles its activation slice spans, then reads
//             the slice with plain loads (nothing read it earlier in the
//             launch, so no cache holds a stale copy);
//   partials  each split stores its fp32 partial, waits for the stores to
//             land and takes the tile's ticket (agent-scope atomic); the
//             split that arrives last adds the partials in split order,
//             writes the output and raises the flag, and re-arms the ticket.
// Flags hold the epoch, which advances at the end of every launch, so they
// never need clearing.
//
// Roles in a block (5 waves).  A wave's memory counter is in order: waiting
// for one load waits for every load the wave issued before it.  So waves that
// stream weights never poll, and a control wave does every latency-bound step:
//   4 compute waves = wt tiles x (4 / wt) k-slices: load the unit's activation
//                     slice into LDS (reordered to the nibble k order) once
//                     the control wave saw its flags, stream packed weights
//                     through a ring of masked buffer loads, dequantise
//                     exactly, run 16x16x32 MFMAs (group scale once per group
//                     on the fp32 sum), hand the sums over in LDS and request
//                     the next unit's first groups right away;
//   control wave    = waits for the ready flags of the unit's input tiles,
//                     adds the k-slices and writes the output tile and its
//                     flag, or the fp32 split partial and, when it arrives
//                     last, the reduced output and its flag.
// Hand-offs inside a block go through LDS counters, so the control wave's
// waits never hold up the weight stream.  A poll that exceeds its bound sets
// the error and abort words; pollers also watch the abort word, so all blocks
// leave instead of hanging.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kCW = kChainComputeWaves;
constexpr int kThreads = kChainThreads;
constexpr int kComputeThreads = 64 * kCW;
constexpr int D = 3;                                // groups in flight per compute wave
constexpr unsigned kSpinLimit = 1u << 20;
constexpr uint32_t kSlotWords = kChainSlot / sizeof(unsigned);
// LDS row of one group's activations: 128 fp16 + 16 bytes of padding (8 lanes
// reading one 16-byte column hit distinct banks)
constexpr int kXRowWords = (kGroup * 2 + 16) / 4;
constexpr int kXGroupWords = 16 * kXRowWords;
constexpr int kXWords = kChainMaxGroups * kXGroupWords;
constexpr int kXPer = kChainMaxGroups * 256 / kComputeThreads;   // slice chunks per thread
static_assert(kChainMaxGroups * 256 % kComputeThreads == 0, "slice chunks split evenly");
static_assert(kXPer <= 32, "pending mask is 32 bits");
constexpr int kRedWords = kCW * 16 * 64;            // one fp32 accumulator set per compute wave

struct WFrag {
  u32x4 w[4];        // 4 quads of packed rows, 4 columns each
  uint32_t zw;       // zero-point word holding the lane's 4 columns at bit (l & 1) * 16
  u32x2 s;           // 4 fp16 scales
};

// The unit of block b in linear L as compute wave w sees it.
struct UnitPlan {
  bool valid;
  int wt, wk;                     // tiles per block, k-slices per block
  int ti, ki;                     // this wave's tile and k-slice
  int cb, split, gs0, glen;       // column block, split, its groups
  int g0, n;                      // this wave's groups
  int col;                        // the column this lane reads (clamped below N)
  uint32_t ow, oz, os;            // lane byte offsets for group 0
  uint32_t gw, gz, gs;            // per-group strides
};

__device__ __forceinline__ UnitPlan plan_unit(const ChainLinear& L, int b, int w, int lane,
                                              bool exists) {
  UnitPlan u{};
  u.valid = exists && b < L.units;
  u.wt = L.wt;
  u.wk = kCW / L.wt;
  u.ti = w % u.wt;
  u.ki = w / u.wt;
  const int bb = u.valid ? b : 0;
  u.cb = bb / L.splits;
  u.split = bb - u.cb * L.splits;
  const int G = L.K / kGroup;
  u.gs0 = (int)((unsigned)(G * u.split) / (unsigned)L.splits);
  u.glen = (int)((unsigned)(G * (u.split + 1)) / (unsigned)L.splits) - u.gs0;
  u.g0 = u.gs0 + u.glen * u.ki / u.wk;
  u.n = u.valid ? u.gs0 + u.glen * (u.ki + 1) / u.wk - u.g0 : 0;
  const int T = (L.N + kColTile - 1) / kColTile;
  const int tile = u.cb * u.wt + u.ti;
  const int col_raw = tile * kColTile + 4 * (lane & 15);
  u.col = (u.valid && tile < T && col_raw < L.N) ? col_raw : L.N - 4;
  const uint32_t N = (uint32_t)L.N;
  u.ow = ((uint32_t)(lane >> 4) * N + u.col) * 4;
  u.gw = 64 * N;
  u.oz = (uint32_t)(u.col >> 3) * 4;
  u.gz = (N >> 3) * 4;
  u.os = (uint32_t)u.col * 2;
  u.gs = N * 2;
  return u;
}

struct WRsrc {
  rsrc_t w, z, s;
};
__device__ __forceinline__ WRsrc weight_rsrc(const ChainLinear& L) {
  return WRsrc{make_rsrc(L.qweight), make_rsrc(L.qzeros), make_rsrc(L.scales)};
}

// Weights, zero-points and scales of local group j of the wave (masked past n).
__device__ __forceinline__ void load_w(WFrag& f, const WRsrc& r, const UnitPlan& u, int j) {
  const uint32_t g = (uint32_t)(u.g0 + (j < u.n ? j : 0));
  const uint32_t skip = j < u.n ? 0u : kNoLoad;
#pragma unroll
  for (int it = 0; it < 4; ++it)
    f.w[it] = ld_x4<kNT>(r.w, (u.ow + it * (u.gw >> 2) + g * u.gw) | skip);
  f.zw = ld_x1(r.z, (u.oz + g * u.gz) | skip);
  f.s = ld_x2(r.s, (u.os + g * u.gs) | skip);
}

__device__ __forceinline__ void st_agent_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent_u32(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A descriptor read with scalar loads (constant address space): the values
// land in scalar registers, and the wait for them counts against the scalar
// counter, not behind the wave's outstanding weight loads.  Descriptors are
// written before the launch and never changed by it.
typedef __attribute__((address_space(4))) const uint32_t* const_u32_ptr;
__device__ __forceinline__ ChainLinear load_linear(const ChainLinear* p) {
  constexpr int kWords = sizeof(ChainLinear) / 4;
  const_u32_ptr src = (const_u32_ptr)(p);
  uint32_t w[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) w[i] = src[i];
  ChainLinear d;
  __builtin_memcpy(&d, w, sizeof(d));
  return d;
}
__device__ __forceinline__ uint32_t uniform_u32(const unsigned* p) {
  return __builtin_amdgcn_readfirstlane(*p);
}

// ---- hand-offs inside the block: monotone LDS counters
__device__ __forceinline__ unsigned lds_load(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Counts this wave in at *p after its LDS writes so far.
__device__ __forceinline__ void lds_signal(unsigned* p, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if (lane == 0) __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Waits until *p reaches target; false once the block gives up (abort word).
__device__ __forceinline__ bool lds_wait(const unsigned* p, unsigned target, const unsigned* abort) {
  while (__builtin_amdgcn_readfirstlane(lds_load(p)) < target) {
    if (__builtin_amdgcn_readfirstlane(lds_load(abort))) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return true;
}

// A poll that gave up: report it and make every poller leave.
__device__ __forceinline__ void give_up(ChainHeader* hdr, unsigned* s_abort, int lane) {
  if (lane == 0) {
    st_agent_u32(&hdr->error, 1u);
    st_agent_u32(&hdr->abort, 1u);
    __hip_atomic_store(s_abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}
__device__ __forceinline__ void leave(unsigned* s_abort, int lane) {
  if (lane == 0) __hip_atomic_store(s_abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}
// Sum of the WK k-slices of tile ti for this lane, in k-slice order.  The
// slice count is a template argument so that every LDS read is issued before
// the first add waits on one.
template <int WK>
__device__ __forceinline__ void sum_slices(const float* red, int wt, int ti, int lane, float out[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) out[e] = red[(ti * 16 + e) * 64 + lane];
#pragma unroll
  for (int k = 1; k < WK; ++k) {
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = red[((k * wt + ti) * 16 + e) * 64 + lane];
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] += v[e];
  }
}

// Bounded wait between polls: false (after reporting) once the spin bound is
// passed or another block gave up.
__device__ __forceinline__ bool poll_again(unsigned& spins, ChainHeader* hdr, unsigned* s_abort,
                                           int lane) {
  if (++spins > kSpinLimit) {
    give_up(hdr, s_abort, lane);
    return false;
  }
  if ((spins & 63u) == 0u && __any(ld_agent_u32(&hdr->abort) != 0u)) {
    leave(s_abort, lane);
    return false;
  }
  __builtin_amdgcn_s_sleep(2);
  return true;
}

// The unit's activation slice (16 rows x glen groups x 16 chunks of 8 k) into
// LDS, reordered to the nibble k order; thread t holds chunk t of every group.
// Called once the ready flags of the tiles it spans were seen: no block reads
// them before that in the launch, so plain loads find no stale copy.
__device__ __forceinline__ void load_slice(uint32_t* xlds, const _Float16* xin, int64_t ldin,
                                           const UnitPlan& u, int M) {
  const rsrc_t rx = make_rsrc(xin);
  const int t = (int)threadIdx.x;
  const int row = (t >> 4) & 15, ch = t & 15;
  const int m = row < M ? row : M - 1;              // rows past M: never stored
  const uint32_t off0 = ((uint32_t)m * (uint32_t)ldin + u.gs0 * kGroup + ch * 8) * 2;
  static_assert(kComputeThreads == 256, "one chunk of every group per thread");
  u32x4 v[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i)
    v[i] = ld_x4s(rx, i < u.glen ? off0 : kNoLoad, (uint32_t)i * kGroup * 2);
#pragma unroll
  for (int i = 0; i < kXPer; ++i)
    if (i < u.glen)
      *reinterpret_cast<f16x8*>(xlds + i * kXGroupWords + row * kXRowWords + ch * 4) =
          permute_for_int4(v[i]);
}

__global__ __launch_bounds__(kThreads) void w4a16_chain_kernel(ChainHeader* hdr,
                                                               const _Float16* __restrict__ x,
                                                               int64_t ldx, _Float16* y,
                                                               int64_t ldy, int M_arg, int K0,
                                                               int N_last) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values kept in scalar registers: a value the compiler takes
  // for divergent turns every buffer resource built from it into a per-lane
  // loop around each load
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, chunk = lane & 15;
  const int b = blockIdx.x;

  // a workspace that was not prepared for this call: report and touch nothing else
  if (hdr->magic != kChainMagic || (int)hdr->M != M_arg || (int)hdr->K0 != K0 ||
      (int)hdr->N_last != N_last || hdr->blocks != gridDim.x || hdr->abort != 0u) {
    if (threadIdx.x == 0 && b == 0) st_agent_u32(&hdr->error, 2u);
    return;
  }
  const uint32_t lin_offset = uniform_u32(reinterpret_cast<const unsigned*>(&hdr->lin_offset));
  const ChainLinear* lins =
      reinterpret_cast<const ChainLinear*>(reinterpret_cast<const char*>(hdr) + lin_offset);
  const int nlin = (int)uniform_u32(&hdr->n_linears);
  const int M = (int)uniform_u32(&hdr->M);

  __shared__ uint32_t xlds[kXWords];                // the unit's activation slice
  __shared__ float red[kRedWords];                  // compute waves' sums for the control wave
  __shared__ float sums[4 * 16 * 64];               // the control wave's tile sums
  // LDS counters: inputs ready, slices loaded, sums handed over, sums taken; abort word
  __shared__ unsigned s_epoch, s_in_ready, s_x_ready, s_red_ready, s_red_free, s_abort;
  if (threadIdx.x == 0) {
    s_epoch = ld_agent_u32(&hdr->epoch);
    s_in_ready = s_x_ready = s_red_ready = s_red_free = s_abort = 0u;
  }
  __syncthreads();
  const unsigned epoch = __builtin_amdgcn_readfirstlane(s_epoch);
  const unsigned target = epoch + 1u;               // ready flags written by this launch

  if (wave < kCW) {
    // =========================== compute waves ===========================
    const uint32_t magic = in_vgpr(0x64006400u);
    const int zshift = (lane & 1) * 16;
    ChainLinear L = load_linear(lins);
    ChainLinear Ln = load_linear(lins + (nlin > 1 ? 1 : 0));
    UnitPlan u = plan_unit(L, b, wave, lane, true);
    WRsrc r = weight_rsrc(L);
    WFrag f[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      load_w(f[i], r, u, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    const _Float16* xin = x;                        // this linear's input rows
    int64_t ldin = ldx;
    for (int l = 0; l < nlin; ++l) {
      // the slice buffer is free once every compute wave finished the math of
      // l - 1, and the inputs are ready once the control wave saw their flags
      if (!lds_wait(&s_red_ready, (unsigned)(kCW * l), &s_abort)) return;
      if (!lds_wait(&s_in_ready, (unsigned)(l + 1), &s_abort)) return;
      if (u.valid) load_slice(xlds, xin, ldin, u, M);
      lds_signal(&s_x_ready, lane);
      if (!lds_wait(&s_x_ready, (unsigned)(kCW * (l + 1)), &s_abort)) return;

      f32x4 acc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      // group j0 + i sits in ring slot i; after its math the slot is refilled
      // with the group D further on (masked past the unit's last group)
      const int nsteps = (u.n + D - 1) / D * D;
      for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int j = j0 + i;
          if (j < u.n) {
            const uint32_t* xt = xlds + (u.g0 - u.gs0 + j) * kXGroupWords;
            ZeroPair zz[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) zz[c] = zero_pair((f[i].zw >> (zshift + 4 * c)) & 0xFu);
            f32x4 tmp[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) tmp[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < 4; ++it) {
              const f16x8 av =
                  *reinterpret_cast<const f16x8*>(xt + chunk * kXRowWords + (it * 4 + kb) * 4);
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
              for (int rr = 0; rr < 4; ++rr) acc[c][rr] = __builtin_fmaf(sc[c], tmp[c][rr], acc[c][rr]);
          }
          load_w(f[i], r, u, j0 + D + i);
        }
      }
      // hand the sums over once the control wave has taken the previous ones;
      // element e = rr*4 + c of lane l sits at red[(wave*16 + e)*64 + l]
      if (!lds_wait(&s_red_free, (unsigned)l, &s_abort)) return;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[(wave * 16 + rr * 4 + c) * 64 + lane] = acc[c][rr];
      lds_signal(&s_red_ready, lane);

      // the next linear's first groups stream in while this one is published
      xin = L.out;
      ldin = L.ldo;
      L = Ln;
      u = plan_unit(L, b, wave, lane, l + 1 < nlin);
      r = weight_rsrc(L);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        load_w(f[i], r, u, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      Ln = load_linear(lins + (l + 2 < nlin ? l + 2 : nlin - 1));
    }
    return;
  }

  // ============================== control wave ==============================
  ChainLinear P{};                                  // the previous linear
  ChainLinear L = load_linear(lins);
  ChainLinear Ln = load_linear(lins + (nlin > 1 ? 1 : 0));
  for (int l = 0; l < nlin; ++l) {
    const bool valid = b < L.units;
    const int wt = L.wt, wk = kCW / wt;
    // ---- wait for the ready flags of the input tiles of this block's unit
    //      (lane i watches tile 2 gs0 + i: a 128-k group spans two 64-column tiles)
    if (valid && l > 0) {
      const int split = b - (b / L.splits) * L.splits;
      const int G = L.K / kGroup;
      const int gs0 = (int)((unsigned)(G * split) / (unsigned)L.splits);
      const int glen = (int)((unsigned)(G * (split + 1)) / (unsigned)L.splits) - gs0;
      const unsigned* f = P.flags + 2 * gs0 + lane;
      bool ok = lane >= 2 * glen;
      unsigned spins = 0;
      while (true) {
        if (!ok) ok = ld_agent_u32(f) == target;
        if (__all(ok)) break;
        if (!poll_again(spins, hdr, &s_abort, lane)) return;
      }
    }
    lds_signal(&s_in_ready, lane);
    if (!lds_wait(&s_red_ready, (unsigned)(kCW * (l + 1)), &s_abort)) return;
    // ---- the sums of each tile (lane holds rows 4 kb + r, columns 4 chunk + c)
    // copied into the control wave's own LDS area so that the compute waves
    // may hand over the next linear's sums while this one is published
#pragma unroll 1
    for (int ti = 0; ti < (valid ? wt : 0); ++ti) {
      float o[16];
      if (wk == 4) sum_slices<4>(red, wt, ti, lane, o);
      else if (wk == 2) sum_slices<2>(red, wt, ti, lane, o);
      else sum_slices<1>(red, wt, ti, lane, o);
#pragma unroll
      for (int e = 0; e < 16; ++e) sums[(ti * 16 + e) * 64 + lane] = o[e];
    }
    lds_signal(&s_red_free, lane);
    // this lane's 16 sums of tile ti: rows 4 kb + rr, columns 4 chunk + c at rr * 4 + c
    auto tile_sums = [&](int ti, float o[16]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] = sums[(ti * 16 + e) * 64 + lane];
    };

    if (valid) {
      const int S = L.splits;
      const int cb = b / S;
      const int split = b - cb * S;
      const int T = (L.N + kColTile - 1) / kColTile;
      const bool last_lin = l == nlin - 1;
      const rsrc_t rd = make_rsrc(last_lin ? y : L.out);
      const int64_t ldd = last_lin ? ldy : L.ldo;
      // the output row segment (m, col .. col + 3)
      auto store_out = [&](int m, int col, float a0, float a1, float a2, float a3) {
        const u32x2 w = {pack_f16x2(L.alpha * a0, L.alpha * a1), pack_f16x2(L.alpha * a2, L.alpha * a3)};
        const uint32_t off = (uint32_t)(((size_t)m * ldd + col) * 2);
        if (last_lin) __builtin_amdgcn_raw_buffer_store_b64(w, rd, off, 0, 0);
        else st_agent_x2(rd, off, w);
      };
      // after this block's output stores of its tiles have landed, their ready flags
      auto raise_flags = [&]() {
        if (last_lin) return;
        __builtin_amdgcn_s_waitcnt(0);
        if (lane < wt && cb * wt + lane < T) st_agent_u32(L.flags + cb * wt + lane, target);
      };
      if (S == 1) {
#pragma unroll 1
        for (int ti = 0; ti < wt; ++ti) {
          const int tile = cb * wt + ti;
          const int col = tile * kColTile + 4 * chunk;
          if (tile < T && col < L.N) {
            float o[16];
            tile_sums(ti, o);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int m = 4 * kb + rr;
              if (m < M) store_out(m, col, o[rr * 4 + 0], o[rr * 4 + 1], o[rr * 4 + 2], o[rr * 4 + 3]);
            }
          }
        }
        raise_flags();
      } else {
        // partials: [split][16 rows][ncols], all 16 rows written; the split
        // that arrives last at a tile's ticket adds them in split order
        const size_t ncols = (size_t)L.cb * wt * kColTile;
        const uint32_t split_bytes = (uint32_t)(16 * ncols * 4);
        const rsrc_t pr = make_rsrc(L.partials);
        uint32_t lo[4];                             // lane offsets of rows 4 kb + rr, column 4 chunk
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) lo[rr] = (uint32_t)(((size_t)(4 * kb + rr) * ncols + 4 * chunk) * 4);
#pragma unroll 1
        for (int ti = 0; ti < wt; ++ti) {
          const uint32_t tcol = (uint32_t)((cb * wt + ti) * kColTile) * 4;
          float o[16];
          tile_sums(ti, o);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            st_agent_x4(pr, lo[rr] + tcol + (uint32_t)split * split_bytes,
                        u32x4{__builtin_bit_cast(uint32_t, o[rr * 4 + 0]), __builtin_bit_cast(uint32_t, o[rr * 4 + 1]),
                              __builtin_bit_cast(uint32_t, o[rr * 4 + 2]), __builtin_bit_cast(uint32_t, o[rr * 4 + 3])});
        }
        __builtin_amdgcn_s_waitcnt(0);              // the partials have landed
        unsigned last = 0u;
        if (lane < wt && cb * wt + lane < T) {
          unsigned* tk = L.tickets + (size_t)(cb * wt + lane) * kSlotWords;
          const unsigned prev =
              __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (prev == (unsigned)S - 1) {
            st_agent_u32(tk, 0u);                   // re-armed for the next launch
            last = 1u;
          }
        }
        unsigned finished = 0u;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) finished |= (__shfl(last, ti, 64) & 1u) << ti;
        finished = __builtin_amdgcn_readfirstlane(finished);
        if (finished) {
#pragma unroll 1
          for (int ti = 0; ti < wt; ++ti) {
            if (!((finished >> ti) & 1u)) continue;
            const int col = (cb * wt + ti) * kColTile + 4 * chunk;
            const uint32_t tcol = (uint32_t)((cb * wt + ti) * kColTile) * 4;
            f32x4 sum[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sum[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int sp0 = 0; sp0 < S; sp0 += 4) {
              u32x4 v[4][4];
#pragma unroll
              for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                  v[q][rr] = ld_x4s<kSC1>(pr, sp0 + q < S ? lo[rr] + tcol : kNoLoad,
                                          (uint32_t)(sp0 + q) * split_bytes);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (sp0 + q < S)
#pragma unroll
                  for (int rr = 0; rr < 4; ++rr) sum[rr] += __builtin_bit_cast(f32x4, v[q][rr]);
            }
            if (col < L.N)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int m = 4 * kb + rr;
                if (m < M) store_out(m, col, sum[rr][0], sum[rr][1], sum[rr][2], sum[rr][3]);
              }
          }
          if (!last_lin) {
            __builtin_amdgcn_s_waitcnt(0);
            if (lane < wt && ((finished >> lane) & 1u)) st_agent_u32(L.flags + cb * wt + lane, target);
          }
        }
      }
    }
    P = L;
    L = Ln;
    Ln = load_linear(lins + (l + 2 < nlin ? l + 2 : nlin - 1));
  }

  // the last block out advances the epoch
  __builtin_amdgcn_s_waitcnt(0);
  if (lane == 0) {
    const unsigned e =
        __hip_atomic_fetch_add(&hdr->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e == gridDim.x - 1) {
      st_agent_u32(&hdr->exit_count, 0u);
      __builtin_amdgcn_s_waitcnt(0);
      st_agent_u32(&hdr->epoch, epoch + 1u);
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
