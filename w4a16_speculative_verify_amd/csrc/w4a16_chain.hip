// A chain of W4A16 linears (the target's layers during one verify pass,
// section 3 of "Efficient LLM Challenge Results") in ONE persistent launch,
// gfx950.
//
// Why one launch: at M <= 16 rows a linear moves 5-27 MB, 1-4 us of HBM time,
// while a kernel launch costs about 2.5 us by itself; 144 launches cannot get
// near the HBM bound.  Here one block per CU stays resident for the whole
// chain and the weight stream never waits for the activations: weights do
// not depend on them, so each block's share of every linear is streamed into
// LDS as far ahead as the ring allows, while the dependent steps between
// linears (a memory round trip or two each) run.
//
// Work units.  Linear l's output columns are dealt to G groups of blocks
// (G = 8: the hardware deals workgroups round-robin over the eight XCDs, so
// block b sits on XCD b % 8 -- checked at run time, see below).  Inside its
// group, a block owns one unit: nb 16-column blocks x ng 128-k groups (one
// K-split of a tile of columns).  The host plan picks nb and the split count
// S per linear, and prepacks every block's units, in chain order, into one
// contiguous byte stream at the same byte count as the canonical layout: per
// 128-k group, nb KiB of packed words in MFMA lane order (lane l of column
// block cb: the four words of packed rows 4 it + l / 16, it = 0..3, column
// 16 cb + l % 16), then the group's fp16 scales and zero-point words.
//
// Waves (9 per block, one block per CU):
//   loader     copies the block's stream into a 112 KiB LDS ring with LDS DMA
//              (24 KiB in flight), publishing how many KiB have landed; it
//              waits only for ring space, which the compute waves release group
//              by group (each publishes the stream position below which it
//              needs nothing more; the loader refills up to the lowest);
//   8 compute  per unit: wait for the input tiles' ready flags (agent-scope
//              polls by wave 0), load their k-slice of the activation rows
//              straight into registers in the MFMA A layout (nibble k order),
//              then per group: dequantise the packed words from LDS exactly
//              (q - z in fp16), v_mfma_f32_16x16x32_f16 over the 128 k, the
//              group's scale once on the fp32 sum; the eight k-slices are
//              added through LDS in fixed order.
// Epilogue:
//   S = 1      alpha, fp16 RNE, agent-scope stores of the tile, then its flag;
//   S > 1      splits 1..S-1 store fp32 partials and raise a flag each; split
//              0 keeps its own sums in LDS, waits for the other flags, adds
//              all partials in split order, stores and flags the tile (no
//              atomics: on gfx950 every atomic is a memory-side round trip).
//              The splits of a tile belong to one group; when every block of
//              the group reports the same XCD, partials and split flags stay
//              in that XCD's L2 (plain stores, L1-bypassing loads: about 0.2 us
//              per hop instead of 0.55 us through the memory side); otherwise
//              they take the agent-scope path.
// Output tiles are read by the next linear with plain loads after their
// flags: each linear has its own output buffer, written once per launch, so
// no cache holds a stale copy (the launch boundary invalidates).  Flags hold
// the epoch + 1, so they never need clearing.  Every wait is bounded: a poll
// that exceeds its bound sets the error and abort words and every block
// leaves.
#include <type_traits>

#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kCW = kChainComputeWaves;
constexpr unsigned kRing = kChainRingBytes;
constexpr unsigned kRingKB = kRing / 1024;
constexpr int kNbMax = kChainMaxNb;
constexpr int kWgMax = kChainMaxWaveGroups;
constexpr int kInflight = 24;                       // loader DMA requests in flight (1 KiB each)
constexpr unsigned kSpinLimit = 1u << 22;

// s_waitcnt immediate with vmcnt = n and the other counters left alone (gfx9
// encoding: vmcnt[3:0] bits 3:0, vmcnt[5:4] bits 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(4))) const uint32_t* const_u32_ptr;
// A descriptor read with scalar loads: the values land in SGPRs and the wait
// for them counts against the scalar counter, not behind vector loads.
// Descriptors are written before the launch and never changed by it.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  constexpr int kWords = sizeof(T) / 4;
  const_u32_ptr src = (const_u32_ptr)(p);
  uint32_t w[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) w[i] = src[i];
  T d;
  __builtin_memcpy(&d, w, sizeof(d));
  return d;
}

__device__ __forceinline__ void st_agent_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent_u32(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned lds_load(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

struct Shared {
  unsigned prog[kChainComputeWaves];   // per compute wave: stream bytes it no longer needs
  unsigned epoch, published, cw, abort, last, local;
};

// The compute waves' barrier: a monotone LDS counter (the loader never joins)
__device__ __forceinline__ bool cw_sync(Shared& sh, unsigned& phase, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if (lane == 0) __hip_atomic_fetch_add(&sh.cw, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  ++phase;
  while (__builtin_amdgcn_readfirstlane(lds_load(&sh.cw)) < (unsigned)kCW * phase) {
    if (__builtin_amdgcn_readfirstlane(lds_load(&sh.abort))) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return true;
}

// A poll that gave up: report it and make every block leave.
__device__ __forceinline__ void give_up(ChainHeader* hdr, Shared& sh, int lane) {
  if (lane == 0) {
    st_agent_u32(&hdr->error, 1u);
    st_agent_u32(&hdr->abort, 1u);
    lds_store(&sh.abort, 1u);
  }
}
// Bounded wait between global polls: false once the bound is passed or
// another block gave up.
__device__ __forceinline__ bool poll_again(unsigned& spins, ChainHeader* hdr, Shared& sh, int lane) {
  if (++spins > kSpinLimit) {
    give_up(hdr, sh, lane);
    return false;
  }
  if ((spins & 63u) == 0u) {
    if (__any(ld_agent_u32(&hdr->abort) != 0u) ||
        __builtin_amdgcn_readfirstlane(lds_load(&sh.abort))) {
      if (lane == 0) lds_store(&sh.abort, 1u);
      return false;
    }
  }
  __builtin_amdgcn_s_sleep(1);
  return true;
}

// One KiB from global memory straight into LDS (buffer_load_dwordx4 ... lds:
// lane l's 16 bytes land at M0 + 16 l).  Issued from inline assembly: the
// builtin makes the compiler treat the DMA as an LDS write that any later LDS
// access might alias, so it waited for every DMA in flight before the
// loader's next LDS counter update and the ring stream ran one KiB per memory
// round trip.  The instruction has no destination register; the loader waits
// for its DMAs itself with s_waitcnt vmcnt.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4s dma_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, 0x7fffffffu, 0x00020000u};
}
__device__ __forceinline__ void dma_1k(uint32_t lds_addr, u32x4s src, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(off), "s"(src)
      : "memory");
}

__global__ __launch_bounds__(kChainThreads) void w4a16_chain_kernel(ChainHeader* hdr,
                                                                    const _Float16* __restrict__ x,
                                                                    int64_t ldx, _Float16* y,
                                                                    int64_t ldy, int M_arg, int K0,
                                                                    int N_last) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values in scalar registers (a value the compiler takes for
  // divergent turns a buffer resource built from it into a per-lane loop)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;

  // a workspace that was not prepared for this call: report, touch nothing else
  if (hdr->magic != kChainMagic || (int)hdr->M != M_arg || (int)hdr->K0 != K0 ||
      (int)hdr->N_last != N_last || hdr->blocks != gridDim.x || hdr->abort != 0u) {
    if (threadIdx.x == 0 && b == 0) st_agent_u32(&hdr->error, 2u);
    return;
  }

  __shared__ __attribute__((aligned(16))) unsigned char ring[kRing];
  __shared__ float red[kCW * kNbMax * 4 * 64];   // the k-slices' sums: [(w*kNbMax+cb)*4+r][lane]
  __shared__ Shared sh;
  if (threadIdx.x == 0) {
    sh.epoch = ld_agent_u32(&hdr->epoch);
    sh.published = sh.cw = sh.abort = sh.last = sh.local = 0u;
    for (int w = 0; w < kCW; ++w) sh.prog[w] = 0u;
  }
  __syncthreads();
  const unsigned epoch = __builtin_amdgcn_readfirstlane(sh.epoch);
  const unsigned target = epoch + 1u;               // flags written by this launch

  const char* ws = reinterpret_cast<const char*>(hdr);
  const int blocks = (int)gridDim.x;
  const int nlin = (int)__builtin_amdgcn_readfirstlane(hdr->n_linears);

  if (wave == kCW) {
    // ================================ loader ================================
    const ChainStream st = sload(reinterpret_cast<const ChainStream*>(
                                     ws + __builtin_amdgcn_readfirstlane((unsigned)hdr->stream_offset)) +
                                 b);
    const u32x4s rs = dma_rsrc(ws + st.offset);
    const uint32_t ring_lds = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)ring);
    const unsigned total = st.kb;
    unsigned issued = 0, landed = 0, slot = 0;        // slot = issued % kRingKB
    auto publish = [&](unsigned v) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) lds_store(&sh.published, v);
    };
    unsigned spins = 0;
    // KiB of the stream that every compute wave is done with
    auto consumed = [&]() -> unsigned {
      unsigned m = lds_load(&sh.prog[0]);
#pragma unroll
      for (int w = 1; w < kCW; ++w) {
        const unsigned v = lds_load(&sh.prog[w]);
        m = v < m ? v : m;
      }
      return __builtin_amdgcn_readfirstlane(m) / 1024u;
    };
    // bursts of DMAs up to the free ring space, kInflight KiB in flight,
    // progress published every kPublish KiB
    constexpr int kPublish = 4;
    while (issued < total) {
      unsigned limit = consumed() + kRingKB;
      if (issued >= limit) {
        // ring full: let the waiting compute waves see everything that landed
        __builtin_amdgcn_s_waitcnt(0);
        landed = issued;
        publish(landed);
        spins = 0;
        while (issued >= consumed() + kRingKB) {
          if (__builtin_amdgcn_readfirstlane(lds_load(&sh.abort))) return;
          if (++spins > kSpinLimit) {
            give_up(hdr, sh, lane);
            return;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        continue;
      }
      limit = limit < total ? limit : total;
      while (issued < limit) {
        dma_1k(ring_lds + slot * 1024u, rs, issued * 1024u + (uint32_t)lane * 16u);
        slot = slot + 1u == kRingKB ? 0u : slot + 1u;
        ++issued;
        if (issued >= landed + kInflight) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInflight - kPublish));
          landed = issued - (kInflight - kPublish);
          publish(landed);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    publish(total);
    return;
  }

  // =============================== compute waves ===============================
  const int tid = (int)threadIdx.x;                 // 0 .. 64*kCW-1
  const int kb = lane >> 4, ln = lane & 15;
  const int M = (int)__builtin_amdgcn_readfirstlane(hdr->M);
  const int G = (int)__builtin_amdgcn_readfirstlane(hdr->groups);
  const int P = (int)__builtin_amdgcn_readfirstlane(hdr->group_blocks);
  const ChainLinear* lins = reinterpret_cast<const ChainLinear*>(
      ws + __builtin_amdgcn_readfirstlane((unsigned)hdr->lin_offset));
  const ChainUnit* units = reinterpret_cast<const ChainUnit*>(
      ws + __builtin_amdgcn_readfirstlane((unsigned)hdr->unit_offset));
  unsigned* xcc_tab = reinterpret_cast<unsigned*>(const_cast<char*>(ws) +
                                                  __builtin_amdgcn_readfirstlane((unsigned)hdr->xcc_offset));
  unsigned phase = 0;

  // ---- does every block of this block's group sit on this block's XCD?
  if (wave == 0) {
    const unsigned myx = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 15u;   // HW_REG_XCC_ID[3:0]
    if (lane == 0) st_agent_u32(xcc_tab + b, (target << 4) | myx);
    unsigned ok = 0u;
    if (G > 1) {
      bool seen = lane >= P, same = true;
      const unsigned* e = xcc_tab + (b % G) + G * (lane < P ? lane : 0);
      unsigned spins = 0;
      while (true) {
        if (!seen) {
          const unsigned v = ld_agent_u32(e);
          if ((v >> 4) == (target & 0x0fffffffu)) {
            seen = true;
            same = (v & 15u) == myx;
          }
        }
        if (__all(seen)) break;
        if (!poll_again(spins, hdr, sh, lane)) return;
      }
      ok = __all(same) ? 1u : 0u;
    }
    if (lane == 0) lds_store(&sh.local, ok);
  }
  if (!cw_sync(sh, phase, lane)) return;
  const bool local = __builtin_amdgcn_readfirstlane(lds_load(&sh.local)) != 0u;

  const uint32_t magic = in_vgpr(0x64006400u);
  for (int l = 0; l < nlin; ++l) {
    const ChainUnit U = sload(units + (size_t)l * blocks + b);
    if (U.col0 < 0) continue;
    const ChainLinear L = sload(lins + l);
    const bool last_lin = l == nlin - 1;

    // ---- inputs: wait for the ready flags of the tiles this unit reads
    const _Float16* in = x;
    int64_t ldin = ldx;
    if (l > 0) {
      const ChainLinear Pv = sload(lins + l - 1);
      in = Pv.out;
      ldin = Pv.ld_out;
      if (wave == 0 && U.nf > 0) {
        const unsigned* f = Pv.flags + U.f0 + (lane < U.nf ? lane : 0);
        bool ok = lane >= U.nf;
        unsigned spins = 0;
        while (true) {
          if (!ok) ok = ld_agent_u32(f) == target;
          if (__all(ok)) break;
          if (!poll_again(spins, hdr, sh, lane)) return;
        }
      }
      if (!cw_sync(sh, phase, lane)) return;
    }

    // ---- this wave's k-slice of the activation rows, requested at once in the
    //      MFMA A layout (reordered to the nibble k order group by group, so
    //      the math of the first group starts as soon as its rows land)
    // groups wave, wave + kCW, ... of the unit (interleaved, so that the ring
    // drains front to back and is refilled while the unit is computed)
    const int ngw = U.ng > wave ? (U.ng - wave + kCW - 1) / kCW : 0;
    const unsigned uend = U.soff + (unsigned)U.ng * U.gbytes;
    auto release = [&](int gi) {                    // this wave needs nothing before group gi
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");   // ring reads done
      if (lane == 0)
        lds_store(&sh.prog[wave], gi < ngw ? U.soff + (unsigned)(wave + kCW * gi) * U.gbytes : uend);
    };
    release(0);
    const rsrc_t rx = make_rsrc(in);
    const int row = ln < M ? ln : M - 1;            // rows past M: computed, never stored
    const uint32_t xrow = (uint32_t)row * (uint32_t)ldin;
    u32x4 raw[kWgMax][4];
#pragma unroll
    for (int gi = 0; gi < kWgMax; ++gi)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const uint32_t k = (uint32_t)(U.g0 + wave + kCW * gi) * kGroup + it * 32 + kb * 8;
        raw[gi][it] = ld_x4(rx, gi < ngw ? (xrow + k) * 2u : kNoLoad);
      }

    // ---- the unit's groups of this wave, weights from the LDS ring
    f32x4 acc[kNbMax];
#pragma unroll
    for (int cb = 0; cb < kNbMax; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nb = U.nb;
    // one group for NB column blocks: every LDS read first, then NB independent
    // MFMA chains the compiler can interleave
    auto group_math = [&](auto nbc, const unsigned gpos, const f16x8 (&a)[4]) __attribute__((always_inline)) {
      constexpr int NB = decltype(nbc)::value;
      // ring positions: the group's bytes wrap past the ring's end at most once;
      // the wave-uniform base of each KiB block is wrapped on the scalar unit,
      // the lane offset only when that block straddles the end (rare)
      const unsigned mpos0 = gpos + (unsigned)NB * 1024u;      // the group's scales and zeros
      const unsigned mpos = mpos0 >= kRing ? mpos0 - kRing : mpos0;
      u32x4 q[NB];
      _Float16 sc[NB];
      uint32_t zw[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        unsigned base = gpos + (unsigned)cb * 1024u;
        base = base >= kRing ? base - kRing : base;
        unsigned a0 = base + (unsigned)lane * 16u;
        if (base + 1024u > kRing) a0 = a0 >= kRing ? a0 - kRing : a0;     // wave-uniform test
        q[cb] = *reinterpret_cast<const u32x4*>(ring + a0);
      }
      if (mpos + (unsigned)NB * 40u <= kRing) {                          // wave-uniform test
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          sc[cb] = *reinterpret_cast<const _Float16*>(ring + mpos + (unsigned)(cb * 16 + ln) * 2u);
          zw[cb] = *reinterpret_cast<const uint32_t*>(ring + mpos + (unsigned)NB * 32u +
                                                      (unsigned)(cb * 2 + (ln >> 3)) * 4u);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          unsigned a1 = mpos + (unsigned)(cb * 16 + ln) * 2u;
          a1 = a1 >= kRing ? a1 - kRing : a1;
          unsigned a2 = mpos + (unsigned)NB * 32u + (unsigned)(cb * 2 + (ln >> 3)) * 4u;
          a2 = a2 >= kRing ? a2 - kRing : a2;
          sc[cb] = *reinterpret_cast<const _Float16*>(ring + a1);
          zw[cb] = *reinterpret_cast<const uint32_t*>(ring + a2);
        }
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const ZeroPair zz = zero_pair((zw[cb] >> (4 * (ln & 7))) & 0xFu);
        const uint32_t w0 = q[cb].x, w1 = q[cb].y, w2 = q[cb].z, w3 = q[cb].w;
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        t = mfma16x16x32(a[0], dequant_int4_word(w0, zz, magic), t);
        t = mfma16x16x32(a[1], dequant_int4_word(w1, zz, magic), t);
        t = mfma16x16x32(a[2], dequant_int4_word(w2, zz, magic), t);
        t = mfma16x16x32(a[3], dequant_int4_word(w3, zz, magic), t);
        const float sf = (float)sc[cb];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cb][r] = __builtin_fmaf(sf, t[r], acc[cb][r]);
      }
    };
#pragma unroll
    for (int gi = 0; gi < kWgMax; ++gi) {
      if (gi >= ngw) break;                         // wave-uniform
      const unsigned goff = U.soff + (unsigned)(wave + kCW * gi) * U.gbytes;
      const unsigned need = (goff + U.gbytes + 1023u) / 1024u;
      unsigned spins = 0;
      while (__builtin_amdgcn_readfirstlane(lds_load(&sh.published)) < need) {
        if (__builtin_amdgcn_readfirstlane(lds_load(&sh.abort))) return;
        if (++spins > kSpinLimit) {
          give_up(hdr, sh, lane);
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      const unsigned gpos = goff % kRing;
      f16x8 a[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) a[it] = permute_for_int4(raw[gi][it]);
      switch (nb) {
        case 1: group_math(std::integral_constant<int, 1>{}, gpos, a); break;
        case 2: group_math(std::integral_constant<int, 2>{}, gpos, a); break;
        case 3: group_math(std::integral_constant<int, 3>{}, gpos, a); break;
        case 4: group_math(std::integral_constant<int, 4>{}, gpos, a); break;
        default: group_math(std::integral_constant<int, kNbMax>{}, gpos, a); break;
      }
      release(gi + 1);
    }

    // ---- add the k-slices through LDS
#pragma unroll
    for (int cb = 0; cb < kNbMax; ++cb) {
      if (cb >= nb) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((wave * kNbMax + cb) * 4 + r) * 64 + lane] = acc[cb][r];
    }
    if (!cw_sync(sh, phase, lane)) return;

    // output element (row, col) of the unit: column block cb = col / 16 of
    // lane (col % 16) + 16 (row / 4), accumulator slot row % 4
    const int ncol4 = nb * 4;                       // 4-column chunks per row
    const int nchunks = 16 * ncol4;
    auto chunk_sum = [&](int c, float v[4]) {
      const int rr = c / ncol4, col = (c - rr * ncol4) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cj = col + j, cb = cj >> 4;
        const int li = (cj & 15) + 16 * (rr >> 2), r = rr & 3;
        float s = red[((0 * kNbMax + cb) * 4 + r) * 64 + li];
#pragma unroll
        for (int w = 1; w < kCW; ++w) s += red[((w * kNbMax + cb) * 4 + r) * 64 + li];
        v[j] = s;
      }
    };
    _Float16* dst = last_lin ? y : L.out;
    const int64_t ldd = last_lin ? ldy : L.ld_out;
    const rsrc_t rd = make_rsrc(dst);
    auto store_out = [&](int rr, int col, float a0, float a1, float a2, float a3) {
      const u32x2 w = {pack_f16x2(L.alpha * a0, L.alpha * a1), pack_f16x2(L.alpha * a2, L.alpha * a3)};
      const uint32_t off = (uint32_t)(((size_t)rr * (size_t)ldd + (size_t)(U.col0 + col)) * 2);
      if (last_lin) __builtin_amdgcn_raw_buffer_store_b64(w, rd, off, 0, 0);
      else st_agent_x2(rd, off, w);
    };
    auto raise_flag = [&]() -> bool {
      __builtin_amdgcn_s_waitcnt(0);                // this thread's output stores landed
      if (!cw_sync(sh, phase, lane)) return false;
      if (!last_lin && wave == 0 && lane == 0) st_agent_u32(L.flags + U.tile, target);
      return true;
    };

    if (U.S == 1) {
      for (int c = tid; c < nchunks; c += 64 * kCW) {
        float v[4];
        chunk_sum(c, v);
        const int rr = c / ncol4;
        if (rr < M) store_out(rr, (c - rr * ncol4) * 4, v[0], v[1], v[2], v[3]);
      }
      if (!raise_flag()) return;
      continue;
    }

    // ---- split K: splits 1..S-1 publish fp32 partials [S-1][16][ncols] and a
    //      flag each; split 0 keeps its own sums in LDS, waits for the others'
    //      flags and adds everything in split order
    const int ncols = nb * 16;
    const rsrc_t rp = make_rsrc(L.partials + U.part_off);
    unsigned* sflags = L.sflags + (size_t)U.tile * U.S;
    if (U.split != 0) {
      for (int c = tid; c < nchunks; c += 64 * kCW) {
        float v[4];
        chunk_sum(c, v);
        const int rr = c / ncol4, col = (c - rr * ncol4) * 4;
        const uint32_t off = (uint32_t)((((U.split - 1) * 16 + rr) * ncols + col) * 4);
        const u32x4 pv = {__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                          __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
        if (local) __builtin_amdgcn_raw_buffer_store_b128(pv, rp, off, 0, 0);
        else st_agent_x4(rp, off, pv);
      }
      __builtin_amdgcn_s_waitcnt(0);                // this thread's partials landed
      if (!cw_sync(sh, phase, lane)) return;
      if (wave == 0 && lane == 0) {
        if (local) __hip_atomic_store(sflags + U.split, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else st_agent_u32(sflags + U.split, target);
      }
      continue;
    }
    if (wave == 0) {
      // L1-bypassing polls: they read the L2 of this XCD (local) or the memory side
      const unsigned* f = sflags + (lane >= 1 && lane < U.S ? lane : 1);
      bool ok = lane < 1 || lane >= U.S;
      unsigned spins = 0;
      while (true) {
        if (!ok) ok = ld_agent_u32(f) == target;
        if (__all(ok)) break;
        if (!poll_again(spins, hdr, sh, lane)) return;
      }
    }
    if (!cw_sync(sh, phase, lane)) return;
    for (int c = tid; c < nchunks; c += 64 * kCW) {
      const int rr = c / ncol4, col = (c - rr * ncol4) * 4;
      float v[4];
      chunk_sum(c, v);
      f32x4 sum = {v[0], v[1], v[2], v[3]};
      for (int s0 = 1; s0 < U.S; s0 += 8) {
        u32x4 pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pv[u] = ld_agent_x4(rp, s0 + u < U.S ? (uint32_t)((((s0 + u - 1) * 16 + rr) * ncols + col) * 4)
                                               : kNoLoad);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < U.S) sum += __builtin_bit_cast(f32x4, pv[u]);
      }
      if (rr < M) store_out(rr, col, sum[0], sum[1], sum[2], sum[3]);
    }
    if (!raise_flag()) return;
  }

  // ---- the last block out advances the epoch
  if (!cw_sync(sh, phase, lane)) return;
  if (wave == 0 && lane == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned e =
        __hip_atomic_fetch_add(&hdr->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e == (unsigned)blocks - 1u) {
      st_agent_u32(&hdr->exit_count, 0u);
      __builtin_amdgcn_s_waitcnt(0);
      st_agent_u32(&hdr->epoch, epoch + 1u);
    }
  }
}

// Copies linear l's weights into the blocks' streams: block (b, gi) writes
// group gi of block b's unit (nb KiB of lane-ordered words, then the scales
// and zero-point words, zero padding to 16 bytes).
__global__ __launch_bounds__(64) void w4a16_chain_prepack_kernel(
    const ChainUnit* __restrict__ units, const ChainStream* __restrict__ streams,
    const uint32_t* __restrict__ qweight, const _Float16* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, char* __restrict__ ws) {
  const int b = blockIdx.x, gi = blockIdx.y, lane = threadIdx.x;
  const ChainUnit U = units[b];
  if (U.col0 < 0 || gi >= U.ng) return;
  char* dst = ws + streams[b].offset + U.soff + (size_t)gi * U.gbytes;
  const int g = U.g0 + gi;
  for (int cb = 0; cb < U.nb; ++cb) {
    const int col = U.col0 + cb * 16 + (lane & 15);
    u32x4 w;
#pragma unroll
    for (int it = 0; it < 4; ++it)
      w[it] = qweight[(size_t)(g * 16 + 4 * it + (lane >> 4)) * N + col];
    *reinterpret_cast<u32x4*>(dst + cb * 1024 + lane * 16) = w;
  }
  char* meta = dst + U.nb * 1024;
  for (int j = lane; j < U.nb * 16; j += 64)
    reinterpret_cast<_Float16*>(meta)[j] = scales[(size_t)g * N + U.col0 + j];
  for (int j = lane; j < U.nb * 2; j += 64)
    reinterpret_cast<uint32_t*>(meta + U.nb * 32)[j] = qzeros[(size_t)g * (N / 8) + U.col0 / 8 + j];
  for (int j = U.nb * 40 + lane; j < (int)(U.gbytes - (unsigned)U.nb * 1024u); j += 64) meta[j] = 0;
}

}  // namespace

hipError_t launch_w4a16_chain(ChainHeader* hdr, const _Float16* x, int64_t ldx, _Float16* y,
                              int64_t ldy, int M, int K0, int N_last, int blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(w4a16_chain_kernel, dim3(blocks), dim3(kChainThreads), 0, stream, hdr, x, ldx,
                     y, ldy, M, K0, N_last);
  return hipGetLastError();
}

hipError_t launch_w4a16_chain_prepack(const ChainUnit* units, const ChainStream* streams,
                                      int blocks, int max_ng, const uint32_t* qweight,
                                      const _Float16* scales, const uint32_t* qzeros, int N,
                                      char* ws, hipStream_t stream) {
  hipLaunchKernelGGL(w4a16_chain_prepack_kernel, dim3(blocks, max_ng), dim3(64), 0, stream, units,
                     streams, qweight, scales, qzeros, N, ws);
  return hipGetLastError();
}

}  // namespace w4v
