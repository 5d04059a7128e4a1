// Device-side helpers shared by the gfx950 kernels of libw4v (internal header).
//
// Wave64 MFMA operand layout used throughout (v_mfma_f32_16x16x32_f16):
//   A (16 x 32): lane l holds row (l % 16), eight k values of k-block (l / 16)
//   B (32 x 16): lane l holds column (l % 16), eight k values of k-block (l / 16)
//   D (16 x 16): lane l holds rows 4*(l / 16) + r (r = 0..3) of column (l % 16)
// A and B index k identically, so any fixed permutation of the eight k values
// inside a k-block is harmless as long as both operands use it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4v {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Pointers that were stored in LDS (or any memory) come back as generic
// pointers, and generic (flat) loads count against both the vector-memory and
// the LDS counters, so every LDS wait would also wait for them.  as_global()
// restores the global address space for such pointers.
#define W4V_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const W4V_GLOBAL T* as_global(const T* p) {
  return (const W4V_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ W4V_GLOBAL T* as_global_mut(T* p) {
  return (W4V_GLOBAL T*)(p);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Keeps a constant in a VGPR so that the compiler can fuse AND+OR into one
// v_and_or_b32 (VOP3 on gfx950 takes no literal operand).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint32_t sub_pair(uint32_t a, f16x2 b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) - b);
}

__device__ __forceinline__ uint32_t fma_pair(uint32_t a, f16x2 m, f16x2 b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) * m - b);
}

// Zero-point of one column as the two fp16 offsets the dequantisation needs.
struct ZeroPair {
  f16x2 z1024;   // (1024 + z, 1024 + z)
  f16x2 z64;     // (64 + z, 64 + z)
};

__device__ __forceinline__ ZeroPair zero_pair(uint32_t z) {
  ZeroPair p;
  p.z1024 = __builtin_bit_cast(f16x2, (0x6400u | z) * 0x00010001u);
  p.z64 = __builtin_bit_cast(f16x2, (0x5400u | (z << 4)) * 0x00010001u);
  return p;
}

// Eight unsigned 4-bit weights of one word, minus the zero-point, as fp16,
// with no rounding anywhere:
//   * 0x6400 is 1024.0 in fp16 (mantissa step 1).  A nibble q OR-ed into mantissa
//     bits 0..3 gives 1024 + q; subtracting 1024 + z leaves q - z.
//   * A nibble left in bits 4..7 gives 1024 + 16q; one fused multiply-add
//     (1024 + 16q) * 1/16 - (64 + z) leaves q - z (exactly representable, so
//     the single rounding of the FMA is exact).
// Pair p of the result holds nibbles p (low half) and p + 4 (high half), so
// the eight fp16 values follow k offsets {0, 4, 1, 5, 2, 6, 3, 7} of the word.
// `magic` must hold 0x64006400 (in a VGPR, see in_vgpr).
__device__ __forceinline__ f16x8 dequant_int4_word(uint32_t w, const ZeroPair& z, uint32_t magic) {
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const uint32_t r0 = (w & 0x000F000Fu) | magic;
  const uint32_t r1 = (w & 0x00F000F0u) | magic;
  const uint32_t r2 = (w8 & 0x000F000Fu) | magic;
  const uint32_t r3 = (w8 & 0x00F000F0u) | magic;
  const u32x4 o = {sub_pair(r0, z.z1024), fma_pair(r1, sixteenth, z.z64), sub_pair(r2, z.z1024),
                   fma_pair(r3, sixteenth, z.z64)};
  return __builtin_bit_cast(f16x8, o);
}

// Eight consecutive fp16 activations (four dwords, natural k order) reordered
// to the {0, 4, 1, 5, 2, 6, 3, 7} order that dequant_int4_word produces.
__device__ __forceinline__ f16x8 permute_for_int4(u32x4 d) {
  const u32x4 r = {__builtin_amdgcn_perm(d.z, d.x, 0x05040100u),
                   __builtin_amdgcn_perm(d.z, d.x, 0x07060302u),
                   __builtin_amdgcn_perm(d.w, d.y, 0x05040100u),
                   __builtin_amdgcn_perm(d.w, d.y, 0x07060302u)};
  return __builtin_bit_cast(f16x8, r);
}

// Four int8 weights (one dword, natural k order) as four fp16 in two pairs.
// XOR 0x80 maps the signed byte b to b + 128 in 0..255; placing that byte
// under the exponent byte 0x64 gives 1024 + b + 128 exactly, and subtracting
// 1152 leaves b exactly.
__device__ __forceinline__ uint32_t int8_pair_lo(uint32_t u) {
  const f16x2 off = __builtin_bit_cast(f16x2, 0x64806480u);   // (1152, 1152)
  return __builtin_bit_cast(
      uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off);
}

__device__ __forceinline__ uint32_t int8_pair_hi(uint32_t u) {
  const f16x2 off = __builtin_bit_cast(f16x2, 0x64806480u);
  return __builtin_bit_cast(
      uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off);
}

// Eight int8 weights (two dwords, natural k order) as eight fp16.
__device__ __forceinline__ f16x8 dequant_int8_x8(u32x2 d) {
  const uint32_t u0 = d.x ^ 0x80808080u;
  const uint32_t u1 = d.y ^ 0x80808080u;
  const u32x4 o = {int8_pair_lo(u0), int8_pair_hi(u0), int8_pair_lo(u1), int8_pair_hi(u1)};
  return __builtin_bit_cast(f16x8, o);
}

// ---- cross-block hand-off without whole-cache maintenance -------------------
// Blocks of one launch publish fp32 partial results that the last block to
// arrive combines.  The partials are written and read with relaxed
// agent-scope atomic accesses (coherent across the XCDs' separate L2 caches
// without writing back or invalidating the whole L2, which a device-wide fence
// would do), and every thread waits for its stores to complete before the
// block takes its ticket.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Vector forms of the same agent-scope accesses, through buffer instructions
// with the sc1 cache-policy bit (the bit the scalar forms above carry).  The
// resource covers [base, base + 2 GiB); offsets are in bytes.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kSC1 = 16;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void st_agent_x4(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSC1);
}
__device__ __forceinline__ void st_agent_x2(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kSC1);
}
__device__ __forceinline__ u32x4 ld_agent_x4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1);
}

// The same hand-off for blocks known to share one XCD's L2: plain stores
// (written through the vector L1 into the L2) and loads with the sc0 bit
// (they miss the L1).  Valid only when every block that writes or reads the
// partials runs on the same XCD.  It saves the sc1 round trips; by the
// fetch counters the partials still travel to and from the memory side.
constexpr int kSC0 = 1;

// Block barrier that orders LDS accesses only.  __syncthreads() also waits
// for every global load in flight, which would drain a load pipeline at each
// step; this one leaves them in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Plain buffer loads (cache policy Aux: 0, or kNT for streaming data).  An
// offset at or past 2 GiB lies outside every resource made by make_rsrc and
// reads zeros without touching memory: a branch-free way to skip a load.
constexpr int kNT = 2;
constexpr uint32_t kNoLoad = 0x80000000u;
template <int Aux = 0>
__device__ __forceinline__ u32x4 ld_x4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, Aux);
}
// The same with a wave-uniform byte offset in the scalar operand (added to
// the per-lane offset before the range check).
template <int Aux = 0>
__device__ __forceinline__ u32x4 ld_x4s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, Aux);
}
__device__ __forceinline__ u32x2 ld_x2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld_x1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Takes the block's ticket on `ticket` after all of the block's agent-scope
// stores have completed.  True (in every thread) for the block that arrives
// last of `count`; that block re-arms the counter to zero.
__device__ __forceinline__ bool arrive_last(unsigned* ticket, unsigned count) {
  __shared__ unsigned s_prev;
  __builtin_amdgcn_s_waitcnt(0);     // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    s_prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const bool last = s_prev == count - 1;
  if (last && threadIdx.x == 0)
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// ---- global -> LDS copies without registers (buffer_load ... lds) ----------
// Lane l's 16 bytes land at M0 + 16 l.  Issued from inline assembly so that
// the compiler does not wait for them at unrelated LDS accesses; the kernels
// that use them wait with explicit vmcnt counts (M0 saved and restored).
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4s dma_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, 0x7fffffffu, 0x00020000u};
}
__device__ __forceinline__ void dma16(uint32_t lds_addr, u32x4s src, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(off), "s"(src)
      : "memory");
}
// The same with 4 bytes per lane (to M0 + 4 l).
__device__ __forceinline__ void dma4(uint32_t lds_addr, u32x4s src, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(off), "s"(src)
      : "memory");
}
// LDS row swizzle for tiles of 64-byte rows (four 16-byte chunks): chunk c of
// row r sits at r * 4 + (c ^ lds_sw4(r)).  gfx950 LDS (measured): 64 banks of
// 4 bytes; a 16-byte read serves in one cycle the 4 lane quads of a 32-lane
// half whose quad index (lane bits 2..4) has the same bit parity, a 16-byte
// write 8 consecutive lanes.  For an MFMA operand read (16 consecutive rows,
// chunk l / 16) that is rows {0-3, 12-15} of one chunk with rows {4-11} of
// the next; -(r / 4) mod 4 spreads each such set over all 64 banks and keeps
// 8 consecutive rows of one chunk in distinct banks for the writes.
__device__ __forceinline__ int lds_sw4(int r) { return (4 - ((r >> 2) & 3)) & 3; }

// Total order for greedy argmax: larger value first, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

}  // namespace w4v
