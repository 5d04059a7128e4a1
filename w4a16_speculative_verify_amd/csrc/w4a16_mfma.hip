// W4A16 linear for many activation rows (the batched verify block of several
// sequences, prefill-shaped blocks), gfx950: a dense contraction bound by the
// matrix cores ("Efficient LLM Challenge Results", section 4: the long
// bucket's cost is prefill compute), so the 4-bit weights are dequantised
// once per block tile into LDS and shared by all of the tile's rows.
//
// Block tile 256 rows x 256 columns (128 or 192 rows for calls with no more
// rows than that), 32 k per stage.  Every global load is an
// LDS DMA (buffer_load ... lds: no registers; issued from inline assembly so
// that the compiler does not wait for it at unrelated LDS accesses -- the
// kernel waits itself with explicit vmcnt counts), kSlots stages deep in a
// ring of LDS slots (5, or 7 / 9 with the smaller tiles), so that a stage's
// data has several stages of MFMA time to arrive.  A slot holds one stage's
//   A     the tile's rows x 32 k fp16, row r's 16-byte chunk c stored at
//         r * 4 + (c ^ lds_sw4(r));
//   W     the packed words, 4 packed rows x 256 columns;
//   meta  the stage's quantisation group: 256 fp16 scales, 32 zero words.
// One stage ahead of the MFMAs, the block dequantises the next stage's words
// from LDS into a double-buffered fp16 B tile in natural k order, as
// fp16(s * (q - z)) (q - z exact, one rounding for the scale, the fp32
// accumulation unchanged).  Column 64 g + 4 j + c of the tile sits at
// position v = 64 g + 16 c + j, its chunk c' at v * 4 + (c' ^ lds_sw4(v)).
// The row swizzle lds_sw4 (w4v_device.h) keeps the MFMA operand reads and
// the dequantisation writes free of LDS bank conflicts.
// 8 waves as 2 (rows) x 4 (columns) of 128 x 64 (or 64 / 96 x 64 with the
// smaller tiles): 8 x 4 v_mfma_f32_16x16x32_f16
// tiles with fp32 accumulators; MFMA tile c of a wave reads positions
// 16 c .. 16 c + 15 of its 64, i.e. columns 4 j + c, so every lane ends up with
// 4 adjacent columns of each row it holds and stores them with one write.
// One block barrier per stage; after it the MFMAs run with the next stage's
// dequantisation between them, then the stage kSlots - 1 ahead is requested.
// Blocks are ordered in groups of 8 row blocks, so that the blocks running
// together share their activation rows and packed weights in L2.
// Split-K: block (tile, split) computes a contiguous range of stages and
// stores fp32 partials [split][tile][BM x BN]; a second kernel adds them in
// split order.  With few tiles every tile is split; with more tiles than CUs
// the full rounds take whole tiles and only the last, partial round's tiles
// are split over the CUs that round would leave idle.
#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int BN = 256, BK = 32;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupM = 8;                          // row blocks per raster group
constexpr uint32_t kBTile = 16384;                  // fp16 B tile: 256 columns x 32 k
constexpr uint32_t kLdsLimit = 160 * 1024;          // LDS per block on gfx950

// LDS layout for MTW m-tiles per wave (block tiles of 32 MTW rows): a slot
// holds one stage's activation tile, packed words, scales and zero words; as
// many slots as fit beside the two B tiles and the sink, so that smaller
// tiles keep more stages in flight
template <int MTW>
struct Lds {
  static constexpr uint32_t kA = 0;                          // 32 MTW rows x 64 bytes
  static constexpr uint32_t kW = 2048u * MTW;                // 4 packed rows x 256 columns
  static constexpr uint32_t kScale = kW + 4096;              // 256 fp16 scales
  static constexpr uint32_t kZero = kScale + 1024;           // 32 zero words (1 KiB reserved)
  static constexpr uint32_t kSlotBytes = kZero + 1024;
  static constexpr int kSlots = (int)((kLdsLimit - 2 * kBTile - 1024) / kSlotBytes);
  static constexpr int kAhead = kSlots - 1;                  // stages requested ahead of the MFMAs
  static constexpr uint32_t kSink = kSlots * kSlotBytes + 2 * kBTile;   // DMAs with no data
  static constexpr uint32_t kBytes = kSink + 1024;
  static_assert(kBytes <= kLdsLimit, "LDS layout exceeds the block's LDS");
};

// raster: tile index -> (row block, column block), in groups of kGroupM row
// blocks with the column blocks inside a group
__device__ __forceinline__ void tile_coords(int tile, int mblocks, int nblocks, int& mblk,
                                            int& nblk) {
  const int per_group = kGroupM * nblocks;
  const int m_first = tile / per_group * kGroupM;
  const int gm = mblocks - m_first < kGroupM ? mblocks - m_first : kGroupM;
  mblk = m_first + (tile % per_group) % gm;
  nblk = (tile % per_group) / gm;
}

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 field layout)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr uint32_t kNoMem = 0x80000000u;            // past every resource: reads no memory

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

// Q = 1: group size 128, 4: group size 32.  MTW 16-row m-tiles per wave: block
// tiles of 32 MTW rows (256, or 192 / 128 for blocks of fewer rows, which then
// spend no MFMAs and no activation reads on rows that do not exist).
// Blocks 0 .. dp-1 take whole tiles over all of K (stored as fp16); the
// blocks after them split each remaining tile dp + u over S contiguous stage
// ranges (block dp + split * ntail + u) and store fp32 partials
// [split][u][BM x BN] for the reduce kernel.
template <int Q, int MTW>
__global__ __launch_bounds__(kThreads) void w4a16_mfma_kernel(GemmArgs a, int mblocks, int nblocks,
                                                              int dp, int ntail, int S,
                                                              float* partials) {
  constexpr int BM = 32 * MTW;
  using L = Lds<MTW>;
  constexpr int kSlots = L::kSlots, kAhead = L::kAhead;
  constexpr uint32_t kA = L::kA, kW = L::kW, kScale = L::kScale, kZero = L::kZero;
  constexpr uint32_t kSlotBytes = L::kSlotBytes, kSink = L::kSink;
  static_assert(3 * (kAhead - 1) <= 63, "vmcnt counts past its range");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[L::kBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;          // 2 x 4 waves
  const int l16 = lane & 15, kb = lane >> 4;

  const int bid = blockIdx.x;
  const bool whole = bid < dp;
  // split tiles in split-major order: the blocks of one stage range run together
  const int tile = whole ? bid : dp + (bid - dp) % ntail;
  const int split = whole ? 0 : (bid - dp) / ntail;
  const int nsplit = whole ? 1 : S;
  int mblk, nblk;
  tile_coords(tile, mblocks, nblocks, mblk, nblk);
  const int m0 = mblk * BM, n0 = nblk * BN;
  const int M = a.M, N = a.N;
  const int stages = a.K / BK;
  const int s_lo = stages * split / nsplit, s_hi = stages * (split + 1) / nsplit;

  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)lds);

  // ---- the wave's three DMAs of a stage (offsets for stage 0):
  //   two of 16 activation rows (rows 32 wave + 16 i + lane / 4, stored chunk
  //   lane % 4); then waves 0-3 packed row `wave` of the stage's four, wave 4
  //   the scales, wave 5 the zero words, waves 6 and 7 nothing (into the sink)
  const u32x4s rx = dma_rsrc(a.x);
  uint32_t xo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wave * 32 + i * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ lds_sw4(r);
    // rows past M or past the tile: the DMA is issued (fixed counts) but reads
    // nothing; those rows' results are never stored
    xo[i] = r < BM && m0 + r < M ? ((uint32_t)(m0 + r) * (uint32_t)a.ldx + (uint32_t)chunk * 8) * 2
                                 : kNoMem;
  }
  const uint32_t Nu = (uint32_t)N;
  u32x4s r3 = dma_rsrc(a.qweight);
  uint32_t o3 = kNoMem, d3 = kSink;                 // third DMA: source offset, LDS offset
  uint32_t step3 = 0;                               // its source step per stage (waves 0-3)
  if (wave < 4) {
    const uint32_t c = (uint32_t)(n0 + 4 * lane);
    o3 = c < Nu ? ((uint32_t)wave * Nu + c) * 4 : kNoMem;
    d3 = kW + (uint32_t)wave * 1024;
    step3 = 4 * Nu * 4;
  } else if (wave == 4) {
    r3 = dma_rsrc(a.scales);
    const uint32_t c = (uint32_t)(n0 + 8 * lane);
    o3 = lane < 32 && c < Nu ? c * 2 : kNoMem;
    d3 = kScale;
  } else if (wave == 5) {
    r3 = dma_rsrc(a.qzeros);
    const uint32_t c = (uint32_t)(n0 + 8 * lane);
    o3 = lane < 32 && c < Nu ? (c >> 3) * 4 : kNoMem;
    d3 = kZero;
  }
  const uint32_t gstep = wave == 4 ? Nu * 2 : (Nu >> 3) * 4;     // meta bytes per group
  // stage s into its slot; a stage past the block's range is requested too,
  // with no source (kNoMem: zeros into a free slot), so that every stage costs
  // a wave exactly three DMAs and the waits below are fixed counts
  auto issue = [&](int s) {
    const bool live = s < s_hi;
    const uint32_t slot = lds0 + (uint32_t)((s - s_lo) % kSlots) * kSlotBytes;
    // waves whose rows lie past a smaller tile write their (empty) DMAs to the sink
    const uint32_t base = wave * 32 < BM ? slot + kA + (uint32_t)wave * 2048 : lds0 + kSink;
    const uint32_t base1 = wave * 32 < BM ? base + 1024 : lds0 + kSink;
    dma16(base, rx, live ? xo[0] + (uint32_t)s * BK * 2 : kNoMem);      // kNoMem + s BK 2 stays
    dma16(base1, rx, live ? xo[1] + (uint32_t)s * BK * 2 : kNoMem);     // past 2 GiB
    uint32_t o = o3;
    if (o != kNoMem)
      o += wave < 4 ? (uint32_t)s * step3 : (uint32_t)(s * BK / (128 / Q)) * gstep;
    o = live ? o : kNoMem;
    const uint32_t d = d3 == kSink ? lds0 + kSink : slot + d3;
    if (wave == 5) dma4(d, r3, o);
    else dma16(d, r3, o);
  };

  // ---- dequantisation: thread t fills B-tile position v = t % 256 (column
  //      dn), chunks 2 (t / 256) and 2 (t / 256) + 1.  Split in its LDS reads
  //      and its arithmetic + writes, so that the arithmetic can run between
  //      the MFMAs of the stage before.
  const int v = t & 255, dh = t >> 8;
  const int dn = (v & ~63) | ((v & 15) << 2) | ((v >> 4) & 3);
  const uint32_t magic = in_vgpr(0x64006400u);
  struct DqIn { uint32_t zw, sb, w0, w1; };
  auto dq_read = [&](int s) {
    const unsigned char* slot = lds + ((s - s_lo) % kSlots) * kSlotBytes;
    DqIn d;
    d.zw = *reinterpret_cast<const uint32_t*>(slot + kZero + (dn >> 3) * 4);
    d.sb = *reinterpret_cast<const unsigned short*>(slot + kScale + dn * 2);
    d.w0 = *reinterpret_cast<const uint32_t*>(slot + kW + ((dh * 2) * 256 + dn) * 4);
    d.w1 = *reinterpret_cast<const uint32_t*>(slot + kW + ((dh * 2 + 1) * 256 + dn) * 4);
    return d;
  };
  const int bw0 = (v * 4 + ((dh * 2) ^ lds_sw4(v))) * 16, bw1 = (v * 4 + ((dh * 2 + 1) ^ lds_sw4(v))) * 16;
  auto dq_write = [&](int s, const DqIn& d) {
    const uint32_t z = (d.zw >> (4 * (dn & 7))) & 0xFu;
    const f16x2 z1024 = __builtin_bit_cast(f16x2, (0x6400u | z) * 0x00010001u);
    const f16x2 sc = __builtin_bit_cast(f16x2, d.sb * 0x00010001u);
    unsigned char* bt = lds + kSlots * kSlotBytes + ((s - s_lo) & 1) * kBTile;
    *reinterpret_cast<u32x4*>(bt + bw0) = dequant_natural(d.w0, z1024, sc, magic);
    *reinterpret_cast<u32x4*>(bt + bw1) = dequant_natural(d.w1, z1024, sc, magic);
  };

  int ao[MTW], bo[4];                               // MFMA operand offsets within a tile
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
    const int r = wm * 16 * MTW + mt * 16 + l16;
    ao[mt] = (r * 4 + (kb ^ lds_sw4(r))) * 16;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int p = wn * 64 + c * 16 + l16;
    bo[c] = (p * 4 + (kb ^ lds_sw4(p))) * 16;
  }
  auto read_a = [&](int s, f16x8 (&av)[MTW]) {
    const unsigned char* as = lds + ((s - s_lo) % kSlots) * kSlotBytes + kA;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) av[mt] = *reinterpret_cast<const f16x8*>(as + ao[mt]);
  };

  f32x4 acc[MTW][4];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- one stage: B fragments of stage s, the next stage's words and A
  //      fragments read, the 32 MFMAs with the next stage's dequantisation
  //      between them, then stage s + kAhead requested.  On entry stage s + 1 has
  //      landed for this wave (DMAs of the two stages after it may still be in
  //      flight); after the barrier it has for every wave, B(s) is complete and
  //      every wave is done with the slot and B tile of stage s - 1.
  auto step = [&](int s, const f16x8 (&av)[MTW], f16x8 (&an)[MTW]) {
    // stages s + 2 .. s + kAhead - 1 still in flight, three DMAs each
    __builtin_amdgcn_s_waitcnt(vmcnt_only(3 * (kAhead - 2)));
    lds_barrier();
    const unsigned char* bs = lds + kSlots * kSlotBytes + ((s - s_lo) & 1) * kBTile;
    f16x8 bv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bv[c] = *reinterpret_cast<const f16x8*>(bs + bo[c]);
    const DqIn d = dq_read(s + 1);
    read_a(s + 1, an);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[mt][c] = mfma16x16x32(av[mt], bv[c], acc[mt][c]);
    dq_write(s + 1, d);
    // last: a DMA instruction can stall its wave at issue while the memory
    // path is busy; issued after the MFMAs, the stall of one wave leaves the
    // matrix unit to the other wave of its SIMD
    issue(s + kAhead);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);      // B fragment reads
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);     // dequant inputs, next A fragments
#pragma unroll
    for (int i = 0; i < 4 * MTW; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);    // two VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);      // B tile writes
  };

  // ---- prologue: request the first kAhead stages, dequantise the first
  //      stage and read its A fragments
#pragma unroll
  for (int i = 0; i < kAhead; ++i) issue(s_lo + i);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(3 * (kAhead - 1)));   // stage s_lo has landed
  lds_barrier();
  dq_write(s_lo, dq_read(s_lo));
  f16x8 a0[MTW], a1[MTW];
  read_a(s_lo, a0);

  int s = s_lo;
  for (; s + 1 < s_hi; s += 2) {
    step(s, a0, a1);
    step(s + 1, a1, a0);
  }
  if (s < s_hi) step(s, a0, a1);

  // ---- epilogue: lane holds rows 16 mt + 4 kb + e, columns 4 l16 .. + 3 of its tile
  const int col = n0 + wn * 64 + 4 * l16;
  if (col >= N) return;                             // N % 8 == 0: 4 columns all in or all out
  if (!whole) {
    float* pp = partials + ((size_t)split * ntail + (tile - dp)) * BM * BN + (col - n0);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wm * 16 * MTW + mt * 16 + 4 * kb + e;
        if (m0 + r < M) {
          const f32x4 val = {acc[mt][0][e], acc[mt][1][e], acc[mt][2][e], acc[mt][3][e]};
          *reinterpret_cast<f32x4*>(pp + (size_t)r * BN) = val;
        }
      }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + wm * 16 * MTW + mt * 16 + 4 * kb + e;
      if (m < M) {
        const f16x2 lo = {(_Float16)(a.alpha * acc[mt][0][e]), (_Float16)(a.alpha * acc[mt][1][e])};
        const f16x2 hi = {(_Float16)(a.alpha * acc[mt][2][e]), (_Float16)(a.alpha * acc[mt][3][e])};
        const u32x2 val = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<u32x2*>(a.y + (size_t)m * a.ldy + col) = val;
      }
    }
}

// y = fp16(alpha * sum of the S partials in split order) over the split
// tiles, 4 columns per thread; BM / 4 blocks of 256 threads per tile
__global__ __launch_bounds__(256) void w4a16_mfma_reduce_kernel(const float* __restrict__ partials,
                                                                int S, int M, int N, float alpha,
                                                                _Float16* __restrict__ y,
                                                                int64_t ldy, int BM, int mblocks,
                                                                int nblocks, int dp, int ntail) {
  const int per_tile = BM / 4;
  const int u = blockIdx.x / per_tile;
  const int q = (blockIdx.x % per_tile) * 256 + threadIdx.x;   // quad within the tile
  const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
  int mblk, nblk;
  tile_coords(dp + u, mblocks, nblocks, mblk, nblk);
  const int m = mblk * BM + r, n = nblk * BN + c;
  if (m >= M || n >= N) return;                     // N % 8 == 0: 4 columns all in or all out
  const size_t tile_elems = (size_t)BM * BN;
  const size_t i = (size_t)u * tile_elems + (size_t)r * BN + c;
  f32x4 s = *reinterpret_cast<const f32x4*>(partials + i);
  for (int k = 1; k < S; ++k)
    s += *reinterpret_cast<const f32x4*>(partials + (size_t)k * ntail * tile_elems + i);
  const f16x2 lo = {(_Float16)(alpha * s[0]), (_Float16)(alpha * s[1])};
  const f16x2 hi = {(_Float16)(alpha * s[2]), (_Float16)(alpha * s[3])};
  *reinterpret_cast<u32x2*>(y + (size_t)m * ldy + n) = u32x2{__builtin_bit_cast(uint32_t, lo),
                                                             __builtin_bit_cast(uint32_t, hi)};
}

template <int MTW>
void launch_m(const GemmArgs& a, const MfmaPlan& p, dim3 grid, float* partials,
              hipStream_t stream) {
  if (a.group_size == 32)
    hipLaunchKernelGGL((w4a16_mfma_kernel<4, MTW>), grid, dim3(kThreads), 0, stream, a, p.mblocks,
                       p.nblocks, p.dp, p.ntail, p.splits, partials);
  else
    hipLaunchKernelGGL((w4a16_mfma_kernel<1, MTW>), grid, dim3(kThreads), 0, stream, a, p.mblocks,
                       p.nblocks, p.dp, p.ntail, p.splits, partials);
}

}  // namespace

MfmaPlan plan_w4a16_mfma(int M, int N, int K, int num_cus) {
  MfmaPlan p{};
  // block rows: 256, or the smallest of 128 / 192 that holds every row
  p.mtw = M <= 128 ? 4 : (M <= 192 ? 6 : 8);
  const int BM = 32 * p.mtw;
  p.mblocks = (M + BM - 1) / BM;
  p.nblocks = (N + BN - 1) / BN;
  const int tiles = p.mblocks * p.nblocks;
  const int stages = K / BK;
  // time ~ rounds of blocks (one block per CU) x stages per block (~0.5 us
  // each), plus for split tiles their partials written and read again (fp32
  // at ~5 TB/s) and the reduce launch
  p.dp = tiles;
  p.splits = 1;
  const double tile_bytes = (double)BM * BN * 4;
  if (tiles <= num_cus) {
    // few tiles: every tile split S ways
    double best = 0;
    for (int S = 1; S <= 32 && stages / S >= 8; ++S) {
      const double rounds = (double)((tiles * S + num_cus - 1) / num_cus);
      double t = rounds * ((stages + S - 1) / S) * 0.5;
      if (S > 1) t += 2.0 * S * M * (double)N * 4 / 5e6 + 3.0;
      if (S == 1 || t < best - 1e-9) {
        best = t;
        p.splits = S;
        p.dp = S > 1 ? 0 : tiles;
      }
    }
  } else if (tiles % num_cus != 0) {
    // whole tiles for the full rounds, and the last partial round's tiles
    // split over the CUs that round would leave idle (M = 2048 gate+up: 608
    // tiles = 2 rounds + 96 tiles x 2 splits instead of 3 rounds)
    // (a full-size tile's stage takes ~1 us with a CU to itself, measured on
    // MI355X at 2048 and 8192 rows)
    const int full = tiles / num_cus, rem = tiles % num_cus;
    int st = num_cus / rem;
    while (st > 1 && stages / st < 8) --st;
    if (st > 1) {
      const double stage_us = 1.0;
      const double t_whole = (full + 1) * stages * stage_us;
      const double t_tail = full * stages * stage_us + ((stages + st - 1) / st) * stage_us +
                            2.0 * st * rem * tile_bytes / 5e6 + 3.0;
      if (t_tail < t_whole) {
        p.dp = full * num_cus;
        p.splits = st;
      }
    }
  }
  p.ntail = p.splits > 1 ? tiles - p.dp : 0;
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * p.ntail * (size_t)BM * BN * sizeof(float) : 0;
  return p;
}

hipError_t launch_w4a16_mfma(const GemmArgs& a, const MfmaPlan& p, float* partials,
                             hipStream_t stream) {
  if (p.dp + p.ntail != p.mblocks * p.nblocks || (p.splits > 1) != (p.ntail > 0))
    return hipErrorInvalidValue;
  const dim3 grid(p.dp + p.ntail * p.splits);
  if (p.mtw == 8) launch_m<8>(a, p, grid, partials, stream);
  else if (p.mtw == 6) launch_m<6>(a, p, grid, partials, stream);
  else if (p.mtw == 4) launch_m<4>(a, p, grid, partials, stream);
  else return hipErrorInvalidValue;
  if (p.ntail > 0) {
    const int bm = 32 * p.mtw;
    hipLaunchKernelGGL(w4a16_mfma_reduce_kernel, dim3((unsigned)(p.ntail * (bm / 4))), dim3(256),
                       0, stream, partials, p.splits, a.M, a.N, a.alpha, a.y, a.ldy, bm,
                       p.mblocks, p.nblocks, p.dp, p.ntail);
  }
  return hipGetLastError();
}

}  // namespace w4v
