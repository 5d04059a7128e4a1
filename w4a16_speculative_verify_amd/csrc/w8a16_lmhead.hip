// 8-bit lm_head with fused greedy argmax, optionally followed by the greedy
// prefix acceptance, gfx950 (section 3 of the organisers' results page:
// untied lm_head quantised to 8 bits, temperature-0 verification).
//
// Work decomposition
//   wave pass = TILES x 16 vocabulary rows over the whole hidden width H, in
//     steps of 128 k.  Lane l streams 32 consecutive bytes (k = 32*(l/16) ..)
//     of row v0 + 16*t + l%16 per step: two 128-bit loads per tile.  Each
//     8-byte slice is the B operand of one 16x16x32 MFMA.  With fp16 weights
//     (a half-precision head) the lane streams 64 bytes, four 128-bit loads,
//     each the B operand of one MFMA as loaded.
//   A (hidden rows) = one 128-k chunk per step, loaded once per block (16
//     bytes per thread and load round) into a double-buffered LDS tile that
//     the block's waves share: per-wave loads of it would cost a CU as much
//     load throughput as half the weights.  A block of at most 16 rows with
//     H <= kWholeH instead stages the whole hidden rows in LDS once, before
//     its first step (80 KiB at H = 2560): the steps then need no hidden
//     loads, no LDS writes and no barrier.  Its 16-byte chunks are swizzled
//     within each 128-k segment (chunk c of row r at c ^ g(r)), which makes
//     the A-fragment reads conflict-free under gfx950's ds_read_b128 service
//     order (per cycle, the four lane quads of a 32-lane half whose quad
//     indices have equal bit parity).
//   The block's passes are one sequence of steps streamed through a ring of
//     D register sets; every load is unconditional (rows past V read row 0,
//     steps past the block's work read zeros from outside the buffer
//     resource), because a load under a branch makes the compiler wait for
//     every load in flight.
//   Logits stay in fp32 registers (never stored): logit = s8[v] * acc.
//   Argmax: per lane running best over its columns (strict '>' keeps the
//     lowest index because a lane's v only grows), then 16-lane butterflies
//     and a fixed-order merge over the block's waves under the total order
//     (value descending, index ascending); one (value, index) per row and
//     block goes to the workspace, and the last block to arrive merges them.
//   The merging block also runs the greedy prefix scan when asked to.
#include <math.h>

#include "w4v_device.h"
#include "w4v_launch.h"

namespace w4v {

namespace {

constexpr int kChunk = 128;                         // k per step
// LDS row of the per-step hidden chunk: 16 chunks of 16 bytes, unpadded; chunk c
// of row r sits at c ^ hswz(r % 16), as in the whole-row tile
constexpr int kHRowWords = kChunk * 2 / 4;
constexpr int kLmheadBlocksPerCU = 1;
constexpr int kWholeH = 2560;                       // widest hidden row staged whole (16-row blocks)

// chunk swizzle of the whole-row hidden tile: rows 4..11 flip bit 2 as well,
// so that in each read cycle the four served quads cover all 16 chunks
__device__ __forceinline__ int hswz(int r) { return r ^ (((r + 4) & 8) >> 1); }

__device__ __forceinline__ void shfl_best(float& v, int& i, int mask) {
  const float ov = __shfl_xor(v, mask, 64);
  const int oi = __shfl_xor(i, mask, 64);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// F16 = 0: int8 weights with one fp16 scale per vocabulary row; F16 = 1: fp16
// weights, no scale (a half-precision lm_head, results page section 5).
template <int MT, int TILES, int F16, int WH, int HR>
struct Step {
  static constexpr int kLoads = F16 ? 4 : 2;      // 128-bit loads per tile row (32 k)
  u32x4 w[TILES][kLoads];  // 32 k of each tile row
  u32x4 h[WH ? 1 : HR];    // this thread's 16-byte pieces of the hidden chunk (not with WH)
  uint32_t sc[TILES];      // fp16 scale of each tile row (int8 only; with a pass's last step)
};

// WH = 1: 16-row block (MT = 1) with the whole hidden rows in LDS, H <= kWholeH.
// NW waves per block (4, or 8 for 96-row blocks: the hidden chunk, which every
// step loads whole, then serves twice as many vocabulary rows).
template <int MT, int TILES, int D, int F16, int WH, int NW>
__global__ __launch_bounds__(64 * NW) void lmhead_argmax_kernel(LmheadArgs a, unsigned* ticket,
                                                                float* pval, int* pidx) {
  static_assert(!WH || (MT == 1 && NW == 4), "whole hidden rows only for 16-row blocks");
  constexpr int kWaves = NW;
  constexpr int kThreads = 64 * NW;
  // hidden chunk: each load round covers 4 NW rows (16 threads per row)
  constexpr int kRowsPerRound = kThreads / 16;
  static_assert((16 * MT) % kRowsPerRound == 0, "hidden rows must fill the load rounds");
  constexpr int HR = 16 * MT / kRowsPerRound;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kb = lane >> 4;
  // Four-wave blocks: grid x = m-blocks, y = vocabulary blocks, so that the
  // m-blocks of one vocabulary share are dispatched together and read its
  // weights at about the same time (the grid can exceed one block per CU).
  // Eight-wave blocks (two m-blocks, one block per CU, all resident at once):
  // x = vocabulary share, so that the two m-blocks of a share (ids v and
  // v + shares) run on one XCD and share its L2 when the share count is a
  // multiple of 8 (128 shares for the 151,936-row head).
  constexpr bool kShareX = NW == 8;
  const int vbk = kShareX ? blockIdx.x : blockIdx.y;
  const int mblk = kShareX ? blockIdx.y : blockIdx.x;
  const int mbase = mblk * 16 * MT;
  const int nvb = kShareX ? gridDim.x : gridDim.y;
  constexpr int kRowsPerPass = kWaves * TILES * 16;
  // this block's vocabulary rows: an equal share [vb0, vb1), in passes
  const int vb0 = (int)((long long)a.V * vbk / nvb);
  const int vb1 = (int)((long long)a.V * (vbk + 1) / nvb);
  const int my_passes = (vb1 - vb0 + kRowsPerPass - 1) / kRowsPerPass;
  const int nchunks = a.H / kChunk;
  const int nsteps = my_passes * nchunks;

  constexpr int kHWords = MT * 16 * kHRowWords;
  constexpr int kHBufWords = WH ? 16 * kWholeH / 2 : 2 * kHWords;
  __shared__ __attribute__((aligned(16))) uint32_t hbuf[kHBufWords];
  const int hrow_words = a.H / 2;                   // whole-row tile: row stride

  const rsrc_t rw = make_rsrc(a.w);
  const rsrc_t rh = make_rsrc(a.h);
  const rsrc_t rs = make_rsrc(a.scales);
  // hidden chunk: thread t loads row t / 16 (+4 NW per round), 8 k at (t % 16) * 8
  const int hr = threadIdx.x >> 4, hc = threadIdx.x & 15;
  uint32_t hoff[HR];
#pragma unroll
  for (int j = 0; j < HR; ++j) {
    int m = mbase + j * kRowsPerRound + hr;
    m = m < a.M ? m : a.M - 1;                     // rows past M: never reported
    hoff[j] = ((uint32_t)m * (uint32_t)a.ldh + hc * 8) * 2;
  }
  // lane row of tile t in pass p; rows past the block's share load nothing
  auto row_of = [&](int pass, int t) {
    return vb0 + pass * kRowsPerPass + wave * TILES * 16 + 16 * t + (lane & 15);
  };

  constexpr int EB = F16 ? 2 : 1;                   // bytes per weight
  auto load_step = [&](Step<MT, TILES, F16, WH, HR>& f, int st) {
    // Offsets are masked by OR-ing kNoLoad (bit 31) in, never by choosing
    // between two loads: the compiler turns a select on a block-uniform
    // condition into a branch around the load.
    const int sc = st < nsteps ? st : 0;
    const uint32_t skip = st < nsteps ? 0u : kNoLoad;
    const int pass = sc / nchunks;
    const int ch = sc - pass * nchunks;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int v = row_of(pass, t);
      const uint32_t off =
          (((uint32_t)(v < vb1 ? v : 0) * (uint32_t)a.H + kb * 32 + ch * kChunk) * EB) | skip |
          (v < vb1 ? 0u : kNoLoad);
#pragma unroll
      for (int u = 0; u < Step<MT, TILES, F16, WH, HR>::kLoads; ++u) f.w[t][u] = ld_x4(rw, off + 16 * u);
    }
    if constexpr (!WH) {
#pragma unroll
      for (int j = 0; j < HR; ++j) f.h[j] = ld_x4(rh, (hoff[j] + ch * kChunk * 2) | skip);
    }
    // the row scales ride with the last step of a pass (a load at the pass end
    // would wait for the whole ring)
    if constexpr (!F16) {
      const uint32_t not_last = ch == nchunks - 1 ? 0u : kNoLoad;
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int v = row_of(pass, t);
        f.sc[t] = __builtin_amdgcn_raw_buffer_load_b16(
            rs, ((uint32_t)(v < vb1 ? v : 0) * 2) | skip | not_last | (v < vb1 ? 0u : kNoLoad), 0,
            0);
      }
    }
  };

  float best[MT][4];
  int bidx[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      best[mt][r] = -INFINITY;
      bidx[mt][r] = 0x7fffffff;
    }
  f32x4 acc[MT][TILES];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // whole hidden rows: thread t stages row t / 16, chunks t % 16 + 16 j of the
  // row (chunk j of 128 k is segment j), all requested before the weights
  constexpr int kWholeLoads = WH ? kWholeH / kChunk : 1;
  u32x4 hw[kWholeLoads];
  if constexpr (WH) {
#pragma unroll
    for (int j = 0; j < kWholeLoads; ++j)
      hw[j] = ld_x4(rh, (hoff[0] + (uint32_t)j * kChunk * 2) | (j < nchunks ? 0u : kNoLoad));
  }
  Step<MT, TILES, F16, WH, HR> f[D];
  // prologue in the loop's order, so the loop head's wait counts agree on entry
#pragma unroll
  for (int i = 0; i < D; ++i) {
    load_step(f[i], i);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (WH) {
    const int c = hswz(hr) ^ hc;
#pragma unroll
    for (int j = 0; j < kWholeLoads; ++j)
      if (j < nchunks)
        *reinterpret_cast<u32x4*>(hbuf + hr * hrow_words + j * 64 + c * 4) = hw[j];
    __syncthreads();
  }
  const int arow = lane & 15;
  const int aswz = hswz(arow);
  // this thread's chunk position in the per-step tile (its rows are hr + a
  // multiple of 16, so they share hr % 16)
  const int hsw = hc ^ hswz(hr & 15);
  // steps padded to a multiple of D: no branch around loads or barriers
  const int nsteps_pad = (nsteps + D - 1) / D * D;
  for (int s0 = 0; s0 < nsteps_pad; s0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int st = s0 + i;
      uint32_t* ht = hbuf + (st & 1) * kHWords;
      if constexpr (!WH) {
#pragma unroll
        for (int j = 0; j < HR; ++j)
          *reinterpret_cast<u32x4*>(ht + (j * kRowsPerRound + hr) * kHRowWords + hsw * 4) =
              f[i].h[j];
        lds_barrier();
      }
      // whole-row tile: this step's 128-k segment
      const uint32_t* hseg = hbuf + arow * hrow_words + (st % nchunks) * 64;
      if (st < nsteps) {                            // block-uniform
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // A: row l % 16, k = 32 (l / 16) + 8 q .. + 7
          f16x8 av[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {  // rows past M repeat row M - 1: never reported
            if constexpr (WH)
              av[mt] = *reinterpret_cast<const f16x8*>(hseg + (((kb * 4 + q) ^ aswz) * 4));
            else
              av[mt] = *reinterpret_cast<const f16x8*>(ht + (mt * 16 + arow) * kHRowWords +
                                                       (((kb * 4 + q) ^ aswz) * 4));
          }
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            f16x8 b;
            if constexpr (F16) {
              b = __builtin_bit_cast(f16x8, f[i].w[t][q]);
            } else {
              const u32x4& src = f[i].w[t][q >> 1];
              const u32x2 d = (q & 1) ? u32x2{src.z, src.w} : u32x2{src.x, src.y};
              b = dequant_int8_x8(d);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][t] = mfma16x16x32(av[mt], b, acc[mt][t]);
          }
        }
        if (st % nchunks == nchunks - 1) {          // end of a pass: logits, argmax
          const int pass = st / nchunks;
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            const int v = row_of(pass, t);
            if (v < vb1) {
              float sv = 1.f;
              if constexpr (!F16) sv = (float)__builtin_bit_cast(_Float16, (uint16_t)f[i].sc[t]);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const float lg = sv * acc[mt][t][r];
                  if (lg > best[mt][r]) {
                    best[mt][r] = lg;
                    bidx[mt][r] = v;
                  }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
      load_step(f[i], st + D);
    }
  }

  // ---- 16-lane butterflies: lanes of one k-block share rows 4*(l/16) + r
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int mask = 1; mask < 16; mask <<= 1) shfl_best(best[mt][r], bidx[mt][r], mask);

  // ---- merge the waves in fixed order
  constexpr int R = 16 * MT;
  __shared__ float s_val[kWaves][R];
  __shared__ int s_idx[kWaves][R];
  if ((lane & 15) == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * kb + r;
        s_val[wave][row] = best[mt][r];
        s_idx[wave][row] = bidx[mt][r];
      }
  }
  __syncthreads();
  const int nblocks = gridDim.x * gridDim.y;
  const int bid = mblk * nvb + vbk;
  if (threadIdx.x < R) {
    float v = s_val[0][threadIdx.x];
    int i = s_idx[0][threadIdx.x];
    for (int w = 1; w < kWaves; ++w)
      if (better(s_val[w][threadIdx.x], s_idx[w][threadIdx.x], v, i)) {
        v = s_val[w][threadIdx.x];
        i = s_idx[w][threadIdx.x];
      }
    // partials: [mblock][vblock][R]
    st_agent(pval + (size_t)bid * R + threadIdx.x, v);
    st_agent(pidx + (size_t)bid * R + threadIdx.x, i);
  }
  if (!arrive_last(ticket, (unsigned)nblocks)) return;

  // ---- last block: merge every block's partials, row by row (one wave per row)
  for (int m = wave; m < a.M; m += kWaves) {
    const int my = m / R, row = m % R;
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (int vb = lane; vb < nvb; vb += 64) {
      const size_t o = ((size_t)my * nvb + vb) * R + row;
      const float ov = ld_agent(pval + o);
      const int oi = ld_agent(pidx + o);
      if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) shfl_best(v, i, mask);
    if (lane == 0) {
      a.target_ids[m] = i;
      if (a.max_logits) a.max_logits[m] = v;
    }
  }

  if (a.B > 0) {
    __threadfence();
    __syncthreads();
    const int k = a.K;
    for (int b = threadIdx.x; b < a.B; b += kThreads) {
      const int32_t* t = a.target_ids + (size_t)b * (k + 1);
      const int32_t* d = a.draft_ids + (size_t)b * k;
      int acc = 0;
      while (acc < k) {
        const int dv = d[acc];
        if (dv < 0 || dv >= a.V || dv != t[acc]) break;
        ++acc;
      }
      a.accepted_len[b] = acc;
      int32_t* o = a.out_tokens + (size_t)b * (k + 1);
      for (int j = 0; j <= k; ++j) o[j] = (j <= acc) ? t[j] : -1;
    }
  }
}

template <int MT, int TILES, int WH, int NW>
void launch_h(const LmheadArgs& a, const LmheadPlan& p, unsigned* ticket, float* pval, int* pidx,
              hipStream_t stream) {
  // grid axes as the kernel reads them (x = vocabulary shares for eight waves)
  const dim3 grid = NW == 8 ? dim3(p.vblocks, p.mblocks) : dim3(p.mblocks, p.vblocks);
  if (a.f16)
    hipLaunchKernelGGL((lmhead_argmax_kernel<MT, TILES, 3, 1, WH, NW>), grid, dim3(64 * NW), 0,
                       stream, a, ticket, pval, pidx);
  else
    hipLaunchKernelGGL((lmhead_argmax_kernel<MT, TILES, 3, 0, WH, NW>), grid, dim3(64 * NW), 0,
                       stream, a, ticket, pval, pidx);
}

template <int MT, int TILES>
void launch_t(const LmheadArgs& a, const LmheadPlan& p, unsigned* ticket, float* pval, int* pidx,
              hipStream_t stream) {
  if constexpr (MT == 1) {
    if (a.H <= kWholeH) {
      launch_h<1, TILES, 1, 4>(a, p, ticket, pval, pidx, stream);
      return;
    }
  }
  if constexpr (MT == 6) {
    if (p.waves == 8) {
      launch_h<6, TILES, 0, 8>(a, p, ticket, pval, pidx, stream);
      return;
    }
  }
  launch_h<MT, TILES, 0, 4>(a, p, ticket, pval, pidx, stream);
}

}  // namespace

LmheadPlan plan_lmhead(int M, int H, int V, int num_cus) {
  (void)H;
  LmheadPlan p{};
  // rows per block: 16, 32, 64, then 96 (a batched verify block of 8 x 21 rows
  // takes two blocks of 96 per vocabulary share; measured on MI355X at M = 168:
  // 299 us against 344 us with 64-row blocks and 454 us with 32-row blocks,
  // all with four waves per block)
  p.mt = (M <= 16) ? 1 : (M <= 32 ? 2 : (M <= 64 ? 4 : 6));
  p.mblocks = (M + 16 * p.mt - 1) / (16 * p.mt);
  // 32 rows per wave pass when the vocabulary fills the chip, else 16 (two
  // tiles measured best on MI355X for the 151,936-row head; the ring depth,
  // 3 to 8 steps, made no difference); the vocabulary is shared equally
  // among one block per CU
  p.tiles = ((long)V >= 32L * 4 * num_cus) ? 2 : 1;
  p.depth = 3;
  // two 96-row blocks: eight waves each (256 vocabulary rows per pass, so the
  // hidden chunk that each step loads whole serves twice as many weight
  // rows), one block per CU: 257 against 301 us at M = 168 on MI355X
  p.waves = (p.mt == 6 && p.mblocks == 2) ? 8 : 4;
  const int rows_per_pass = p.waves * p.tiles * 16;
  const int npasses = (V + rows_per_pass - 1) / rows_per_pass;
  const int per_cu = p.waves == 8 ? num_cus / p.mblocks : kLmheadBlocksPerCU * num_cus;
  p.vblocks = npasses < per_cu ? npasses : per_cu;
  const size_t nblocks = (size_t)p.vblocks * p.mblocks;
  p.ticket_bytes = kTicketRegion;
  p.partial_bytes = align_up(nblocks * 16 * p.mt * sizeof(float), kWorkspaceAlign) +
                    nblocks * 16 * p.mt * sizeof(int);
  return p;
}

hipError_t launch_lmhead_argmax(const LmheadArgs& a, const LmheadPlan& p, void* workspace,
                                hipStream_t stream) {
  unsigned* ticket = static_cast<unsigned*>(workspace);
  char* base = static_cast<char*>(workspace) + p.ticket_bytes;
  const size_t nblocks = (size_t)p.vblocks * p.mblocks;
  float* pval = reinterpret_cast<float*>(base);
  int* pidx = reinterpret_cast<int*>(base + align_up(nblocks * 16 * p.mt * sizeof(float),
                                                     kWorkspaceAlign));
  if (p.depth != 3 || (p.tiles != 1 && p.tiles != 2) || (p.waves != 4 && p.waves != 8) ||
      (p.waves == 8 && p.mt != 6))
    return hipErrorInvalidValue;
  if (p.mt == 1) {
    if (p.tiles == 2) launch_t<1, 2>(a, p, ticket, pval, pidx, stream);
    else launch_t<1, 1>(a, p, ticket, pval, pidx, stream);
  } else if (p.mt == 2) {
    if (p.tiles == 2) launch_t<2, 2>(a, p, ticket, pval, pidx, stream);
    else launch_t<2, 1>(a, p, ticket, pval, pidx, stream);
  } else if (p.mt == 4) {
    if (p.tiles == 2) launch_t<4, 2>(a, p, ticket, pval, pidx, stream);
    else launch_t<4, 1>(a, p, ticket, pval, pidx, stream);
  } else {
    if (p.tiles == 2) launch_t<6, 2>(a, p, ticket, pval, pidx, stream);
    else launch_t<6, 1>(a, p, ticket, pval, pidx, stream);
  }
  return hipGetLastError();
}

}  // namespace w4v
