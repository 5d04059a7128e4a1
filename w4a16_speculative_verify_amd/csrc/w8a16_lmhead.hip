// 8-bit lm_head with fused greedy argmax, optionally followed by the greedy
// prefix acceptance, gfx950 (section 3 of the organisers' results page:
// untied lm_head quantised to 8 bits, temperature-0 verification).
//
// Work decomposition
//   wave pass = TILES x 16 vocabulary rows over the whole hidden width H.
//     Lane l streams 32 consecutive bytes (k = 128*chunk + 32*(l/16) ..) of
//     row v0 + 16*t + l%16 per 128-k chunk: two 128-bit loads per tile.  Each
//     8-byte slice is the B operand of one 16x16x32 MFMA; the matching A slice
//     is the same 8 k of the hidden rows, read from global memory (L2).
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ void shfl_best(float& v, int& i, int mask) {
  const float ov = __shfl_xor(v, mask, 64);
  const int oi = __shfl_xor(i, mask, 64);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

template <int MT, int TILES>
__global__ __launch_bounds__(kThreads) void lmhead_argmax_kernel(LmheadArgs a, unsigned* ticket,
                                                                 float* pval, int* pidx) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kb = lane >> 4;
  const int mbase = blockIdx.y * 16 * MT;
  const int nvb = gridDim.x;
  const int rows_per_pass = kWaves * TILES * 16;
  const int npasses = (a.V + rows_per_pass - 1) / rows_per_pass;
  const int nchunks = a.H / 128;

  float best[MT][4];
  int bidx[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      best[mt][r] = -INFINITY;
      bidx[mt][r] = 0x7fffffff;
    }

  for (int pass = blockIdx.x; pass < npasses; pass += nvb) {
    const int v0 = pass * rows_per_pass + wave * TILES * 16;
    if (v0 >= a.V) break;      // waves past the vocabulary end have nothing to do
    f32x4 acc[MT][TILES];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < TILES; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // rows past the vocabulary end read row 0 (their logits are never compared)
    const int8_t* wrow[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int v = v0 + 16 * t + (lane & 15);
      wrow[t] = a.w + (size_t)(v < a.V ? v : 0) * a.H + kb * 32;
    }
    // hidden rows past M read row mbase and are zeroed at use
    const int m_a = mbase + (lane & 15);
    const _Float16* hrow[MT];
    bool mok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m_a + mt * 16;
      mok[mt] = m < a.M;
      hrow[mt] = a.h + (size_t)(mok[mt] ? m : mbase) * a.ldh + kb * 32;
    }

    // Two-deep software pipeline over 128-k chunks.  Per chunk the hidden
    // rows (L2) are loaded before the next chunk's weights are requested, so
    // waiting for them never waits for the prefetch.
    u32x4 wa[TILES][2], wb[TILES][2];
    auto load_w = [&](u32x4 (&dst)[TILES][2], int ch) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        // plain (cached) loads: each instruction uses half of every 128-byte line
        // it touches and the next instruction the other half, which must still
        // be in the L2 then
        const u32x4* p = reinterpret_cast<const u32x4*>(wrow[t] + ch * 128);
        dst[t][0] = p[0];
        dst[t][1] = p[1];
      }
    };
    auto chunk = [&](const u32x4 (&wv)[TILES][2], int ch, bool prefetch, u32x4 (&nxt)[TILES][2]) {
      u32x4 hv[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4* p = reinterpret_cast<const u32x4*>(hrow[mt] + ch * 128);
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[mt][q] = p[q];
      }
      __builtin_amdgcn_sched_barrier(0);
      if (prefetch) load_w(nxt, ch + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x8 av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          av[mt] = __builtin_bit_cast(f16x8, mok[mt] ? hv[mt][q] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
          const u32x4& src = wv[t][q >> 1];
          const u32x2 d = (q & 1) ? u32x2{src.z, src.w} : u32x2{src.x, src.y};
          const f16x8 b = dequant_int8_x8(d);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][t] = mfma16x16x32(av[mt], b, acc[mt][t]);
        }
      }
    };
    load_w(wa, 0);
    for (int ch = 0; ch < nchunks; ch += 2) {
      chunk(wa, ch, ch + 1 < nchunks, wb);
      if (ch + 1 < nchunks) chunk(wb, ch + 1, ch + 2 < nchunks, wa);
    }

#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int v = v0 + 16 * t + (lane & 15);
      if (v < a.V) {
        const float s = (float)a.scales[v];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lg = s * acc[mt][t][r];
            if (lg > best[mt][r]) {
              best[mt][r] = lg;
              bidx[mt][r] = v;
            }
          }
      }
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
  const int bid = blockIdx.y * gridDim.x + blockIdx.x;
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

template <int MT, int TILES>
void launch_t(const LmheadArgs& a, const LmheadPlan& p, unsigned* ticket, float* pval, int* pidx,
              hipStream_t stream) {
  hipLaunchKernelGGL((lmhead_argmax_kernel<MT, TILES>), dim3(p.vblocks, p.mblocks),
                     dim3(kThreads), 0, stream, a, ticket, pval, pidx);
}

}  // namespace

LmheadPlan plan_lmhead(int M, int H, int V, int num_cus) {
  (void)H;
  LmheadPlan p{};
  p.mt = (M <= 16) ? 1 : 2;
  p.mblocks = (M + 16 * p.mt - 1) / (16 * p.mt);
  // 64 rows per wave pass when the vocabulary fills the chip, else 16
  p.tiles = ((long)V >= 64L * 4 * num_cus) ? 4 : 1;
  const int rows_per_pass = kWaves * p.tiles * 16;
  const int npasses = (V + rows_per_pass - 1) / rows_per_pass;
  p.vblocks = npasses < 4 * num_cus ? npasses : 4 * num_cus;
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
  if (p.mt == 1) {
    if (p.tiles == 4) launch_t<1, 4>(a, p, ticket, pval, pidx, stream);
    else launch_t<1, 1>(a, p, ticket, pval, pidx, stream);
  } else {
    if (p.tiles == 4) launch_t<2, 4>(a, p, ticket, pval, pidx, stream);
    else launch_t<2, 1>(a, p, ticket, pval, pidx, stream);
  }
  return hipGetLastError();
}

}  // namespace w4v
