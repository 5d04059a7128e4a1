// Host-side launch plans and launchers of libw4v (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4v {

constexpr int kGroup = 128;        // quantisation group along k
constexpr int kColTile = 64;       // output columns per wave (4 per lane x 16 lanes)
constexpr int kWorkspaceAlign = 256;

// Every workspace that needs arrival counters starts with this fixed counter
// region (one 32-bit counter per output tile, each in a 256-byte slot of its
// own: counters that share a cache line serialise their atomics at the
// memory side); partial results follow it.  Because the counters sit at the
// same place for every shape and every kernel leaves them at zero, calls of
// different shapes may share one workspace as long as they are ordered on
// one stream.
constexpr size_t kTicketRegion = 64 * 1024;
// Split-K partials of the skinny linear follow the counter prefix and never
// exceed this many bytes (the plan keeps them within it); other paths place
// their data after it.
constexpr size_t kPartialRegion = 4u << 20;
constexpr size_t kTicketStride = 64;            // 32-bit words between two counters
constexpr size_t kMaxTickets = kTicketRegion / (kTicketStride * sizeof(unsigned));

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- W4A16 GEMM
struct GemmArgs {
  const _Float16* x; int64_t ldx;
  const uint32_t* qweight; const _Float16* scales; const uint32_t* qzeros;
  _Float16* y; int64_t ldy;
  int M, N, K;
  float alpha;
  int group_size;    // 128, or 32 (four quantisation groups per 128-k step)
  int xcd_local;     // set by the launcher: blocks with ids equal mod 8 share an XCD
};

struct GemmPlan {
  int mt;            // 16-row m-tiles per block (1 or 2)
  int mblocks;       // blocks along M, each 16*mt rows
  int tiles;         // ceil(N / 64)
  int wt;            // 64-column tiles per block (1 or 2)
  int wk;            // k-slices per block (4)
  int col_blocks;    // ceil(tiles / wt)
  int splits;        // split-K factor across blocks (1 = none)
  int depth;         // groups in flight per wave (2)
  size_t ticket_bytes;
  size_t partial_bytes;
  size_t workspace_bytes() const { return ticket_bytes + partial_bytes; }
};

GemmPlan plan_w4a16(int M, int N, int K, int num_cus);
hipError_t launch_w4a16_skinny(const GemmArgs& a, const GemmPlan& p, void* workspace,
                               hipStream_t stream, bool may_probe = true);

// From this many rows on: the LDS-tiled MFMA kernel (weights dequantised once
// per 256 x 256 block tile into LDS), split-K with fp32 partials in the
// workspace for shapes with few tiles
constexpr int kMfmaMinRows = 33;
struct MfmaPlan {
  int mtw;               // 16-row m-tiles per wave: block tiles of 32 mtw rows x 256 columns
  int mblocks, nblocks;
  int dp;                // tiles computed whole (the first dp of the raster order)
  int ntail;             // tiles after them, each split `splits` ways (0 when splits == 1)
  int splits;            // K-splits of the tail tiles (1 = none)
  size_t partial_bytes;  // fp32 [splits][ntail][32 mtw x 256] when splits > 1
};
MfmaPlan plan_w4a16_mfma(int M, int N, int K, int num_cus);
hipError_t launch_w4a16_mfma(const GemmArgs& a, const MfmaPlan& p, float* partials,
                             hipStream_t stream);

// y = alpha * x @ wt^T through the vendor library (wt: fp16 [N x K], row
// stride ldw); false if the library has no plan for the shape or reports an
// error before launching (the fp16 linear only)
constexpr size_t kLibWorkspace = 64ull << 20;   // the library GEMM's own scratch
bool lib_gemm_f16_tn(const _Float16* x, int64_t ldx, const _Float16* wt, int64_t ldw, _Float16* y,
                     int64_t ldy, int M, int N, int K, float alpha, void* scratch,
                     size_t scratch_bytes, hipStream_t stream);

// ---------------------------------------------------------------- lm_head
struct LmheadArgs {
  const _Float16* h; int64_t ldh;
  const void* w;         // int8 [V x H] with fp16 scales [V], or fp16 [V x H] (scales NULL)
  const _Float16* scales;
  int f16;               // 1: fp16 weights, no scales
  int32_t* target_ids; float* max_logits;
  int M, H, V;
  // fused greedy verify (draft_ids may be NULL when K == 0; B == 0 disables it)
  const int32_t* draft_ids; int B, K;
  int32_t* accepted_len; int32_t* out_tokens;
};

struct LmheadPlan {
  int mt;            // 16-row m-tiles per block (1, 2, 4 or 6)
  int mblocks;
  int tiles;         // 16-row vocabulary tiles per wave pass (1 or 2)
  int depth;         // steps in flight per wave (3)
  int vblocks;       // blocks along the vocabulary
  int waves;         // waves per block (4, or 8 for two 96-row blocks)
  size_t ticket_bytes;
  size_t partial_bytes;
  size_t workspace_bytes() const { return ticket_bytes + partial_bytes; }
};

LmheadPlan plan_lmhead(int M, int H, int V, int num_cus);
hipError_t launch_lmhead_argmax(const LmheadArgs& a, const LmheadPlan& p, void* workspace,
                                hipStream_t stream);

// ---------------------------------------------------------------- chain of linears
// One persistent launch for a chain of W4A16 linears at M <= 16 rows.  Each
// block's share of every linear (its "unit": nb 16-column blocks x ng 128-k
// groups) is prepacked, in chain order, into one contiguous byte stream per
// block, which a loader wave copies into an LDS ring ahead of the math.
constexpr unsigned kChainMagic = 0x32435734u;   // "4WC2"
constexpr int kChainComputeWaves = 8;           // two per SIMD
constexpr int kChainThreads = 64 * (kChainComputeWaves + 1);   // + the loader wave
constexpr int kChainRingBytes = 112 * 1024;     // LDS ring of the weight stream (multiple of 1 KiB)
constexpr int kChainMaxNb = 5;                  // 16-column blocks per unit
constexpr int kChainMaxWaveGroups = 3;          // 128-k groups per compute wave (A in registers)
constexpr int kChainMaxRows = 16;
constexpr int kChainMaxFlags = 64;              // input tiles one unit may wait for
constexpr int kChainGroups = 8;                 // blocks dealt round-robin over the XCDs

// bytes of one 128-k group of a unit of nb column blocks in the stream:
// nb x 1 KiB of packed words (lane-ordered), then nb*16 fp16 scales and
// 2*nb zero-point words, padded to 16 bytes
inline constexpr unsigned chain_group_bytes(int nb) {
  return (unsigned)nb * 1024u + (unsigned)((40 * nb + 15) / 16 * 16);
}

// Device-side header at offset 0 of a prepared chain workspace (256 bytes).
struct ChainHeader {
  unsigned magic;
  unsigned n_linears;
  unsigned blocks;       // grid size the plan was made for (one block per CU)
  unsigned M;
  unsigned epoch;        // launches completed: launch e raises flags to e + 1
  unsigned abort;        // a launch gave up a wait: results invalid until prepared again
  unsigned exit_count;   // blocks that finished the current launch (re-armed by the last)
  unsigned error;        // byte offset 28: 1 a wait timed out, 2 workspace not prepared for this call
  unsigned K0;           // width of the input rows
  unsigned N_last;       // width of the output rows
  unsigned groups;       // block groups (kChainGroups, or 1)
  unsigned group_blocks; // blocks per group
  uint64_t lin_offset;   // byte offsets of the tables below
  uint64_t unit_offset;
  uint64_t stream_offset;
  uint64_t xcc_offset;
  unsigned pad[44];
};
static_assert(sizeof(ChainHeader) == 256, "chain header is 256 bytes");

struct ChainLinear {
  _Float16* out;         // fp16 [16][ld_out] (NULL for the last linear)
  unsigned* flags;       // [tiles] output tile ready flags (epoch + 1 once written)
  unsigned* sflags;      // [tiles][S] split partial ready flags (S > 1)
  float* partials;       // per tile [S - 1][16][cols of the tile] fp32 (S > 1)
  int K, N, ld_out;
  float alpha;
  int S, tiles, pad0, pad1;
};
static_assert(sizeof(ChainLinear) == 64, "chain linear descriptor is 64 bytes");

struct ChainUnit {       // block b's share of linear l
  int col0;              // first output column (-1: no unit)
  int nb;                // 16-column blocks
  int g0, ng;            // 128-k groups
  int split, S;          // K-split index and count of the unit's tile
  int tile;              // tile index in the linear (flags, tickets, partials)
  int f0, nf;            // input tiles of the previous linear this unit reads
  unsigned soff;         // byte offset of the unit's data in the block's stream
  int part_off;          // float offset of the tile's partials (S > 1)
  unsigned gbytes;       // stream bytes per group (chain_group_bytes(nb))
};
static_assert(sizeof(ChainUnit) == 48, "chain unit descriptor is 48 bytes");

struct ChainStream {     // block b's weight stream in the workspace
  uint64_t offset;       // byte offset from the workspace start (1 KiB aligned)
  unsigned kb;           // length in KiB
  unsigned pad;
};
static_assert(sizeof(ChainStream) == 16, "chain stream descriptor is 16 bytes");

hipError_t launch_w4a16_chain(ChainHeader* hdr, const _Float16* x, int64_t ldx, _Float16* y,
                              int64_t ldy, int M, int K0, int N_last, int blocks,
                              hipStream_t stream);
// copies linear l's weights into the blocks' streams (grid: blocks x max groups per unit)
hipError_t launch_w4a16_chain_prepack(const ChainUnit* units, const ChainStream* streams,
                                      int blocks, int max_ng, const uint32_t* qweight,
                                      const _Float16* scales, const uint32_t* qzeros, int N,
                                      char* ws, hipStream_t stream);

// ---------------------------------------------------------------- drafting
constexpr int kNgramMaxN = 64;
hipError_t launch_ngram_draft(const int32_t* history, int64_t ld, const int32_t* lengths, int B,
                              int n_max, int n_min, int K, int32_t* drafts, hipStream_t stream);
hipError_t launch_append_accepted(int32_t* history, int64_t ld, int32_t* lengths, int B, int K,
                                  const int32_t* out_tokens, const int32_t* accepted_len,
                                  hipStream_t stream);

// ---------------------------------------------------------------- recurrent state commit
constexpr int kGdnMaxT = 32;      // positions of a verify block (K + 1) the commit stages
hipError_t launch_gdn_commit(float* state, const float* k, const float* v, const float* alpha,
                             const float* beta, const int32_t* accepted_len, int B, int T, int H,
                             int D, hipStream_t stream);

// ---------------------------------------------------------------- verify
// HBM read-bandwidth probe: kReadProbeBlocks blocks, one XOR word each in out
constexpr int kReadProbeBlocks = 2048;
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* out, hipStream_t stream);

hipError_t launch_greedy_verify(const int32_t* target_ids, const int32_t* draft_ids, int B, int K,
                                int V, int32_t* accepted_len, int32_t* out_tokens,
                                hipStream_t stream);

}  // namespace w4v
