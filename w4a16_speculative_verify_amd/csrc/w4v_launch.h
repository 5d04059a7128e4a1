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
};

struct GemmPlan {
  int mt;            // 16-row m-tiles per block (1 or 2)
  int mblocks;       // blocks along M, each 16*mt rows
  int tiles;         // ceil(N / 64)
  int wt;            // 64-column tiles per block (1 or 2)
  int wk;            // k-slices per block (4)
  int col_blocks;    // ceil(tiles / wt)
  int splits;        // split-K factor across blocks (1 = none)
  int depth;         // groups in flight per wave (3)
  size_t ticket_bytes;
  size_t partial_bytes;
  size_t workspace_bytes() const { return ticket_bytes + partial_bytes; }
};

GemmPlan plan_w4a16(int M, int N, int K, int num_cus);
hipError_t launch_w4a16_skinny(const GemmArgs& a, const GemmPlan& p, void* workspace,
                               hipStream_t stream);
// LDS-tiled MFMA GEMM for M > 32 rows (no workspace)
hipError_t launch_w4a16_tiled(const GemmArgs& a, hipStream_t stream);
constexpr int kTiledMinRows = 33;

// From this many rows on, with a workspace: weights dequantised to a
// transposed fp16 copy in the workspace, then a plain fp16 GEMM from the
// vendor library (without a workspace: the LDS-tiled kernel).
constexpr int kLibMinRows = 33;
constexpr size_t kLibWorkspace = 64ull << 20;   // the library GEMM's own scratch
hipError_t launch_dequant_w4_f16t(const uint32_t* qweight, const _Float16* scales,
                                  const uint32_t* qzeros, int K, int N, int group_size,
                                  _Float16* wt, hipStream_t stream);
// y = alpha * x @ wt^T through the library (wt: fp16 [N x K], row stride
// ldw); false if the library has no plan for the shape or reports an error
// before launching.
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
  size_t ticket_bytes;
  size_t partial_bytes;
  size_t workspace_bytes() const { return ticket_bytes + partial_bytes; }
};

LmheadPlan plan_lmhead(int M, int H, int V, int num_cus);
hipError_t launch_lmhead_argmax(const LmheadArgs& a, const LmheadPlan& p, void* workspace,
                                hipStream_t stream);

// ---------------------------------------------------------------- chain of linears
constexpr unsigned kChainMagic = 0x37435734u;   // "4WC7"
constexpr int kChainComputeWaves = 4;           // tiles x k-slices of a unit
constexpr int kChainThreads = 64 * (kChainComputeWaves + 1);   // + one control wave
constexpr int kChainMaxGroups = 24;             // 128-k groups of one unit's activation slice (LDS)
constexpr int kChainMaxRows = 16;
constexpr size_t kChainSlot = 256;              // bytes per ticket (one cache line or more)

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
  unsigned pad0[2];
  uint64_t lin_offset;   // byte offset of the ChainLinear table
  uint64_t pad1;
  unsigned pad2[48];
};
static_assert(sizeof(ChainHeader) == 256, "chain header is 256 bytes");

struct ChainLinear {
  const uint32_t* qweight;
  const _Float16* scales;
  const uint32_t* qzeros;
  _Float16* out;         // fp16 [16][ldo] (NULL for the last linear)
  float* partials;       // fp32 [splits][16][cb * wt * 64] when splits > 1
  unsigned* tickets;     // [cb * wt] split arrivals per tile, one 256-byte slot each
  unsigned* flags;       // [ceil(N / 64)] tile ready flags (epoch + 1 once written)
  int K, N, ldo, splits;
  int cb;                // column blocks of wt tiles
  int units;             // cb * splits <= blocks: one unit per block
  float alpha;
  int wt;                // 64-column tiles per block (1, 2 or 4); 4 / wt k-slices
};
static_assert(sizeof(ChainLinear) == 88, "chain linear descriptor is 88 bytes");

struct ChainLayout {
  size_t bytes;          // total workspace bytes
  size_t lin_offset;
  size_t counters_offset;   // tickets and ready flags, zeroed by prepare
  size_t buffers_offset;    // outputs and partials
};

hipError_t launch_w4a16_chain(ChainHeader* hdr, const _Float16* x, int64_t ldx, _Float16* y,
                              int64_t ldy, int M, int K0, int N_last, int blocks,
                              hipStream_t stream);

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
hipError_t launch_greedy_verify(const int32_t* target_ids, const int32_t* draft_ids, int B, int K,
                                int V, int32_t* accepted_len, int32_t* out_tokens,
                                hipStream_t stream);

}  // namespace w4v
