/*
 * w4v.h -- C ABI of the W4A16 speculative-verify library (libw4v.so, gfx950).
 *
 * The operations follow the organisers' page "Efficient LLM Challenge
 * Results" (adaptfm.gitlab.io/competition-results), section 3: a drafter
 * proposes K tokens, one forward pass of the target over the K+1 positions
 * checks them all, and the drafts are kept up to the first one that differs
 * from the target's greedy token; the winning target is W4A16 GPTQ with group
 * size 128 and an untied lm_head quantised to 8 bits, served greedily; the
 * runner-up fills every draft up to a constant K=20 with -1, which can never
 * equal a greedy token.  Section 5 names the W8A16 lm_head.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises on these calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous and ordered on that stream.
 *   - Arguments are validated on the host before any HIP call; a failure
 *     returns a negative w4v_status and launches nothing.  A launch error
 *     returns W4V_ERR_HIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation.  No C++ exception crosses this interface.
 *   - fp16 means IEEE binary16; row-major everywhere; leading dimensions
 *     (ld*) are in elements.
 *   - Workspaces: size them with the *_workspace_size query and zero them
 *     ONCE after allocation.  Kernels leave their counters at zero when they
 *     finish, and the counters sit at the same offset for every call, so one
 *     workspace sized for the largest call may be shared by calls of any
 *     shape that are ordered on one stream.  Calls that overlap in time must
 *     not share a workspace.  After a kernel fault, zero the workspace again.
 */
#ifndef W4V_H
#define W4V_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4V_ABI_VERSION 1

typedef enum {
  W4V_OK = 0,
  W4V_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad stride           */
  W4V_ERR_UNSUPPORTED = -2,   /* valid request this build does not implement  */
  W4V_ERR_ALIGNMENT = -3,     /* pointer or stride breaks a stated alignment  */
  W4V_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required   */
  W4V_ERR_HIP = -5            /* the HIP runtime reported an error            */
} w4v_status;

/* Static English text for a status code (never NULL). */
const char* w4v_status_string(int status);

/* W4V_ABI_VERSION of the built library. */
int w4v_abi_version(void);

/* ------------------------------------------------------------------------
 * HBM read-bandwidth probe (a measurement helper, not a step of the verify
 * path; the measurement method of the hot path asks for the read bandwidth
 * the device actually reaches, reported beside the 8 TB/s peak).
 * Reads `bytes` of device memory at `src` once (16-byte non-temporal loads)
 * and writes one 32-bit XOR per block of what it read to `out`, so that the
 * loads are not dropped; timing the call gives the read rate.
 *   src    device, 16-byte aligned; bytes > 0, a multiple of 16.
 *   out    device, w4v_read_probe_blocks() words, caller-owned.
 * Enqueued on `stream`; returns W4V_ERR_INVALID_ARG (null, bad size),
 * W4V_ERR_ALIGNMENT or W4V_ERR_HIP.
 */
int w4v_read_probe_blocks(void);
int w4v_read_probe(const void* src, size_t bytes, uint32_t* out, void* stream);

/* ------------------------------------------------------------------------
 * W4A16 linear (section 3: 4-bit weights, group size 128, 16-bit activations;
 * section 5: group size 32 for team #5's compressed-tensors target)
 *
 *   y[m, n] = fp16_rne( alpha * sum_k x[m, k] * s[k/g, n] * (q[k, n] - z[k/g, n]) ),
 *   g = group_size
 *
 * x        fp16  [M x K], row stride ldx >= K; 16-byte aligned, ldx % 8 == 0.
 * qweight  int32 [K/8 x N]: nibble j (bits 4j..4j+3) of word (i, n) is
 *          q[8i + j][n], an unsigned 4-bit value; 16-byte aligned.
 * scales   fp16  [K/group_size x N]; 16-byte aligned.
 * qzeros   int32 [K/group_size x N/8]: nibble j of word (g, i) is z[g][8i + j];
 *          4-byte aligned.
 * y        fp16  [M x N] out, row stride ldy >= N; 16-byte aligned, ldy % 8 == 0.
 *          y must not overlap x.
 * Sizes    M >= 0 (M == 0 or N == 0: nothing to do, W4V_OK), K > 0,
 *          N % 8 == 0, K % group_size == 0; group_size must be 128 or 32,
 *          and K % 128 == 0 for both (W4V_ERR_UNSUPPORTED otherwise: the
 *          kernels step 128 k at a time).  The packed weights (K*N/2 bytes),
 *          the scales and the rows of x (M*ldx*2 bytes) must each stay below
 *          2 GiB (W4V_ERR_UNSUPPORTED otherwise).
 * alpha    epilogue scale applied to the fp32 accumulator before the single
 *          round-to-nearest-even to fp16.
 * Paths    M <= 32: weights dequantised exactly in registers, each group's
 *          scale applied to that group's fp32 sum (split-K across blocks).
 *          M >= 33 (the batched verify block, prefill shapes: bound by the
 *          matrix cores): an LDS-tiled MFMA kernel that dequantises each
 *          256-column x 32-k weight tile once per block tile of 256 rows (128
 *          or 192 for calls with no more rows), as w = fp16_rne(s * (q - z))
 *          (q - z exact, one rounding; the fp32 accumulation and the alpha /
 *          output rounding as above); shapes with fewer block tiles than CUs
 *          are split along K, and with more, the tiles of the last partial
 *          round are, with fp32 partials in the workspace added in split
 *          order by a second kernel.  The plan (and so the result) depends on
 *          the shape alone.
 * workspace  device memory of at least w4a16_gemm_workspace_size(M, N, K,
 *          group_size) bytes (may be NULL when that size is 0), 256-byte
 *          aligned, zeroed once by the caller.  Its first 64 KiB hold the
 *          split-K arrival counters of the M <= 32 path (every call leaves them
 *          at zero), the next 4 MiB at most that path's fp32 partial sums; the
 *          M >= 33 path's fp32 partials [splits x split tiles x tile rows x
 *          256] come after those 4 MiB.  A workspace smaller than the query's size (NULL included)
 *          returns W4V_ERR_WORKSPACE.  Partials are added in split order, so
 *          the result does not depend on the order in which they arrive.  One
 *          workspace sized for the largest call serves calls of every shape
 *          ordered on one stream.
 * Placement  the first M <= 32 call with a K-split on a device, outside
 *          stream capture, enqueues on `stream` a small probe of how the
 *          device deals blocks to its XCDs (with a copy of its one-word result
 *          to pinned host memory and an event; nothing waits for them); when a
 *          later call outside capture finds the probe done and blocks whose
 *          ids agree mod 8 share an XCD, it and later calls pass the split-K
 *          partials with plain stores and L1-missing loads instead of
 *          device-coherent (sc1) ones, valid because every split of a tile
 *          then runs on one XCD (same result bits either way).
 * ---------------------------------------------------------------------- */
size_t w4a16_gemm_workspace_size(int M, int N, int K, int group_size);

int w4a16_gemm(const void* x, int64_t ldx,
               const int32_t* qweight, const void* scales, const int32_t* qzeros,
               void* y, int64_t ldy,
               int M, int N, int K, int group_size, float alpha,
               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * W4A16 linear that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results (bit for bit) and launch plan as w4a16_gemm, minus
 * the workspace: the scratch a plan needs lives in a device array of
 * W4V_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  A shape whose w4a16_gemm_workspace_size exceeds
 * that returns W4V_ERR_UNSUPPORTED before any launch.  The first calls on a
 * device clear the array's ticket region with a small kernel on `stream`
 * (also when captured); the kernels re-arm it after every call.
 * Calls on one GPU share the array: two calls whose executions overlap on
 * one GPU (different streams, or graphs replayed concurrently) race, so
 * order them on one stream.  Never calls hipMalloc, hipFree or any other
 * allocating routine: it never starts the XCD placement probe (whose result
 * word is pinned host memory), and keeps the split-K hand-off on the memory
 * side until a w4a16_gemm call's probe result is known.
 * ---------------------------------------------------------------------- */
#define W4V_STATIC_SCRATCH_BYTES (32u << 20)

int w4a16_gemm_noalloc(const void* x, int64_t ldx,
                       const int32_t* qweight, const void* scales, const int32_t* qzeros,
                       void* y, int64_t ldy,
                       int M, int N, int K, int group_size, float alpha, void* stream);

/* ------------------------------------------------------------------------
 * 8-bit lm_head with fused greedy argmax (section 3: untied lm_head
 * quantised to 8 bits, temperature-0 serving; section 5: W8A16 lm_head)
 *
 *   logit[m, v]   = float(s8[v]) * sum_h h[m, h] * q8[v, h]     (fp32, never stored)
 *   target_ids[m] = the lowest v with the largest logit[m, v]
 *
 * h          fp16 [M x H], row stride ldh >= H; 16-byte aligned, ldh % 8 == 0.
 * w          int8 [V x H] row-major, one vocabulary row per output; 16-byte
 *            aligned.  Symmetric: no zero-point.  Any int8 value is accepted.
 * scales     fp16 [V], one scale per vocabulary row.
 * target_ids int32 [M] out.
 * max_logits fp32 [M] out (the winning logit), or NULL.
 * Sizes      M >= 0 (0: nothing to do), V > 0, H > 0 and H % 128 == 0;
 *            V*H bytes of weights and M*ldh*2 bytes of h below 2 GiB
 *            (W4V_ERR_UNSUPPORTED otherwise).
 * workspace  at least w8a16_lmhead_argmax_workspace_size(M, H, V) bytes,
 *            256-byte aligned, zeroed once.  Holds per-block (value, index)
 *            partials and an arrival counter.
 * ---------------------------------------------------------------------- */
size_t w8a16_lmhead_argmax_workspace_size(int M, int H, int V);

int w8a16_lmhead_argmax(const void* h, int64_t ldh,
                        const int8_t* w, const void* scales,
                        int32_t* target_ids, float* max_logits,
                        int M, int H, int V,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Greedy prefix acceptance (section 3)
 *
 * For each sequence b (rows b*(K+1) + j of target_ids, j = 0..K, row j being
 * the target's greedy token after drafts 0..j-1):
 *   accepted_len[b] = the number of leading drafts equal to their target
 *                     token; the scan stops at the first mismatch.  A draft
 *                     outside [0, V) -- the -1 sentinel included -- never
 *                     matches (not an error).
 *   out_tokens[b]   = target_ids[b][0 .. a_b] (the accepted drafts and the
 *                     target's bonus token), then -1 up to K+1 entries.
 *
 * target_ids   int32 [B x (K+1)], values in [0, V).
 * draft_ids    int32 [B x K] (may be NULL when K == 0).
 * accepted_len int32 [B] out;  out_tokens int32 [B x (K+1)] out.
 * Sizes        B >= 0 (0: nothing to do), K >= 0, V > 0.
 * ---------------------------------------------------------------------- */
int greedy_verify(const int32_t* target_ids, const int32_t* draft_ids,
                  int B, int K, int V,
                  int32_t* accepted_len, int32_t* out_tokens, void* stream);

/* ------------------------------------------------------------------------
 * lm_head + argmax + greedy acceptance in one launch: the block that reduces
 * the last argmax partials also runs the prefix scan, so the verify step's
 * tail needs no extra kernel.  Same arguments and results as
 * w8a16_lmhead_argmax followed by greedy_verify with M = B * (K + 1);
 * the same workspace size as w8a16_lmhead_argmax.
 * ---------------------------------------------------------------------- */
int w8a16_lmhead_argmax_verify(const void* h, int64_t ldh,
                               const int8_t* w, const void* scales,
                               int32_t* target_ids, float* max_logits,
                               int H, int V,
                               const int32_t* draft_ids, int B, int K,
                               int32_t* accepted_len, int32_t* out_tokens,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Half-precision parts of a partly quantised target (section 5: team #5
 * serves a W4A16 group-size-32 target that keeps its first two and last two
 * layers and its lm_head in fp16).
 *
 * fp16 lm_head with fused greedy argmax, optionally the greedy verify:
 *   logit[m, v] = sum_h h[m, h] * w[v, h]  (fp32, never stored);
 *   target_ids[m] = argmax_v logit[m, v], ties -> lowest v.
 * w        fp16 [V x H] row-major (one vocabulary row per output), 16-byte
 *          aligned; V * H * 2 bytes below 2 GiB (W4V_ERR_UNSUPPORTED).
 * h, target_ids, max_logits, M, H, workspace: as for w8a16_lmhead_argmax
 *          (same workspace size: f16_lmhead_argmax_workspace_size).
 * B == 0   argmax only (draft_ids, accepted_len, out_tokens ignored).
 * B > 0    M must equal B * (K + 1) (W4V_ERR_INVALID_ARG otherwise); then the
 *          greedy prefix acceptance of w8a16_lmhead_argmax_verify runs in the
 *          same launch.
 * ---------------------------------------------------------------------- */
size_t f16_lmhead_argmax_workspace_size(int M, int H, int V);

int f16_lmhead_argmax_verify(const void* h, int64_t ldh, const void* w,
                             int32_t* target_ids, float* max_logits, int M, int H, int V,
                             const int32_t* draft_ids, int B, int K,
                             int32_t* accepted_len, int32_t* out_tokens,
                             void* workspace, size_t workspace_bytes, void* stream);

/* fp16 linear: y[m, n] = fp16_rne( alpha * sum_k x[m, k] * w[n, k] ), fp32
 * accumulation, computed by the vendor library's plain fp16 GEMM.
 * x        fp16 [M x K], row stride ldx >= K; w fp16 [N x K] (one row per
 *          output, the layout of a dense layer), row stride ldw >= K;
 *          y fp16 [M x N] out, row stride ldy >= N.  All 16-byte aligned,
 *          strides multiples of 8; y must overlap neither x nor w.
 * workspace  f16_gemm_workspace_size(M, N, K) bytes, 256-byte aligned: the
 *          library GEMM's scratch after the first 64 KiB + 4 MiB, which are
 *          left alone (the split-K counters and partials of w4a16_gemm), so
 *          one workspace serves both kinds of linear on a stream.
 * Errors   W4V_ERR_UNSUPPORTED when the library has no plan for the shape
 *          or fails before launching; there is no other path.
 * ---------------------------------------------------------------------- */
size_t f16_gemm_workspace_size(int M, int N, int K);

int f16_gemm(const void* x, int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
             int M, int N, int K, float alpha, void* workspace, size_t workspace_bytes,
             void* stream);

/* ------------------------------------------------------------------------
 * Committing a Gated DeltaNet state to the verify's accepted prefix (results
 * page, hazards list: rejected drafts corrupted the recurrent state of the
 * target's Gated DeltaNet layers; section 3: the runner-up's constant-K fix).
 * The state committed before the verify block is advanced by exactly the
 * accepted positions -- position 0 (the last committed token) and the a_b
 * accepted drafts -- a_b + 1 steps of the gated delta rule:
 *   S <- alpha_t * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 * Rejected positions are never applied.
 * state    fp32 [B x H x D x D] in/out (S[b, h] is [dv x dk] row-major),
 *          16-byte aligned.  H counts heads over all layers committed together.
 * k, v     fp32 [B x T x H x D]: the block's keys (unit length in the layer)
 *          and values at positions 0 .. T-1; 4-byte aligned; must not overlap
 *          the state.
 * alpha, beta  fp32 [B x T x H]: decay gate and write strength.
 * accepted_len int32 [B] (e.g. greedy_verify's output), clamped to [0, T-1].
 * Sizes    B >= 0 (0: nothing to do), T in 1..32, D 64 or 128
 *          (W4V_ERR_UNSUPPORTED otherwise), B*T*H*D*4 bytes below 2 GiB.
 * ---------------------------------------------------------------------- */
int gdn_state_commit(float* state, const float* k, const float* v, const float* alpha,
                     const float* beta, const int32_t* accepted_len, int B, int T, int H, int D,
                     void* stream);

/* ------------------------------------------------------------------------
 * A chain of W4A16 linears in one launch (section 3: the target's forward
 * pass over the verify block -- every linear of every layer -- at M <= 16
 * rows).  Linear l reads the leading K_l columns of linear l-1's output
 * (K_l <= N_{l-1}); the first reads x, the last writes y:
 *
 *   h_0 = x;  h_l = fp16_rne( alpha_l * h_{l-1}[:, :K_l] @ W_l ),  y = h_{n-1}
 *
 * with W_l in the layout of w4a16_gemm.  Each intermediate output is rounded
 * to fp16 exactly as a separate w4a16_gemm call would round it.
 *
 * One block per compute unit stays resident for the whole chain.  Each
 * linear's output columns are dealt to eight groups of blocks (one per XCD:
 * the hardware deals blocks round-robin over the XCDs) and, inside a group,
 * to units of 16-80 columns x one K-split; every block's units are copied,
 * in chain order, into one contiguous stream in the workspace (the same
 * bytes as the canonical layout, reordered), which the block streams into
 * LDS ahead of the math.  A unit of linear l waits only for the output tiles
 * of linear l-1 it reads (ready flags in the workspace); split-K partial sums
 * stay in the group's L2 when all of a group's blocks report the same XCD.
 *
 * w4a16_chain_prepare writes the launch plan for the current device's
 * compute-unit count into the caller's workspace and copies every linear's
 * weights, scales and zero-points into it (stream-ordered kernels, then a
 * device synchronisation); it must not run while a call that uses this
 * workspace is in flight.  After it returns, the linears' own device arrays
 * are no longer read.  The prepared workspace is then used by any number of
 * w4a16_chain calls ordered on one stream, on the same device (also from a
 * captured graph: each launch leaves the buffers the next launch writes in
 * their prepared state).
 *
 * linears    host array of n_linears descriptors (device pointers inside),
 *            1 <= n_linears <= 65535; K % 128 == 0, N % 8 == 0, qweight and
 *            qzeros 4-byte aligned, scales 2-byte aligned; N % 16 != 0, or a
 *            linear the plan cannot fit in one block's LDS ring and registers
 *            (more than 24 groups of 128 k per unit, more than 64 input tiles
 *            per unit), returns W4V_ERR_UNSUPPORTED.
 * M          1..16 rows (W4V_ERR_UNSUPPORTED above 16).
 * x          fp16 [M x K_0], row stride ldx >= K_0, 16-byte aligned, ldx % 8 == 0.
 * y          fp16 [M x N_{n-1}], row stride ldy >= N_{n-1}, 16-byte aligned,
 *            ldy % 8 == 0; must not overlap x.
 * workspace  w4a16_chain_workspace_size(...) bytes (about the linears' own
 *            bytes plus their outputs and partial sums), 256-byte aligned.
 *            Byte offset 28 holds an error word the kernel sets (sticky until
 *            the caller prepares again): 1 = a wait for another block's output
 *            exceeded its bound (results invalid), 2 = the workspace was not
 *            prepared for this M, K_0, N_{n-1} and device, or a previous call
 *            gave up a wait (nothing computed).
 * Each output element is computed in a fixed order, so results are
 * bit-identical from call to call.
 * ---------------------------------------------------------------------- */
typedef struct {
  const int32_t* qweight;   /* int32 [K/8 x N]   */
  const void* scales;       /* fp16  [K/128 x N] */
  const int32_t* qzeros;    /* int32 [K/128 x N/8] */
  int K;
  int N;
  float alpha;
} w4v_chain_linear;

/* ------------------------------------------------------------------------
 * Prompt-lookup (n-gram) drafting (section 3, Table 3 and the paragraph on
 * n-gram drafting: no auxiliary model, copies spans from the prompt, K fixed
 * per deployment -- 23 for the team that used it), the step before the
 * verify, and appending the verify's accepted tokens, the step after it.
 *
 * ngram_draft: for each sequence b with history h[0..L) (L = lengths[b]),
 * for n from n_max down to n_min, the most recent earlier occurrence of the
 * last n tokens that ends at position e <= L-2; the longest n that has one
 * wins.  drafts[b][j] = h[e+1+j] for e+1+j < L, else -1 (constant K, the -1
 * padding of section 3); all -1 when nothing matches.
 *
 * history    int32 [B x ld] (row b holds sequence b's tokens), 4-byte aligned.
 * lengths    int32 [B]: tokens of each history (clamped to [0, ld]).
 * n_max, n_min  1 <= n_min <= n_max <= 64.
 * K          >= 1 drafts per sequence.
 * drafts     int32 [B x K] out, 4-byte aligned; must not overlap history.
 * B          >= 0 (0: nothing to do).
 *
 * append_accepted: history[b][L .. L+a_b] = out_tokens[b][0 .. a_b] with
 * a_b = accepted_len[b] (clamped to [0, K]), cut at the row capacity ld;
 * lengths[b] grows by the tokens written.  out_tokens int32 [B x (K+1)] and
 * accepted_len int32 [B] as written by greedy_verify; K >= 0.
 *
 * Both are stream-ordered; argument errors return before any launch.
 * ---------------------------------------------------------------------- */
int ngram_draft(const int32_t* history, int64_t ld, const int32_t* lengths, int B, int n_max,
                int n_min, int K, int32_t* drafts, void* stream);

int append_accepted(int32_t* history, int64_t ld, int32_t* lengths, int B, int K,
                    const int32_t* out_tokens, const int32_t* accepted_len, void* stream);

size_t w4a16_chain_workspace_size(const w4v_chain_linear* linears, int n_linears, int M);

int w4a16_chain_prepare(const w4v_chain_linear* linears, int n_linears, int M,
                        void* workspace, size_t workspace_bytes);

int w4a16_chain(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int K0, int N_last,
                void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4V_H */
