/*
 * moe_fp8.h -- C ABI of the block-scaled FP8 Mixture-of-Experts layer for AMD Instinct MI355X
 * (gfx950).  Shared library: libmoe_fp8.so.
 *
 * The layer is the MoE block that "RL at 1T Scale: prime-rl Performance Deep Dive" (Prime
 * Intellect blog) runs both at inference and in the trainer:
 *   - a top-k router, whose decisions inference records in a [num_layers, top_k, seq_len]
 *     routing payload and the trainer replays in place of the router (section "Router replay");
 *   - dispatch of tokens to their experts and the combine back to token order, the layer's two
 *     exchange points (sections "Wide EP" and "Parallelism / EP");
 *   - block-scaled FP8 as proposed by DeepSeek V3, used by inference and by training so that both
 *     run the same precision (sections "FP8 inference" and "FP8 training"): activations with one
 *     fp32 scale per 1x128 block, weights with one per 128x128 block, e4m3 codes, fp32 accumulation.
 *
 * Calling order for one layer forward on one GPU:
 *   moe_gate_logits -> moe_route | moe_replay_route -> moe_quant_fp8_block (x, 1x128)
 *   -> moe_dispatch -> moe_grouped_gemm_fp8 (W1, SwiGLU + 1x128 re-quantisation)
 *   -> moe_grouped_gemm_fp8 (W2) -> moe_combine.
 * Expert weights are quantised once with moe_quant_fp8_block (128x128 blocks).
 *
 * Conventions (all entry points):
 *   - Pointers are device pointers allocated and owned by the caller unless stated otherwise; the
 *     library allocates no device memory and keeps no state between calls.  Scratch memory is a
 *     caller-provided workspace of at least moe_workspace_bytes(...) bytes.
 *   - Every call enqueues work on `stream` (a hipStream_t passed as void*, NULL = default stream),
 *     never synchronises and returns an int status: MOE_OK or a negative MOE_ERR_* code.  Argument
 *     checks run on the host before any launch; on an error nothing is enqueued.
 *   - Row-major layouts.  Activations [rows, K] (K contiguous); activation scales [rows, K/128];
 *     expert weights [groups, N, K] (K contiguous, i.e. Y = A * W^T); weight scales
 *     [groups, N/128, K/128].  W1 rows [0, F) are the gate projection and rows [F, 2F) the up
 *     projection.  Indices are int32; scales fp32; codes are OCP FP8 E4M3 ("e4m3fn") bytes.
 *   - Deterministic: identical inputs give bitwise identical outputs (no floating-point atomics).
 *   - Data errors found on the device (a replayed expert id outside [0, E) or repeated within a
 *     token) are counted in an optional device int32 counter; that token is routed to no expert
 *     (index -1, weight 0) and is skipped by dispatch and combine.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)      /* a required pointer is NULL                                  */
#define MOE_ERR_SHAPE (-2)     /* a size is out of range or not a multiple of 128 where needed */
#define MOE_ERR_DTYPE (-3)     /* unsupported dtype code                                     */
#define MOE_ERR_ARG (-4)       /* inconsistent router configuration or other argument         */
#define MOE_ERR_HIP (-5)       /* the HIP runtime reported an error at launch                 */
#define MOE_ERR_WORKSPACE (-6) /* workspace missing or smaller than moe_workspace_bytes()     */

/* dtype codes */
#define MOE_F32 0
#define MOE_BF16 1
#define MOE_FP8_E4M3 2

/* router score functions */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1

/* grouped-GEMM epilogues */
#define MOE_EPI_STORE 0        /* out = A * W^T in out_dtype (bf16 or fp32)                   */
#define MOE_EPI_SWIGLU_QUANT 1 /* h = silu(gate) * up, then 1x128 FP8 quantisation of h     */

/* block-scale forms (moe_quant_fp8_block, moe_grouped_gemm_fp8) */
#define MOE_SCALE_AMAX 0       /* s = amax / 448, any positive fp32                            */
#define MOE_SCALE_POW2 1       /* s a power of two in [2^-127, 2^127] (an E8M0 exponent)       */

/* weight layouts accepted by moe_grouped_gemm_fp8 */
#define MOE_B_ROWMAJOR 0       /* b [groups, N, K] e4m3, row-major                             */
#define MOE_B_PACKED 1         /* b rearranged by moe_pack_weights_fp8 for the same epilogue    */
#define MOE_B_PACKED_FP4 2     /* FP4 weights from moe_pack_weights_fp4 (bs: its scale image)   */

/* workspace query op codes */
#define MOE_OP_DISPATCH 1
#define MOE_OP_GROUPED_GEMM 2

/* Router configuration.
 *   num_experts      E routed experts, 1 <= E <= 1024
 *   top_k            experts per token, 1 <= top_k <= min(E, 64)
 *   score_fn         MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID
 *   renormalize      0: weight = score of the expert; 1: weights divided by their sum over the slots
 *   n_group          1 = no group limit; else experts form n_group contiguous groups (E % n_group == 0)
 *   topk_group       groups kept (1 <= topk_group <= n_group; top_k <= topk_group * E / n_group)
 *   group_score_topk a group's score is the sum of its best group_score_topk expert scores
 */
typedef struct {
  int32_t num_experts, top_k, score_fn, renormalize, n_group, topk_group, group_score_topk;
} moe_router_cfg;

/* Router gate projection (the first step of "the router" whose decisions the blog's section
 * "Router replay" records).  logits[t,e] = sum_h x[t,h] * wg[e,h] (+ bias[e]) computed as one fp32
 * fused-multiply-add chain in ascending h starting from +0, then one fp32 add of the bias, so the
 * routing decided from it is reproducible bit for bit.
 *   x       [T,H] in x_dtype (MOE_F32 or MOE_BF16)      wg [E,H] fp32     bias [E] fp32 or NULL
 *   logits  [T,E] fp32 (output)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (T < 0, H < 1 or H % 8 != 0, E < 1), MOE_ERR_DTYPE, MOE_ERR_HIP.
 * T == 0 is a no-op. */
int moe_gate_logits(const void* x, int x_dtype, const float* wg, const float* bias, int64_t T, int32_t H,
                    int32_t E, float* logits, void* stream);

/* Top-k router (blog section "Router replay": the routing decisions that inference captures).
 * Per token: scores (softmax: exp(z - max z) / sum, the sum in ascending expert order;
 * sigmoid: 1 / (1 + exp(-z)); exp is a fixed Cody-Waite reduction + degree-6 polynomial in fp32),
 * optional group limit, selection of top_k experts by logit descending (ties: lower expert id),
 * slot j = j-th best; weight = score, or score / (sum of the slot scores in slot order) when
 * renormalised.
 *   logits    [T,E] fp32          topk_idx [T,top_k] int32 (out)     topk_w [T,top_k] fp32 (out)
 *   record    NULL, or one layer of the routing payload [top_k, record_ld] int32 (record_ld >= T):
 *             record[j*record_ld + t] = topk_idx[t,j]
 * Logits may be -inf (a masked expert): it ranks below every finite logit by the same rule, so a
 * token with fewer than top_k finite allowed logits fills its last slots with the lowest-index
 * allowed -inf experts.  A softmax router needs at least one finite logit per token (the maximum
 * is subtracted); NaN logits are outside the contract.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ARG (invalid cfg, record_ld < T), MOE_ERR_HIP. */
int moe_route(const float* logits, int64_t T, const moe_router_cfg* cfg, int32_t* topk_idx, float* topk_w,
              int32_t* record, int64_t record_ld, void* stream);

/* moe_route and the 1x128 quantisation of x (moe_quant_fp8_block with block_rows 1, scale_mode)
 * in one launch: the quantisation does not depend on the routing, so its workgroups run beside the
 * router's.  Outputs bitwise those of the two separate calls.
 *   x [T, H] in x_dtype (MOE_F32 / MOE_BF16; H % 128 == 0) -> xq [T, H] e4m3, xs [T, H/128] fp32.
 * Errors: as moe_route and moe_quant_fp8_block. */
int moe_route_quant(const float* logits, int64_t T, const moe_router_cfg* cfg, int32_t* topk_idx, float* topk_w,
                    int32_t* record, int64_t record_ld, const void* x, int x_dtype, int32_t H, int32_t scale_mode,
                    uint8_t* xq, float* xs, void* stream);

/* Router replay (blog section "Router replay": recorded decisions replayed on the trainer in place
 * of the router).  topk_idx[t,j] = replay[j*replay_ld + t] unchanged; weights recomputed from the
 * current logits with cfg's score function and normalisation (group limits do not apply).  A token
 * with an id outside [0,E) or a repeated id gets index -1 and weight 0 in every slot and adds 1 to
 * *bad_count (device int32, accumulated, not reset; may be NULL).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ARG (invalid cfg, replay_ld < T), MOE_ERR_HIP. */
int moe_replay_route(const float* logits, int64_t T, const moe_router_cfg* cfg, const int32_t* replay,
                     int64_t replay_ld, int32_t* topk_idx, float* topk_w, int32_t* bad_count, void* stream);

/* Router replay fused with the gate projection, for sigmoid routers (blog section "Router replay";
 * the trainer replays recorded decisions, and with sigmoid scores a token's weights depend only on
 * the logits of its k recorded experts).  Equivalent, bit for bit, to moe_gate_logits followed by
 * moe_replay_route, but only the k recorded logits of each token are computed (k/E of the gate
 * projection's work): each is the same fp32 chain over h ascending from +0, plus bias[e].
 *   x [T,H] in x_dtype (MOE_F32 or MOE_BF16); wg [E,H] fp32; bias [E] fp32 or NULL;
 *   replay, replay_ld, topk_idx, topk_w, bad_count as in moe_replay_route.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H % 8), MOE_ERR_DTYPE, MOE_ERR_ARG (invalid cfg, a softmax cfg,
 *         replay_ld < T), MOE_ERR_HIP. */
int moe_replay_gate(const void* x, int x_dtype, const float* wg, const float* bias, int64_t T, int32_t H,
                    const moe_router_cfg* cfg, const int32_t* replay, int64_t replay_ld, int32_t* topk_idx,
                    float* topk_w, int32_t* bad_count, void* stream);

/* The router's fixed score function, elementwise, for validating the bit-exact routing contract:
 * y[i] = exp(x[i]) as used in the softmax scores (score_fn MOE_SCORE_SOFTMAX), or
 * y[i] = 1 / (1 + exp(-x[i])) (MOE_SCORE_SIGMOID); exp is the Cody-Waite + degree-6 polynomial fp32
 * evaluation described at moe_route, with its input clamped to [-86, 88].  x, y: [n] fp32.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ARG (score_fn), MOE_ERR_HIP. */
int moe_router_score_eval(const float* x, int64_t n, int score_fn, float* y, void* stream);

/* Block-scaled FP8 quantisation (blog section "FP8 training": block-scaled FP8 as in DeepSeek V3).
 * x is [batch, rows, cols] in x_dtype (MOE_F32 or MOE_BF16); blocks are block_rows x 128 with
 * block_rows = 1 (activations) or 128 (weights).  Per block: amax = max |x|; s = amax / 448 (IEEE
 * fp32 division; s = 1 if amax == 0) with scale_mode MOE_SCALE_AMAX, or with MOE_SCALE_POW2 the
 * smallest power of two at or above that quotient, at least 2^-127 (s = 1 if amax == 0), the form
 * the grouped GEMM applies in the matrix cores; q = e4m3(x / s), x / s an IEEE fp32 division,
 * rounded to nearest even, magnitudes above 448 saturated to 448, sign of zero kept.
 *   q       [batch, rows, cols] e4m3 bytes (out)
 *   scales  [batch, rows/block_rows, cols/128] fp32 (out)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (cols % 128, rows % block_rows), MOE_ERR_ARG (block_rows,
 *         scale_mode), MOE_ERR_DTYPE, MOE_ERR_HIP. */
int moe_quant_fp8_block(const void* x, int x_dtype, int64_t batch, int64_t rows, int32_t cols, int32_t block_rows,
                        int32_t scale_mode, uint8_t* q, float* scales, void* stream);

/* Dispatch (blog sections "Wide EP" / "Parallelism / EP": tokens are sent to their experts).
 * A stable counting sort of the [T,k] expert ids: group e holds the rows of every (t,j) with
 * topk_idx[t,j] == e, in ascending token order; with append_shared, group E holds one row per token
 * (the always-on shared expert), in token order.  G = E + (append_shared ? 1 : 0) groups.
 *   counts    [G] int32 (out)        offsets [G+1] int32 exclusive prefix of counts (out)
 *   dest_row  [T,k] int32: row of slot (t,j), or -1 for a slot with index -1 (out)
 *   src_token [T*k + (append_shared ? T : 0)] int32: token of each row; entries beyond offsets[G]
 *             are left untouched (out)
 *   xq, xs    the 1x128-quantised activations [T,H] and scales [T,H/128]; aq, as receive the
 *             permuted copies [rows,H] and [rows,H/128] (rows = offsets[G]).  With aq NULL and as
 *             given only the scales are permuted (moe_grouped_gemm_fp8_gather then reads the codes
 *             from xq through src_token); with aq and as both NULL only the index outputs are
 *             produced.
 *   workspace >= moe_workspace_bytes(MOE_OP_DISPATCH, T, k, E, 0, 0) bytes.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H % 128, E > 1024), MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
int moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t append_shared,
                 const uint8_t* xq, const float* xs, int32_t H, int32_t* counts, int32_t* offsets, int32_t* dest_row,
                 int32_t* src_token, uint8_t* aq, float* as, void* workspace, size_t workspace_bytes, void* stream);

/* Weight packing for the grouped GEMM (a layout transform, not part of the method).  The GEMM's
 * workgroups read each expert's weights as panels of 256 rows (for MOE_EPI_SWIGLU_QUANT: 128 gate
 * rows [f0, f0+128) followed by the matching up rows [F+f0, F+f0+128)), 128 bytes of K at a time;
 * in row-major order those are 256 separate 128-byte pieces at a stride of K bytes.  The packed
 * layout stores every (group, panel, K step) as one contiguous 32 KB block, already in the order
 * and 16-byte-chunk swizzle the GEMM keeps in LDS, so each K step streams one block from HBM.
 *   b      [groups, N, K] e4m3 row-major (device, read)
 *   packed [moe_packed_weight_bytes(groups, N, K, epilogue)] bytes (device, written); panels of a
 *          STORE weight with N % 256 != 0 are padded with zero rows
 *   epilogue: the epilogue of the GEMM calls that will use the packed weight (it fixes the panels)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (N, K % 128; N % 256 for SwiGLU; a panel row of K bytes
 *         times the panels of one group at or above 2^32), MOE_ERR_ARG (epilogue), MOE_ERR_HIP. */
int moe_pack_weights_fp8(const uint8_t* b, int32_t groups, int32_t N, int32_t K, int32_t epilogue, uint8_t* packed,
                         void* stream);

/* Bytes of a packed weight: groups * ceil(N / 256) * 256 * K (equal to the row-major size when
 * N % 256 == 0).  0 for invalid shapes. */
size_t moe_packed_weight_bytes(int32_t groups, int32_t N, int32_t K, int32_t epilogue);

/* Grouped block-scaled FP8 GEMM (blog sections "FP8 inference" / "FP8 training": the FP8 expert
 * GEMMs).  For each group g and each row r in [offsets[g], offsets[g+1]):
 *   acc[r,n] = sum over 128-wide K blocks kb of (as[r,kb] * bs[g,n/128,kb]) * sum_{k in kb} a[r,k]*b[g,n,k]
 * with fp32 accumulation (e4m3 products accumulated exactly inside each 128-block, then promoted).
 *   a  [max_rows, K] e4m3, as [max_rows, K/128] fp32; offsets [groups+1] device int32, offsets[groups] <= max_rows
 *   b  [groups, N, K] e4m3 (b_layout MOE_B_ROWMAJOR) or the same weight after moe_pack_weights_fp8
 *      with this call's epilogue (b_layout MOE_B_PACKED), or FP4 weights packed by moe_pack_weights_fp4
 *      (b_layout MOE_B_PACKED_FP4, bs its scale image, power-of-two scale_mode only);
 *      bs [groups, N/128, K/128] fp32
 *   epilogue MOE_EPI_STORE:        out [max_rows, N] in out_dtype (MOE_BF16 or MOE_F32)
 *   epilogue MOE_EPI_SWIGLU_QUANT: N = 2F; h[r,f] = silu(acc[r,f]) * acc[r,F+f] in fp32, quantised
 *            1x128 as in moe_quant_fp8_block: out [max_rows, F] e4m3 (out_dtype MOE_FP8_E4M3),
 *            out_scales [max_rows, F/128] fp32
 *   scale_mode: MOE_SCALE_AMAX (any positive fp32 scales: each 128-wide K block's fp32 partial is
 *            promoted into the accumulator with the product of its two scales) or MOE_SCALE_POW2
 *            (every scale in as and bs a power of two in [2^-127, 2^127], as moe_quant_fp8_block
 *            writes them in that mode: the matrix cores apply them as E8M0 exponents and accumulate
 *            directly; only the exponent field of each scale is read; the SwiGLU epilogue then
 *            quantises h with power-of-two scales too)
 *   tile_rows: rows per workgroup tile, 32, 48, 64, 128 or 256 (256: packed weights only), or 0 to
 *            choose from the group sizes: the smallest of 32, 48, 64, 128 at or above
 *            2 * ceil(max_rows / groups), and 256 from 512 on when the weights are packed.  The result
 *            is the same for every height.
 *   Rows beyond offsets[groups] are not written.  workspace >= moe_workspace_bytes(MOE_OP_GROUPED_GEMM,
 *   max_rows, 0, groups, N, K).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (N, K % 128; F % 128 for SwiGLU; (max_rows+1)*K or one group's
 *         weight bytes at or above 2^32), MOE_ERR_DTYPE, MOE_ERR_ARG (epilogue, scale_mode, tile_rows,
 *         b_layout),
 *         MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
int moe_grouped_gemm_fp8(const uint8_t* a, const float* as, const int32_t* offsets, int32_t groups, int64_t max_rows,
                         const uint8_t* b, int32_t b_layout, const float* bs, int32_t N, int32_t K, int32_t epilogue,
                         int32_t scale_mode, int32_t tile_rows, void* out, int out_dtype, float* out_scales,
                         void* workspace, size_t workspace_bytes, void* stream);

/* moe_grouped_gemm_fp8 for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): the same computation and results
 * (bitwise), with the tile plan kept in the library's own device scratch (MOE_NOALLOC_SCRATCH_BYTES,
 * a static device array of each GPU the library runs on, held until the process ends) instead of a
 * caller workspace.  The call allocates and frees nothing; the caller still passes every input and
 * output.  Limit: moe_workspace_bytes(MOE_OP_GROUPED_GEMM, max_rows, 0, groups, N, K) must not
 * exceed MOE_NOALLOC_SCRATCH_BYTES (about max_rows + 32 * groups <= 65000 * 32 rows), else
 * MOE_ERR_WORKSPACE and nothing is enqueued.  Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's plan: calls that overlap on one GPU (several streams, or host threads without
 * ordering) race and must be serialised by the caller.  The first call on a device looks up the
 * scratch's device address (hipGetSymbolAddress) with that device current.
 * Errors: as moe_grouped_gemm_fp8, with MOE_ERR_WORKSPACE for a plan larger than the scratch. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)
int moe_grouped_gemm_fp8_noalloc(const uint8_t* a, const float* as, const int32_t* offsets, int32_t groups,
                                 int64_t max_rows, const uint8_t* b, int32_t b_layout, const float* bs, int32_t N,
                                 int32_t K, int32_t epilogue, int32_t scale_mode, int32_t tile_rows, void* out,
                                 int out_dtype, float* out_scales, void* stream);

/* Grouped GEMM in two steps, so that one tile plan serves several GEMMs over the same groups
 * (the layer's W1 and W2 GEMMs) and the GEMM launch itself is one kernel (two for a plan of 256-row
 * tiles: the groups' full tiles and short tiles of more than 128 rows, then the short remainders of
 * up to 128 rows as 128-row tiles).
 * moe_grouped_gemm_plan writes the list of row tiles of `offsets` (device) into `workspace`
 * (>= moe_workspace_bytes(MOE_OP_GROUPED_GEMM, max_rows, 0, groups, 0, 0) bytes, caller-owned, and
 * holding the plan until the last GEMM that uses it has run) and fills `plan` (host) with the tile
 * height (tile_rows as in moe_grouped_gemm_fp8) and the sizes.  moe_grouped_gemm_fp8_planned then
 * computes exactly what moe_grouped_gemm_fp8 computes, for the groups, max_rows and tile height of
 * the plan, with the same `offsets` contents.  A plan of 256-row tiles (chosen, or automatic for
 * groups averaging more than 256 rows) serves packed weights only: a planned call with row-major
 * weights on it returns MOE_ERR_ARG.
 * Errors: as moe_grouped_gemm_fp8 (MOE_ERR_NULL also for a NULL plan). */
typedef struct moe_gemm_plan {
  int32_t tile_rows;   /* chosen row-tile height */
  int32_t groups;
  int64_t max_rows;
  void* workspace;     /* where the tile list lives */
} moe_gemm_plan;

int moe_grouped_gemm_plan(const int32_t* offsets, int32_t groups, int64_t max_rows, int32_t tile_rows,
                          void* workspace, size_t workspace_bytes, moe_gemm_plan* plan, void* stream);

int moe_grouped_gemm_fp8_planned(const moe_gemm_plan* plan, const uint8_t* a, const float* as, const int32_t* offsets,
                                 const uint8_t* b, int32_t b_layout, const float* bs, int32_t N, int32_t K,
                                 int32_t epilogue, int32_t scale_mode, void* out, int out_dtype, float* out_scales,
                                 void* stream);

/* Dispatch and tile plan in one call: moe_dispatch (same arguments and outputs) followed by
 * moe_grouped_gemm_plan(offsets, G, max_rows = T*k + (append_shared ? T : 0), tile_rows,
 * gemm_workspace, ...) for the G = E + (append_shared ? 1 : 0) groups it produces.  With G <= 1024
 * the dispatch's own one-workgroup kernel (the whole dispatch for decode-sized batches, else the
 * scan of the chunk histograms) also writes the tile lists, which saves the plan's own launch;
 * otherwise the plan kernel runs after the dispatch.  The plan is the same either way.
 * Errors: as moe_dispatch and moe_grouped_gemm_plan. */
int moe_dispatch_plan(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t append_shared,
                      const uint8_t* xq, const float* xs, int32_t H, int32_t* counts, int32_t* offsets,
                      int32_t* dest_row, int32_t* src_token, uint8_t* aq, float* as, void* workspace,
                      size_t workspace_bytes, int32_t tile_rows, void* gemm_workspace, size_t gemm_workspace_bytes,
                      moe_gemm_plan* plan, void* stream);

/* moe_grouped_gemm_fp8_planned with the rows of A gathered instead of stored in group order (blog
 * sections "Wide EP" / "Parallelism / EP": the dispatch permutation, here folded into the GEMM's
 * loads): group row r (r < offsets[groups]) multiplies the codes of row a_rows[r] of
 * a [a_count, K] (the token-order quantised activations, a_rows the dispatch's src_token), with the
 * scales of group row r in as [max_rows, K/128] (permuted by moe_dispatch with aq NULL).  The
 * result is bitwise that of moe_grouped_gemm_fp8_planned on the permuted copy.  a_rows entries
 * must lie in [0, a_count); the kernel clamps them into that range, so a bad entry cannot read
 * outside a.  g_out: as in moe_grouped_gemm_fp8_swiglu_save (NULL unless epilogue is
 * MOE_EPI_SWIGLU_QUANT).
 * Errors: as moe_grouped_gemm_fp8_planned; MOE_ERR_NULL (a_rows NULL), MOE_ERR_SHAPE (a_count < 1
 * or (a_count + 1) * K at or above 2^32), MOE_ERR_ARG (g_out with the store epilogue). */
int moe_grouped_gemm_fp8_gather(const moe_gemm_plan* plan, const uint8_t* a, int64_t a_count, const int32_t* a_rows,
                                const float* as, const int32_t* offsets, const uint8_t* b, int32_t b_layout,
                                const float* bs, int32_t N, int32_t K, int32_t epilogue, int32_t scale_mode, void* out,
                                int out_dtype, float* out_scales, float* g_out, void* stream);

/* Training forward of GEMM1 (blog section "FP8 training": the trainer runs this layer and then its
 * backward, whose SwiGLU derivative needs the GEMM1 output): moe_grouped_gemm_fp8_planned with
 * epilogue MOE_EPI_SWIGLU_QUANT (h codes into h [max_rows, N/2], scales into h_scales), which in
 * the same pass also stores the fp32 accumulators G = [gate | up] into g_out [max_rows, N] (rows
 * past offsets[groups] are not written).  h and h_scales are bitwise those of the plain call.
 * Errors: as moe_grouped_gemm_fp8_planned (MOE_ERR_NULL for a NULL g_out). */
int moe_grouped_gemm_fp8_swiglu_save(const moe_gemm_plan* plan, const uint8_t* a, const float* as,
                                     const int32_t* offsets, const uint8_t* b, int32_t b_layout, const float* bs,
                                     int32_t N, int32_t K, int32_t scale_mode, uint8_t* h, float* h_scales,
                                     float* g_out, void* stream);

/* Combine (blog sections "Wide EP" / "Parallelism / EP": expert outputs return to token order).
 *   out[t,:] = sum_{j<k, dest_row[t,j] >= 0} topk_w[t,j] * y[dest_row[t,j],:]  (+ y[*shared_first_row + t,:])
 * accumulated in fp32 in slot order, the shared row last, then rounded to out_dtype.
 *   y [rows,H] in y_dtype (MOE_BF16 or MOE_F32); dest_row, topk_w [T,k]; out [T,H] in out_dtype.
 *   shared_first_row: NULL (no shared expert) or a device int32 holding the first row of the shared
 *   group (pass &offsets[E] from moe_dispatch).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H % 8), MOE_ERR_DTYPE, MOE_ERR_HIP. */
int moe_combine(const void* y, int y_dtype, const int32_t* dest_row, const float* topk_w, int64_t T, int32_t k,
                int32_t H, const int32_t* shared_first_row, void* out, int out_dtype, void* stream);

/* Combine on a residual branch (the replay stack of the blog's "Router replay" section runs the same
 * MoE layer several layers deep; each layer's output is added to its input).
 *   o[t,:]      = act(sum_j topk_w[t,j] * y[dest_row[t,j],:] (+ shared row))   -- as moe_combine
 *   x_next[t,:] = act(residual[t,:] + o[t,:])     (fp32 add of the two stored values, one rounding)
 * act = act_dtype (MOE_BF16 or MOE_F32) for residual, out and x_next.  out may be NULL (then only
 * x_next is written); otherwise out receives o, bitwise what moe_combine writes.  x_next may alias
 * residual (each element is read before it is written, by the same thread).
 * Errors: MOE_ERR_NULL (y, dest_row, topk_w, residual or x_next NULL), MOE_ERR_SHAPE, MOE_ERR_DTYPE,
 * MOE_ERR_HIP. */
int moe_combine_residual(const void* y, int y_dtype, const int32_t* dest_row, const float* topk_w, int64_t T,
                         int32_t k, int32_t H, const int32_t* shared_first_row, const void* residual, void* out,
                         void* x_next, int act_dtype, void* stream);

/* Router-replay payload codec (blog section "Router replay": the routing decisions recorded at
 * inference, a [num_layers, top_k, seq_len] integer payload, reach tens of Gbps and hundreds of GB
 * and are handled as an opaque tensor by tensor operations only).  The pages fix no storage format;
 * this one is a lossless fixed-width code.
 * Format: b = max(1, ceil(log2 E)) bits per index; index i of the flattened payload occupies bits
 * [i*b, (i+1)*b) of a little-endian bit stream, least significant bit first (stream bit j is bit j%8
 * of byte j/8), zero-padded to whole groups of 32 indices: moe_payload_bytes(n, E) =
 * ceil(n/32) * 4 * b bytes (E <= 256: one byte per index, 4x smaller than int32).
 *   n: indices (any shape, flattened; 0 <= n <= 2^40), E: experts (1 <= E <= 65536).
 * moe_payload_bytes returns 0 for an invalid (n, E). */
size_t moe_payload_bytes(int64_t n, int32_t E);

/* Pack n int32 indices (device) into `packed` (device, moe_payload_bytes(n, E) bytes).  Indices
 * outside [0, E) are not representable: their low b bits are stored and, if bad_count is not NULL,
 * their number is added to *bad_count (device int32).  idx and packed must be 16-byte aligned.
 * Errors: MOE_ERR_SHAPE (n, E), MOE_ERR_NULL, MOE_ERR_ARG (alignment), MOE_ERR_HIP. */
int moe_payload_pack(const int32_t* idx, int64_t n, int32_t E, uint8_t* packed, int32_t* bad_count, void* stream);

/* Unpack n indices from `packed` (device) into idx (device int32).  16-byte alignment as above.
 * Errors: as moe_payload_pack. */
int moe_payload_unpack(const uint8_t* packed, int64_t n, int32_t E, int32_t* idx, void* stream);

/* Pack on the device into `staging` (device, moe_payload_bytes(n, E) bytes) and copy the packed
 * bytes to `host` asynchronously on `stream` (host should be pinned memory, else the copy is not
 * asynchronous); the host bytes are valid once the stream reaches this point. */
int moe_payload_to_host(const int32_t* idx, int64_t n, int32_t E, uint8_t* staging, void* host, int32_t* bad_count,
                        void* stream);

/* Copy packed bytes from `host` into `staging` (device) and unpack them into idx (device int32),
 * asynchronously on `stream`; host must stay unchanged until the stream reaches this point. */
int moe_payload_from_host(const void* host, int64_t n, int32_t E, uint8_t* staging, int32_t* idx, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward of the layer (blog section "FP8 training": the trainer runs the same block-scaled FP8
 * recipe as inference, so the backward contracts in FP8 too; section "Router replay": the routing
 * selection is replayed, so it is a fixed input of the backward and only the routing weights carry
 * gradient).  Calling order, after a forward whose buffers are still live (dispatch, logits,
 * topk_idx/topk_w, expert rows y):
 *   moe_combine_backward (dY codes, dw) -> moe_grouped_gemm_fp8 (dY x W2^T packed, STORE fp32: dh)
 *   -> [the GEMM1 output G: kept by a forward that ran moe_grouped_gemm_fp8_swiglu_save, else
 *      recomputed by moe_grouped_gemm_fp8 (A x W1 packed for STORE, fp32)]
 *   -> moe_swiglu_backward_quant (dG codes) -> moe_grouped_gemm_fp8 (dG x W1^T packed, fp32: dA)
 *   -> moe_combine (dA, weights 1, fp32: expert part of dx) -> moe_route_backward (dz)
 *   -> moe_gate_backward (dx = expert part + dz Wg, dWg, db).
 * The transposed weights come from moe_transpose_fp8_blocks (a 128x128 block keeps its scale under
 * transposition, so the data-gradient GEMMs need no re-quantisation).
 * ------------------------------------------------------------------------------------------- */

/* Combine backward.  For out[t] = sum_j w[t,j] y[dest_row[t,j]] (+ y[shared_first_row + t]):
 *   dY[dest_row[t,j],:] = w[t,j] * dout[t,:]   (one fp32 product; dY = dout for the shared row)
 * stored 1x128-quantised (codes dyq [rows,H] e4m3, scales dys [rows,H/128] fp32, scale_mode as in
 * moe_quant_fp8_block), and dw[t,j] = sum_h dout[t,h] * y[dest_row[t,j],h] in fp32 (a fixed-order
 * tree reduction; 0 for a slot with dest_row -1, whose dY row is not written).
 *   dout [T,H] in dout_dtype, y [rows,H] in y_dtype (MOE_F32 or MOE_BF16: the forward's expert rows
 *   as the combine read them); dest_row, topk_w [T,k] from the forward; shared_first_row NULL or a
 *   device int32 (&offsets[E]); dw [T,k] fp32 (out); row_w NULL or [rows] fp32 (out): each written
 *   row's factor (topk_w of its slot, 1 for a shared row), for the weight gradients.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H % 128, k > 16), MOE_ERR_DTYPE, MOE_ERR_ARG (scale_mode),
 * MOE_ERR_HIP.  T == 0 is a no-op. */
int moe_combine_backward(const void* dout, int dout_dtype, const void* y, int y_dtype, const int32_t* dest_row,
                         const float* topk_w, int64_t T, int32_t k, int32_t H, const int32_t* shared_first_row,
                         int32_t scale_mode, uint8_t* dyq, float* dys, float* dw, float* row_w, void* stream);

/* SwiGLU backward and 1x128 quantisation of the result.  With G = [gate | up] the GEMM1 output
 * [rows, 2F] fp32 and dh [rows, F] fp32:  s = sigmoid(gate), dgate = dh * up * s * (1 + gate * (1 - s)),
 * dup = dh * gate * s (fp32), dG = [dgate | dup] quantised in 1x128 blocks along 2F:
 * dgq [rows, 2F] e4m3, dgs [rows, 2F/128] fp32.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (F % 128), MOE_ERR_ARG (scale_mode), MOE_ERR_HIP. */
int moe_swiglu_backward_quant(const float* dh, const float* g, int64_t rows, int32_t F, int32_t scale_mode,
                              uint8_t* dgq, float* dgs, void* stream);

/* Router backward with the selection held fixed: dz[t,e] = d(loss)/d(logit[t,e]) from
 * dw[t,j] = d(loss)/d(topk_w[t,j]), with the scores recomputed from the logits by the router's own
 * fixed exp.  Renormalised (w_j = score_j / sum_l score_l):  sigmoid dz_{i_j} = s_j (1 - s_j)
 * (dw_j - sum_l w_l dw_l) / sum_l s_l;  softmax dz_{i_j} = w_j (dw_j - sum_l w_l dw_l).  Not
 * renormalised:  sigmoid dz_{i_j} = dw_j s_j (1 - s_j);  softmax (full softmax p over E)
 * dz_e = [e selected] w_e dw_e - p_e sum_l w_l dw_l.  Every other dz element is 0; slots with index
 * -1 carry nothing.  logits [T,E], topk_idx [T,k], dw [T,k], dz [T,E] (out, every element written).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ARG (score_fn), MOE_ERR_HIP. */
int moe_route_backward(const float* logits, const int32_t* topk_idx, const float* dw, int64_t T,
                       const moe_router_cfg* cfg, float* dz, void* stream);

/* Gate-projection backward (fp32, like the forward's logits):
 *   dx[t,h] = dx_in[t,h] + sum_e dz[t,e] wg[e,h]   (dx_in [T,H] fp32 or NULL; one rounding to dx_dtype)
 *   dwg[e,h] = sum_t dz[t,e] x[t,h]                 (fp32; the token range is split into fixed slices
 *                                                    whose partials are summed in slice order)
 *   db[e] = sum_t dz[t,e]                           (fp32, or db NULL to skip)
 * x [T,H] in x_dtype; wg [E,H] fp32; workspace >= moe_gate_backward_workspace(T, E, H) bytes.
 * Deterministic.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H % 8), MOE_ERR_DTYPE, MOE_ERR_WORKSPACE,
 * MOE_ERR_HIP. */
int moe_gate_backward(const float* dz, const void* x, int x_dtype, const float* wg, int64_t T, int32_t H, int32_t E,
                      const float* dx_in, void* dx, int dx_dtype, float* dwg, float* db, void* workspace,
                      size_t workspace_bytes, void* stream);
size_t moe_gate_backward_workspace(int64_t T, int32_t E, int32_t H);

/* Expert-weight gradients (blog section "FP8 training"): dW2[e] = sum over e's rows of dY^T h
 * ([H,F]) and dW1[e] = sum over e's rows of dG^T x ([2F,H]).  Both operands contract over an expert's
 * rows, so they are quantised in 128x1 blocks (128 consecutive rows of one expert x one column) and
 * stored transposed, one contiguous block per expert: expert e's rows fill n_e = tile_first[e+1] -
 * tile_first[e] whole 128-row tiles (zero-padded), its codes are a row-major [C, 128 n_e] block at
 * byte tile_first[e] * 128 * C and its scales a [C, n_e] block at element tile_first[e] * C.
 * Buffers hold max_tiles = moe_wgrad_max_tiles(max_rows, groups) tiles: codes C * max_tiles * 128
 * bytes, scales C * max_tiles fp32 (past tile_first[groups] * 128 * C nothing is written).
 *   moe_wgrad_tiles: tile_first [groups+1] int32 (device, out) from the dispatch offsets [groups+1].
 *   moe_colwise_quant_rows: column c, row r of the operand = row_scale[r] * x[src_row[r], c]
 *     (x [*, C] in x_dtype; src_row NULL = identity; row_scale NULL = 1): dY from dout with the
 *     dispatch's src_token and moe_combine_backward's row_w, or x itself with src_token.
 *   moe_colwise_quant_swiglu: from the GEMM1 output g [rows, 2F] fp32, h = silu(gate) * up (C = F,
 *     dh NULL) or, with dh [rows, F] fp32, dG = [dgate | dup] as in moe_swiglu_backward_quant (C = 2F).
 *   moe_grouped_gemm_wgrad: c[e] = A_e B_e^T ([groups, M, N] fp32, every expert written; zeros for an
 *     expert with no rows), A_e [M, 128 n_e] and B_e [N, 128 n_e] the experts' blocks of two operands
 *     in the layout above (C = M and C = N); amax scales promoted per 128-row step, power-of-two
 *     scales applied by the matrix cores.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (C, M, N % 128; groups), MOE_ERR_DTYPE, MOE_ERR_ARG
 * (scale_mode), MOE_ERR_HIP.  moe_wgrad_max_tiles returns 0 for invalid sizes. */
int64_t moe_wgrad_max_tiles(int64_t max_rows, int32_t groups);
int moe_wgrad_tiles(const int32_t* offsets, int32_t groups, int32_t* tile_first, void* stream);
int moe_colwise_quant_rows(const void* x, int x_dtype, const int32_t* src_row, const float* row_scale,
                           const int32_t* offsets, const int32_t* tile_first, int32_t groups, int64_t max_tiles,
                           int32_t C, int32_t scale_mode, uint8_t* qt, float* st, void* stream);
int moe_colwise_quant_swiglu(const float* g, const float* dh, int32_t F, const int32_t* offsets,
                             const int32_t* tile_first, int32_t groups, int64_t max_tiles, int32_t scale_mode,
                             uint8_t* qt, float* st, void* stream);
int moe_grouped_gemm_wgrad(const uint8_t* a, const float* as, int32_t M, const uint8_t* b, const float* bs, int32_t N,
                           const int32_t* tile_first, int32_t groups, int64_t max_tiles, int32_t scale_mode, float* c,
                           void* stream);

/* FP4 expert weights: the 4-bit variant of the block-scaled recipe (the blog names NVFP4 as future
 * work; the MI355X matrix cores take OCP microscaling FP4).  Elements are FP4 E2M1 (magnitudes 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6) in 1x32 blocks along K; a block's scale is the smallest power of two at
 * or above fl32(amax / 6), at least 2^-127 (1 for an all-zero block), stored as its E8M0 code (the
 * fp32 exponent field); q = e2m1(x / s), round to nearest with ties to the even code, saturating at
 * 6, sign of zero kept.  Activations stay FP8 with power-of-two 1x128 scales.
 *   moe_quant_mxfp4: w [rows, cols] in w_dtype (MOE_F32 / MOE_BF16; cols % 32 == 0) -> q [rows, cols/2]
 *     (two codes per byte, element 2i in the low nibble), e8 [rows, cols/32] uint8.
 *   moe_packed_fp4_bytes: bytes of the packed codes for moe_pack_weights_fp4 (0 if unsupported);
 *     *scale_bytes (if not NULL) receives the bytes of the packed scale image.
 *   moe_pack_weights_fp4: q [groups, N, K/2], e8 [groups, N, K/32] -> packed_q, packed_e8 in the
 *     order the grouped GEMM streams for `epilogue` (per 256-row panel and 128-wide K step: 16 KB of
 *     codes in MFMA fragment order, 1 KB of scale codes [row][32-wide chunk]).  The GEMM then takes
 *     b = packed_q, b_layout = MOE_B_PACKED_FP4, bs = (const float*)packed_e8, scale_mode
 *     MOE_SCALE_POW2 (activation scales must be powers of two).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ARG (epilogue), MOE_ERR_HIP. */
int moe_quant_mxfp4(const void* w, int w_dtype, int64_t rows, int32_t cols, uint8_t* q, uint8_t* e8, void* stream);
size_t moe_packed_fp4_bytes(int32_t groups, int32_t N, int32_t K, int32_t epilogue, size_t* scale_bytes);
int moe_pack_weights_fp4(const uint8_t* q, const uint8_t* e8, int32_t groups, int32_t N, int32_t K, int32_t epilogue,
                         uint8_t* packed_q, uint8_t* packed_e8, void* stream);

/* Transpose of 128x128-block FP8 weights with their scales: qt[g][c][r] = q[g][r][c],
 * scales_t[g][cb][rb] = scales[g][rb][cb]; q [groups,N,K] -> qt [groups,K,N] (N, K multiples of 128).
 * Exact (the codes are moved, not re-encoded).  qt must not alias q.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ARG (qt == q), MOE_ERR_HIP. */
int moe_transpose_fp8_blocks(const uint8_t* q, const float* scales, int32_t groups, int32_t N, int32_t K,
                             uint8_t* qt, float* scales_t, void* stream);

/* Workspace bytes needed by moe_dispatch (op MOE_OP_DISPATCH: rows_or_T = T, k, E) or
 * moe_grouped_gemm_fp8 (op MOE_OP_GROUPED_GEMM: rows_or_T = max_rows, E = groups, N, K). */
size_t moe_workspace_bytes(int op, int64_t rows_or_T, int32_t k, int32_t E, int32_t N, int32_t K);

/* Static description of a status code. */
const char* moe_status_str(int status);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP8_H */
