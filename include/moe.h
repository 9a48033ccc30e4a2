/*
 * moe.h - C ABI of the MI355X (gfx950) sparse mixture-of-experts layer
 * forward pass.
 *
 * The layer (sources: web pages on sparse MoE layers, tagged
 *   [RC]  randomcommits.com "Mixture-of-Experts routing",
 *   [LBS] letsbuildsolutions.com "How Mixture of Experts Works: Sparse
 *         Gating, Expert Routing, and the Architecture Behind Efficient Large
 *         Language Models",
 *   [HA]  hassanahmed.net "Mixture of Experts explained",
 *   [GN]  getnybble.com "Mixture of Experts (MoE) - conditional computation
 *         at scale",
 *   [FA]  foundry.adhana.ai "Mixture-of-Experts routing"):
 *
 *   1. route     logits = x . Wr^T (+ router bias), probs = softmax(logits),
 *                choose the top-k experts, gates = chosen probs renormalised
 *                to sum to 1                    ([RC], [LBS] Gating Mechanism)
 *   2. dispatch  group the (token, slot) assignments by expert, keep the
 *                first `capacity` per expert in token order, drop the rest
 *                                 ([RC], [LBS] The Capacity Factor, Token
 *                                  Dropping and Overflow Handling)
 *   3. expert    GELU MLP or SwiGLU per expert over its kept rows, plus an
 *                optional always-on shared expert ([RC], [GN] Implementing a
 *                complete MoE layer, DeepSeek-V3)
 *   4. combine   out = x + shared + sum over kept slots of gate * expert out
 *                                 ([RC], [FA] Concept)
 *   5. aux       alpha * E * sum_e f_e * P_e  ([LBS] The Load Balancing
 *                Problem, [GN] Load balancing and expert collapse)
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every pointer argument except `p`, `w` and the problem/weights structs
 *   themselves is a DEVICE pointer on the current HIP device, row-major,
 *   contiguous, at least 16-byte aligned.  The workspace must be 256-byte
 *   aligned.  The caller owns every buffer; the library never allocates,
 *   frees or synchronises.
 * - Each call validates all its arguments on the host first; a non-zero
 *   status means nothing was enqueued.  MOE_OK means the work was enqueued
 *   on `stream`; results are valid when the stream reaches that point.
 * - The library holds no mutable global state, except the scratch of
 *   moe_layer_forward_noalloc (below); calls are reentrant.  Two calls that
 *   share an output or workspace buffer must not overlap.
 * - Element types: `x`, expert weights and biases, `y` and `out` all have
 *   the problem's dtype (MOE_DTYPE_F32 or MOE_DTYPE_BF16).  Router weights,
 *   router/selection biases, logits, gates and probabilities are float32
 *   ([LBS] Dense vs Sparse: the router runs in float32).  Indices and
 *   counts are int32.
 * - Weights use nn.Linear storage ([out, in], the input dimension
 *   contiguous) stacked over experts on a leading axis.
 * - Results are deterministic: the same inputs give bit-identical outputs
 *   (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_EINVAL (-1)     /* null required pointer, bad T/E/k/capacity  */
#define MOE_ENOTSUP (-2)    /* shape or dtype this build does not support */
#define MOE_EWORKSPACE (-3) /* workspace smaller than moe_workspace_bytes */
#define MOE_EHIP (-4)       /* a kernel launch failed                     */

/* ---- enums --------------------------------------------------------------- */
#define MOE_ACT_GELU 0   /* Linear(+b1) -> exact erf GELU -> Linear(+b2)   */
#define MOE_ACT_SWIGLU 1 /* W_down (silu(W_gate x) * (W_up x)), no biases  */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

#define MOE_SCORING_SOFTMAX 0 /* softmax over all experts                */
#define MOE_SCORING_SIGMOID 1 /* per-expert sigmoid                      */

#define MOE_OVERFLOW_DROP 0     /* overflow assignments are dropped      */
#define MOE_OVERFLOW_REASSIGN 1 /* reassigned to free slots at random    */

#define MOE_WQUANT_NONE 0 /* expert weights in the problem dtype          */
#define MOE_WQUANT_INT4 1 /* expert weights as 4-bit codes, see below     */
#define MOE_WQUANT_BF16_TILED 2 /* bf16 expert weights in tiled order    */
#define MOE_Q4_GROUP 128  /* weights per (scale, offset) pair             */

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOP_K 8
/* scratch bytes per GPU of moe_layer_forward_noalloc (32 MiB) */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * Problem description.
 *   T          tokens (rows of x), >= 0.  T * top_k < 2^31.
 *   d_model    hidden size d, a positive multiple of 64.
 *   n_experts  routed experts E, 1..256.
 *   top_k      experts per token k, 1..min(E, 8).
 *   d_ff       expert intermediate size, a positive multiple of 64.
 *              Size limits (MOE_ENOTSUP beyond them): d_model * d_ff <
 *              2^32, (T*top_k + (n_shared+1)*T) * max(d_model, d_ff)
 *              < 2^32 (the GEMMs use 32-bit element offsets; it also
 *              keeps x under 2^32 bytes for the 32-bit byte offsets its
 *              rows are gathered with).
 *   n_shared   always-on shared experts, 0 or 1 ([GN] DeepSeek-V3).
 *   capacity   per-expert cap on kept assignments; <= 0 means no cap.
 *   act        MOE_ACT_GELU or MOE_ACT_SWIGLU.
 *   dtype      MOE_DTYPE_F32 or MOE_DTYPE_BF16.
 *   aux_coef   alpha of the load-balance loss (0.01 for Mixtral: [LBS]).
 *   wquant     MOE_WQUANT_NONE, or MOE_WQUANT_INT4 for 4-bit expert
 *              weights ([LBS] Production Considerations, Quantization for
 *              MoE); INT4 requires dtype BF16 and d_model, d_ff multiples
 *              of 128.  MOE_WQUANT_BF16_TILED: the same bf16 weights
 *              stored in moe_tile_bf16's order (dtype BF16).
 *              Zero-initialised structs get NONE.
 *   scoring    MOE_SCORING_SOFTMAX (default) or MOE_SCORING_SIGMOID
 *              ([FA] The knobs: softmax over all experts versus a
 *              per-expert sigmoid).  With sigmoid scores a selection bias
 *              is added to the float32 score (not the logit); without one
 *              the choice is on the logit (the same order).  The P of the
 *              aux loss is then each token's scores scaled to sum to 1.
 *   raw_gates  0 (default): the chosen scores are renormalised to sum to 1;
 *              1: a gate is the chosen score itself ([FA] The knobs,
 *              norm_topk_prob).
 *   overflow   MOE_OVERFLOW_DROP (default) or MOE_OVERFLOW_REASSIGN
 *              ([LBS] Token Dropping and Overflow Handling, random
 *              reassignment): after the capacity cut the dropped
 *              assignments a = t*k + j are visited in ascending a; each
 *              draws x = Philox4x32-10 word 0 of counter (a, 0, 0, 0) under
 *              key (overflow_seed low, high 32 bits) and takes free slot
 *              r = floor(x * total / 2^32) of the candidate experts (a free
 *              slot and not already one of token t's experts; ascending
 *              index, each contributing its free slots), or stays dropped
 *              when there is none.  Its gate becomes the new expert's
 *              score under the token's normaliser (divided by the sum of
 *              its originally chosen scores unless raw_gates).  An expert's
 *              rows are its kept assignments in token order, then its
 *              reassigned ones in ascending a.  Counts (and the aux loss)
 *              keep the routing decisions.  Used by moe_layer_forward and
 *              moe_dispatch_reassign; moe_dispatch rejects it.
 *   overflow_seed  64-bit key of the reassignment draws.
 */
typedef struct moe_problem {
  int32_t T;
  int32_t d_model;
  int32_t n_experts;
  int32_t top_k;
  int32_t d_ff;
  int32_t n_shared;
  int32_t capacity;
  int32_t act;
  int32_t dtype;
  float aux_coef;
  int32_t wquant;
  int32_t scoring;
  int32_t raw_gates;
  int32_t overflow;
  uint64_t overflow_seed;
} moe_problem;

/*
 * Expert weights (device pointers, problem dtype).
 *   GELU:   w1 = W1 [E, d_ff, d], b1 [E, d_ff], w2 = W2 [E, d, d_ff],
 *           b2 [E, d]; w_up must be NULL.
 *   SwiGLU: w1 = W_gate [E, d_ff, d], w_up = W_up [E, d_ff, d],
 *           w2 = W_down [E, d, d_ff]; b1, b2 must be NULL.
 *   Shared expert (n_shared = 1): the same tensors without the expert axis
 *   in shared_w1 / shared_w_up / shared_w2 / shared_b1 / shared_b2.
 *
 * With wquant = MOE_WQUANT_INT4 the matrices w1, w_up, w2 (and the shared
 * ones) hold 4-bit codes as written by moe_quantize_int4 for the stacked
 * [E*N, K] matrix (E*N*K/2 bytes), and *_q point to their (scale, offset)
 * pairs (E*N*(K/128)*2 float32), in that function's tiled order; the
 * weight is offset + code * scale.  Biases stay in the problem dtype.  The
 * *_q pointers are ignored (may be NULL) without quantisation.
 *
 * With wquant = MOE_WQUANT_BF16_TILED the matrices w1, w_up, w2 (and the
 * shared ones) hold the bf16 weights reordered by moe_tile_bf16 for the
 * stacked [E*N, K] matrix (same size); biases are unchanged.  The values
 * and the results are those of the row-major weights.
 */
typedef struct moe_expert_weights {
  const void* w1;
  const void* w_up;
  const void* w2;
  const void* b1;
  const void* b2;
  const void* shared_w1;
  const void* shared_w_up;
  const void* shared_w2;
  const void* shared_b1;
  const void* shared_b2;
  const float* w1_q;
  const float* w_up_q;
  const float* w2_q;
  const float* shared_w1_q;
  const float* shared_w_up_q;
  const float* shared_w2_q;
} moe_expert_weights;

/*
 * Per-expert capacity: the ideal share T*k/E times the capacity factor
 * cf_num/cf_den, truncated, and at least 1 ([LBS] The Capacity Factor).
 * Exact integer arithmetic.  Host-only.  Returns -1 on bad arguments
 * (T < 0, k < 1, E < 1, cf_num <= 0, cf_den <= 0) or overflow of int32.
 */
int32_t moe_capacity(int32_t T, int32_t top_k, int32_t n_experts,
                     int32_t cf_num, int32_t cf_den);

/*
 * Workspace bytes needed by every entry point below for problem `p`
 * (one size serves all of them).  Host-only; writes *bytes.  For batches
 * large enough for the tiled expert GEMMs the size includes one float32
 * partial tile (256 KiB) and one counter per compute unit of the current
 * device (the K split of the last round of tiles), so query it with the
 * device that will run the calls current.
 * Returns MOE_EINVAL / MOE_ENOTSUP for a problem the library rejects.
 */
int32_t moe_workspace_bytes(const moe_problem* p, size_t* bytes);

/*
 * Step 1, route ([RC] How a sparse MoE layer works; [LBS] Gating Mechanism;
 * [GN] The router, DeepSeek-V3).
 *   x            [T, d] problem dtype.
 *   w_router     [E, d] float32.
 *   router_bias  [E] float32 or NULL: added to the logits (changes choice
 *                and gates).
 *   select_bias  [E] float32 or NULL: added to the float32 logits for the
 *                choice only; gates and probabilities ignore it.
 *   logits       [T, E] float32 output, or NULL to skip writing it.
 *   topk_idx     [T, k] int32 output: chosen experts in descending order of
 *                selection key; equal keys go to the lower expert index.
 *   topk_gate    [T, k] float32 output: gates, summing to 1 per token.
 *   prob_mean    [E] float32 output: mean over tokens of softmax(logits),
 *                the P of the aux loss (0 when T = 0).
 */
int32_t moe_route(const moe_problem* p, const void* x, const float* w_router,
                  const float* router_bias, const float* select_bias,
                  float* logits, int32_t* topk_idx, float* topk_gate,
                  float* prob_mean, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/*
 * Step 2, dispatch and aux loss ([RC] capacity check; [LBS] The Capacity
 * Factor, The Load Balancing Problem).  Assignment a = t*k + j is slot j of
 * token t.
 *   topk_idx   [T, k] int32 input (each row: k distinct experts in [0, E)).
 *   prob_mean  [E] float32 input; may be NULL only if aux_loss is NULL.
 *   counts     [E] int32 output: assignments routed to each expert, before
 *              the capacity cut.
 *   offsets    [E+1] int32 output: exclusive scan of kept counts
 *              (kept = min(count, capacity), or count without a cap).
 *   perm       [T*k] int32 output: rows [offsets[e], offsets[e+1]) hold the
 *              kept assignment ids of expert e in ascending token order;
 *              entries from offsets[E] on are set to -1.
 *   slot_of    [T*k] int32 output: row of perm holding assignment a, or -1
 *              if a was dropped.
 *   n_dropped  [1] int32 output: T*k - offsets[E].
 *   aux_loss   [1] float32 output or NULL: alpha*E*sum_e (count_e/T)*P_e,
 *              0 when T = 0.
 */
int32_t moe_dispatch(const moe_problem* p, const int32_t* topk_idx,
                     const float* prob_mean, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* slot_of,
                     int32_t* n_dropped, float* aux_loss, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Step 2 with overflow reassignment (p->overflow = MOE_OVERFLOW_REASSIGN,
 * see moe_problem): the outputs of moe_dispatch, where kept and offsets
 * include the reassigned rows, plus in-place updates of the routing of the
 * reassigned slots.
 *   topk_idx   [T, k] int32 in/out: a reassigned slot gets its new expert.
 *   topk_gate  [T, k] float32 in/out: a reassigned slot gets its new gate.
 *   logits     [T, E] float32 input: the router logits moe_route wrote
 *              (the new gates need the token's scores).
 *   prob_mean, counts, offsets, perm, slot_of, n_dropped, aux_loss: as in
 *              moe_dispatch (counts and aux from the routing decisions
 *              before the cut and before reassignment).
 * The draws are sequential in a (each takes a free slot).  With one slot
 * per token (k = 1, at most 16384 possible draws, 65536 slots and 512
 * experts) every draw finds a slot while slots last, and the whole sequence
 * is decoded in parallel in one 1024-thread workgroup (about 2.2 us per
 * hundred drops on the Switch-shaped layer: 0.30 ms for 13721); otherwise
 * one wave walks the drops in order (about 10 us per hundred).
 */
int32_t moe_dispatch_reassign(const moe_problem* p, int32_t* topk_idx,
                              float* topk_gate, const float* logits,
                              const float* prob_mean, int32_t* counts,
                              int32_t* offsets, int32_t* perm,
                              int32_t* slot_of, int32_t* n_dropped,
                              float* aux_loss, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Steps 3-4, expert FFNs over each expert's kept rows ([RC]; [GN]
 * Implementing a complete MoE layer; [HA]: group the tokens by expert and
 * run each expert once over its batch).
 *   x        [T, d] input.
 *   perm, offsets  as written by moe_dispatch.
 *   w        expert weights (see moe_expert_weights).
 *   y        [T*k + n_shared*T, d] output, problem dtype: row r <
 *            offsets[E] is expert e (offsets[e] <= r < offsets[e+1]) applied
 *            to token perm[r] / k; row T*k + t is the shared expert applied
 *            to token t.  Rows [offsets[E], T*k) are not written.
 */
int32_t moe_expert_ffn(const moe_problem* p, const void* x,
                       const int32_t* perm, const int32_t* offsets,
                       const moe_expert_weights* w, void* y, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * Step 3 alone, the up projection ([RC]; [GN] Implementing a complete MoE
 * layer): h[r] = act(x[token(r)] . W1^T) for every routed row
 * r < offsets[E] (token(r) = perm[r] / k) and every shared row T*k + t
 * (token t).  SwiGLU: silu(x . W_gate^T) * (x . W_up^T); GELU:
 * gelu(x . W1^T + b1).
 *   h   [T*k + n_shared*T, d_ff] output, problem dtype; rows
 *       [offsets[E], T*k) are not written.
 *   ws  optional workspace (NULL with ws_bytes 0, or at least
 *       moe_workspace_bytes): with it the large-batch GEMM may split its
 *       last round of tiles along K (same results up to summation order);
 *       only its split area is used.
 */
int32_t moe_expert_up(const moe_problem* p, const void* x,
                      const int32_t* perm, const int32_t* offsets,
                      const moe_expert_weights* w, void* h, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/*
 * Step 4 alone, the down projection: y[r] = h[r] . W2^T (+ b2 for GELU) for
 * the same rows as moe_expert_up.
 *   h   [T*k + n_shared*T, d_ff] input as written by moe_expert_up.
 *   y   [T*k + n_shared*T, d] output, problem dtype.
 *   ws  optional workspace, as for moe_expert_up.
 */
int32_t moe_expert_down(const moe_problem* p, const void* h,
                        const int32_t* offsets, const moe_expert_weights* w,
                        void* y, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * Step 5, combine ([RC]: weighted sum plus residual; [LBS] Token Dropping:
 * a dropped slot contributes zero; [FA] Concept).
 *   x_residual  [T, d] or NULL (NULL omits the residual, as the [LBS], [HA]
 *               and [GN] snippets do).
 *   y           [T*k + n_shared*T, d] as written by moe_expert_ffn.
 *   slot_of     [T*k], topk_gate [T, k] as written by dispatch / route.
 *   out         [T, d] output, problem dtype:
 *               out[t] = x[t] + y[T*k+t] (shared) + sum over slots j with
 *               slot_of[t*k+j] >= 0 of gate[t,j] * y[slot_of[t*k+j]],
 *               accumulated in float32 in that order and rounded once.
 *               Surviving gates are not renormalised.
 */
int32_t moe_combine(const moe_problem* p, const void* x_residual,
                    const void* y, const int32_t* slot_of,
                    const float* topk_gate, void* out, hipStream_t stream);

/*
 * The whole layer: steps 1-5 and the aux loss, enqueued back to back with
 * no host synchronisation.  Outputs:
 *   out        [T, d] problem dtype (residual always added: [RC]).
 *   aux_loss   [1] float32 or NULL.
 *   counts     [E] int32 or NULL (pre-capacity assignments per expert).
 *   n_dropped  [1] int32 or NULL.
 *   topk_idx   [T, k] int32 or NULL (the routing decisions).
 * Intermediates live in the workspace.
 */
int32_t moe_layer_forward(const moe_problem* p, const void* x,
                          const float* w_router, const float* router_bias,
                          const float* select_bias,
                          const moe_expert_weights* w, void* out,
                          float* aux_loss, int32_t* counts,
                          int32_t* n_dropped, int32_t* topk_idx, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, outputs and results as moe_layer_forward,
 * without the workspace: the intermediates live in a scratch area of
 * MOE_NOALLOC_SCRATCH_BYTES that the library's code object holds on each
 * GPU it runs on, from the first call on that GPU until the process ends.
 * The call itself allocates nothing (no hipMalloc, no allocating library
 * routine); the first call on a GPU looks up the scratch's device address.
 *   Limit: the problem's intermediates must fit the scratch, which holds
 *   decode-sized batches (about 450 tokens of the Mixtral-shaped layer:
 *   k * (d_ff + d_model) * 2 bytes per token for H and Y, plus small
 *   routing buffers); beyond it the call returns MOE_EWORKSPACE and
 *   enqueues nothing.  The tiled expert GEMMs never split their last round
 *   along K here (no room is kept for the partial tiles); results agree with
 *   moe_layer_forward up to the float32 summation order of those tiles and
 *   are bit-identical wherever no tile is split.
 *   Concurrency: every call on a GPU uses that GPU's one scratch area, and
 *   each call leaves its intermediates there; calls that overlap on one GPU
 *   (on different streams, or from different threads without ordering)
 *   race and give undefined results.  Calls on one stream are ordered.
 */
int32_t moe_layer_forward_noalloc(const moe_problem* p, const void* x,
                                  const float* w_router,
                                  const float* router_bias,
                                  const float* select_bias,
                                  const moe_expert_weights* w, void* out,
                                  float* aux_loss, int32_t* counts,
                                  int32_t* n_dropped, int32_t* topk_idx,
                                  hipStream_t stream);

/*
 * Group-wise 4-bit round-to-nearest quantisation of a bf16 weight matrix
 * ([LBS] Production Considerations, Quantization for MoE: 4-bit expert
 * weights cut Mixtral 8x7B's weights from about 93 GB to about 26 GB).
 *   w        [rows, K] bf16 input; rows a multiple of 16 (stacked expert
 *            matrices [E, N, K] count as E*N rows), K a positive multiple
 *            of 128.
 *   codes    rows*K/2 bytes output.  Per group of 128 consecutive weights
 *            of a row: lo = min, hi = max, scale = (hi - lo) / 15,
 *            code = rint((w - lo) / scale) clamped to 0..15, ties to even,
 *            in float32 with correctly rounded division; a constant group
 *            gets scale 0 and code 0.  The weight is lo + code * scale.
 *            Storage (the GEMM's operand order): one 1024-byte tile per 16
 *            rows x one group, tile (r/16, g) at ((r/16)*(K/128) + g)*1024;
 *            in a tile, 16-byte slot m = r%16 + 16*kq holds row r's
 *            weights kq*32 .. kq*32+31 of the group as four little-endian
 *            32-bit words (word h: weights kq*32 + 8h + 0..7); in a word of
 *            eight consecutive weights k0..k7, nibble i holds k_(2i) for
 *            i < 4 and k_(2(i-4)+1) for i >= 4.
 *   qparams  rows*(K/128)*2 float32 output: one 128-byte tile per 16 rows x
 *            one group, at ((r/16)*(K/128) + g)*16 + r%16 the pair
 *            (scale, lo) of row r.
 * rows may be 0.  Returns MOE_EINVAL for null pointers or rows < 0,
 * MOE_ENOTSUP when K is not a positive multiple of 128, rows is not a
 * multiple of 16, or rows * K / 8 reaches 2^32 (split larger matrices by
 * rows).
 */
int32_t moe_quantize_int4(const void* w, int64_t rows, int32_t K,
                          void* codes, float* qparams, hipStream_t stream);

/*
 * Reorder a row-major bf16 matrix [rows, K] (a stack of expert matrices
 * [E*N, K]) into the tiled order read by the expert GEMMs when wquant =
 * MOE_WQUANT_BF16_TILED.  For the callers that keep expert weights
 * resident and serve many batches: the layout lets every weight load of
 * the GEMMs read 1 KiB of consecutive bytes already in matrix-core
 * operand order, instead of 16-byte pieces of 8 or 16 rows that must be
 * reshuffled through LDS.  A storage order of this library, not of the
 * method: tile (rb, kb) of 16 rows x 32 columns (1 KiB) sits at tile index
 * rb * (K/32) + kb; inside it, 16-byte piece 16*q + r holds row 16*rb + r,
 * columns 32*kb + 8*q .. 32*kb + 8*q + 7.  A permutation: out has rows*K
 * bf16 like w.
 *   w     [rows, K] bf16, device.
 *   rows  a multiple of 16 (>= 0); K a positive multiple of 32.
 *   out   rows*K bf16, device, must not overlap w.
 * Enqueued on stream.  MOE_EINVAL for NULL pointers with rows > 0 or
 * negative rows, MOE_ENOTSUP for other sizes.
 */
int32_t moe_tile_bf16(const void* w, int64_t rows, int32_t K, void* out,
                      hipStream_t stream);

/*
 * One step of auxiliary-loss-free balancing ([GN] DeepSeek-V3: the selection
 * bias of an over-loaded expert decreases, that of an under-loaded expert
 * increases, adjusted during training):
 *   select_bias[e] += gamma * sign(mean count - counts[e])
 * with mean count = sum(counts) / E; the sign is decided exactly in integer
 * arithmetic (sum(counts) - E * counts[e]), the update is one float32
 * addition.
 *   counts       [E] int32 input: pre-capacity assignments per expert, as
 *                written by moe_dispatch.
 *   select_bias  [E] float32, updated in place.
 *   gamma        bias update speed (finite).
 * Only n_experts of `p` is read.  Returns MOE_EINVAL for a bad problem,
 * null pointers or a non-finite gamma.
 */
int32_t moe_update_select_bias(const moe_problem* p, const int32_t* counts,
                               float* select_bias, float gamma,
                               hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
