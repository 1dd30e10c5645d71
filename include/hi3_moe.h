/*
 * hi3_moe.h - C ABI of the routed-expert MoE feed-forward layer of the
 * HunyuanImage-3.0 decoder, for AMD MI355X (gfx950).
 *
 * What the layer computes, per real (non-padding) token row x[t] of length H:
 *
 *   logits = W_r x (W_r is [E, H] fp32, the router kept in fp32:
 *            HunyuanImage-3.0 model-coverage page, "Train"; model API page,
 *            HunyuanImage3ForCausalMM, 'mlp.gate' kept in fp32)
 *   p      = softmax(logits) over all E experts (fp32); take the top K;
 *            renormalise the K selected p to sum to 1 (model API page,
 *            build_moe_config: softmax over all experts, top-k, renormalized,
 *            one shared expert). The top K is taken on the fp32 logits, the
 *            exact order of p (unaffected by fp32 underflow of small p);
 *            equal logits: lower expert index first.
 *   y_e    = W2[e] (SiLU(g) * u) with [u; g] = W13[e] x, where W13[e] is
 *            [2I, H] holding the up rows first and the gate rows second
 *            (layers API page, HunyuanSharedMLP: gate_and_up_proj holds
 *            [up; gate], up first; model-coverage page: fused [up; gate]
 *            expert projections converted to grouped experts)
 *   out[t] = sum_k w_k y_{e_k} + SharedSwiGLU(x[t])  (model API page,
 *            HunyuanImage3Block: routed experts plus the fused shared expert;
 *            technical report section 3.1.1: 64 experts, 8 active, one shared
 *            MLP)
 *
 * Numeric contract (bf16 layers): the router runs in fp32 with products
 * formed exactly; expert and shared projections accumulate in fp32; the
 * SwiGLU activation h is stored as bf16; y stays fp32; the combine sums in
 * fp32 in the order w_0 y_0 + w_1 y_1 + ... + shared and rounds once to bf16
 * (nearest, ties to even). fp32 layers keep every value in fp32.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise; tensors are dense,
 *    row-major, in the layouts given; every pointer must be 16-byte aligned.
 *  - The caller owns every buffer and every stream. The library allocates
 *    no device memory, keeps no pointer after returning and has no global
 *    mutable state: calls on different streams with different workspaces
 *    may run concurrently from any host threads.
 *  - Work is enqueued on hip_stream (a hipStream_t; NULL = the null stream)
 *    and the call returns without waiting. There is no device-to-host
 *    synchronisation inside any call.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    validation error nothing is enqueued, nothing is written and a negative
 *    status is returned. HI3_E_HIP means a launch failed after validation
 *    (earlier stages of the call may have run).
 *  - pad_mask is a [T] uint8 array, nonzero at padding rows (the polarity of
 *    the pages' padding_mask: true at padding). NULL means no padding.
 *    Padding rows are never read from x and never written to out.
 *  - T = 0 returns HI3_OK and enqueues nothing.
 *  - Builder's limits (HI3_E_UNSUPPORTED otherwise): dtype HI3_F32 or
 *    HI3_BF16; 1 <= K <= E <= 64; H, I, I_shared multiples of 64;
 *    T * K < 2^31.
 */
#ifndef HI3_MOE_H
#define HI3_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of x, expert weights, shared weights and out. The router weight is
 * always fp32. bf16 values are raw 16-bit bfloat16 patterns. */
#define HI3_F32 0
#define HI3_BF16 1

/* status codes */
#define HI3_OK 0
#define HI3_E_NULL (-1)        /* a required pointer is NULL */
#define HI3_E_SHAPE (-2)       /* T < 0, a size <= 0, or K > E */
#define HI3_E_UNSUPPORTED (-3) /* outside the builder's limits above */
#define HI3_E_WORKSPACE (-4)   /* workspace smaller than required */
#define HI3_E_HIP (-5)         /* a HIP launch failed */
#define HI3_E_SCRATCH (-6)     /* sizes too large for hi3_moe_forward_noalloc */

/* Number of timed stages of hi3_moe_forward_instrumented. */
#define HI3_NUM_STAGES 5
/* Number of timed stages of hi3_moe_backward_instrumented. */
#define HI3_NUM_BWD_STAGES 10

/*
 * Workspace bytes that hi3_moe_forward and hi3_moe_forward_norm_residual
 * need for these sizes (host-only, no HIP call). With I = I_shared = 0 it
 * returns the smaller amount that hi3_moe_route and hi3_moe_dispatch need;
 * the forward amount also serves them. Returns 0 for invalid sizes and for
 * T = 0.
 */
size_t hi3_moe_workspace_size(int64_t T, int32_t H, int32_t E, int32_t K,
                              int32_t I, int32_t I_shared, int32_t dtype);

/*
 * Router only (softmax over all experts, top-k, renormalised).
 *   x           [T, H] dtype, input rows (the [batch, sequence, hidden] input
 *               of the pages' Block.forward, flattened).
 *   w_router    [E, H] fp32 (linear layout [out, in]).
 *   pad_mask    [T] uint8 or NULL.
 *   topk_idx    [T, K] int32 out: per row the K expert ids in descending
 *               logit (so non-increasing weight), equal logits by ascending
 *               id; padding rows -1.
 *   topk_w      [T, K] fp32 out: renormalised gate weights; padding rows 0.
 *   expert_counts [E] int32 out or NULL: number of real rows routed to each
 *               expert.
 *   workspace   device memory of at least
 *               hi3_moe_workspace_size(T, H, E, K, 0, 0, dtype) bytes.
 */
int hi3_moe_route(const void *x, const float *w_router, const uint8_t *pad_mask,
                  int64_t T, int32_t H, int32_t E, int32_t K, int32_t dtype,
                  int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                  void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Dispatch only: groups given routes by expert (the pages' "grouped
 * experts", model-coverage page, "Model Class"). Slots are numbered expert
 * by expert; inside one expert, pairs keep ascending (token, k) order.
 *   topk_idx      [T, K] int32 in, ids in [0, E); rows with pad_mask set
 *                 are ignored (their ids are not read).
 *   x             [T, H] dtype; read only when x_sorted is not NULL.
 *   expert_offsets [E + 1] int32 out: first slot of each expert; the last
 *                 entry is the number of real (token, k) pairs S.
 *   perm_token    [T * K] int32 out: token of each slot; entries >= S are
 *                 left unwritten.
 *   slot_of       [T * K] int32 out: slot of pair (t, k), -1 for padding.
 *   x_sorted      [T * K, H] dtype out or NULL: x_sorted[s] = x[perm_token[s]]
 *                 for s < S.
 *   workspace     as for hi3_moe_route.
 */
int hi3_moe_dispatch(const int32_t *topk_idx, const uint8_t *pad_mask, const void *x,
                     int64_t T, int32_t H, int32_t E, int32_t K, int32_t dtype,
                     int32_t *expert_offsets, int32_t *perm_token, int32_t *slot_of,
                     void *x_sorted, void *workspace, size_t workspace_bytes,
                     void *hip_stream);

/*
 * The whole layer: router, dispatch, grouped [up; gate] projection with the
 * SwiGLU epilogue, grouped down projection, shared expert, combine; every
 * kernel on hip_stream (the shared expert's rows ride in the grouped
 * launches as one more group).
 *   x                [T, H] dtype.
 *   w_router         [E, H] fp32.
 *   w_up_gate        [E, 2*I, H] dtype; rows [0, I) up, [I, 2I) gate.
 *   w_down           [E, H, I] dtype.
 *   w_shared_up_gate [2*I_shared, H] dtype, same [up; gate] order.
 *   w_shared_down    [H, I_shared] dtype.
 *   pad_mask         [T] uint8 or NULL.
 *   out              [T, H] dtype out; padding rows are not written. Must
 *                    not overlap x (the residual add is the caller's).
 *   topk_idx, topk_w, expert_counts: as in hi3_moe_route, each may be NULL.
 *   workspace        at least hi3_moe_workspace_size(T, H, E, K, I,
 *                    I_shared, dtype) bytes.
 */
int hi3_moe_forward(const void *x, const float *w_router, const void *w_up_gate,
                    const void *w_down, const void *w_shared_up_gate,
                    const void *w_shared_down, const uint8_t *pad_mask,
                    int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                    int32_t I_shared, int32_t dtype, void *out,
                    int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                    void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * hi3_moe_forward with the shared expert (model API page, HunyuanImage3Block:
 * the fused shared expert beside the routed ones) on a second stream of the
 * caller's: its rows need nothing from the routing, so its two GEMMs run
 * alongside the router and dispatch. Same arguments, results (bit for bit)
 * and workspace as hi3_moe_forward, plus:
 *   side_stream  a hipStream_t of the same device, other than hip_stream, or
 *                NULL. It is used only when hi3_moe_forward_shared_on_side
 *                says so (bf16, no padding mask); otherwise, and when NULL or
 *                equal to hip_stream, the call is exactly hi3_moe_forward.
 * The side stream waits for an event recorded on hip_stream at the start of
 * the call, and hip_stream waits for an event recorded on the side stream
 * before the combine: work enqueued on hip_stream after the call is ordered
 * after all of it, work enqueued on side_stream after the call is not. The
 * two events are created and destroyed inside the call (no device memory);
 * a stream capture of hip_stream takes the side stream's work into the
 * same graph (fork and join).
 */
int hi3_moe_forward_overlap(const void *x, const float *w_router, const void *w_up_gate,
                            const void *w_down, const void *w_shared_up_gate,
                            const void *w_shared_down, const uint8_t *pad_mask,
                            int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                            int32_t I_shared, int32_t dtype, void *out,
                            int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                            void *workspace, size_t workspace_bytes, void *hip_stream,
                            void *side_stream);

/*
 * hi3_moe_forward for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results (bit for bit) as hi3_moe_forward, without the
 * workspace: the library's own scratch stands in for it, a device array of
 * HI3_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends (obtained on the first call with that device current;
 * hip_stream must belong to the current device, else HI3_E_UNSUPPORTED).
 * Sizes whose hi3_moe_workspace_size exceeds HI3_NOALLOC_SCRATCH_BYTES are
 * rejected with HI3_E_SCRATCH before anything is enqueued (at H = 4096,
 * E = 64, K = 8, I = I_shared = 3072 in bf16: up to about 620 tokens).
 * The call allocates nothing. Every call on one GPU uses that GPU's one
 * scratch: calls that overlap on a GPU (other streams, other host threads)
 * race and must be ordered by the caller. The scratch keeps the last call's
 * contents; no part of it needs to start at zero.
 */
#define HI3_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int hi3_moe_forward_noalloc(const void *x, const float *w_router, const void *w_up_gate,
                            const void *w_down, const void *w_shared_up_gate,
                            const void *w_shared_down, const uint8_t *pad_mask,
                            int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                            int32_t I_shared, int32_t dtype, void *out,
                            int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                            void *hip_stream);

/*
 * hi3_moe_forward_overlap (hi3_moe_forward when side_stream is NULL) with
 * per-stage timing: stage_events holds HI3_NUM_STAGES + 1 hipEvent_t handles
 * created by the caller; event i is recorded on hip_stream just before stage
 * i is enqueued and the last one after the final stage (stage names:
 * hi3_moe_stage_name). Same results as the untimed calls. When the shared
 * expert runs on the side stream, the GEMM stages time the routed experts
 * alone, and the shared expert's GEMMs run during the routing stages and the
 * first GEMM. stage_events must not be NULL; an entry that is NULL is not
 * recorded (a caller timing one stage passes only the two events around it).
 */
int hi3_moe_forward_instrumented(const void *x, const float *w_router,
                                 const void *w_up_gate, const void *w_down,
                                 const void *w_shared_up_gate,
                                 const void *w_shared_down, const uint8_t *pad_mask,
                                 int64_t T, int32_t H, int32_t E, int32_t K,
                                 int32_t I, int32_t I_shared, int32_t dtype,
                                 void *out, int32_t *topk_idx, float *topk_w,
                                 int32_t *expert_counts, void *workspace,
                                 size_t workspace_bytes, void *hip_stream,
                                 void *side_stream, void *const *stage_events);

/*
 * The block's RMSNorm ahead of the layer (layers API page, HunyuanRMSNorm:
 * normalize in fp32 over the hidden axis, return weight * x in the input
 * dtype, eps 1e-5 by default; model API page, HunyuanImage3Block:
 * post_attention_layernorm before the experts). For every real row:
 *   m = mean of x^2 (accumulated in fp64, rounded to fp32), d = m + eps in
 *   fp32, r = 1 / sqrt(d) rounded once to fp32, n = x * r as an fp32 product
 *   converted to dtype, xn = weight * n rounded once to dtype.
 *   x        [T, H] dtype.
 *   weight   [H] dtype.
 *   eps      finite, >= 0 (HI3_E_UNSUPPORTED otherwise).
 *   pad_mask [T] uint8 or NULL; padding rows of xn are not written.
 *   xn       [T, H] dtype out; may be x itself.
 * H must be a multiple of 64. No workspace.
 */
int hi3_moe_rmsnorm(const void *x, const void *weight, float eps, const uint8_t *pad_mask,
                    int64_t T, int32_t H, int32_t dtype, void *xn, void *hip_stream);

/*
 * The layer inside its decoder block (model API page, HunyuanImage3Block:
 * a pre-norm layer; its MoE half is h + layer(post_attention_layernorm(h))):
 *   out[t] = h[t] + layer(RMSNorm(h)[t])
 * with RMSNorm as in hi3_moe_rmsnorm and the layer as in hi3_moe_forward;
 * the residual is added in fp32 after the shared term, before the one
 * rounding to dtype. Arguments as in hi3_moe_forward, plus:
 *   h            [T, H] dtype: the residual stream (takes the place of x).
 *   norm_weight  [H] dtype, must not be NULL.
 *   eps          finite, >= 0.
 *   out          [T, H] dtype out; may be h itself (updated in place), must
 *                not overlap it otherwise. Padding rows are not written.
 * Routes (topk_idx, topk_w, expert_counts) are those of the normalised rows.
 * Same workspace size as hi3_moe_forward.
 */
int hi3_moe_forward_norm_residual(const void *h, const void *norm_weight, float eps,
                                  const float *w_router, const void *w_up_gate,
                                  const void *w_down, const void *w_shared_up_gate,
                                  const void *w_shared_down, const uint8_t *pad_mask,
                                  int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                                  int32_t I_shared, int32_t dtype, void *out,
                                  int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                                  void *workspace, size_t workspace_bytes,
                                  void *hip_stream);

/*
 * Backward pass of the layer, for fine-tuning (HunyuanImage-3.0
 * model-coverage page, "Train": LoRA and full fine-tuning of the MoE
 * decoder). Given dout = dL/dout for the rows of hi3_moe_forward, computes
 * the gradients of L = sum over real rows t of dout[t] . out[t] with the
 * routes held fixed (the top-k choice is piecewise constant; the router gets
 * its gradient through the renormalised weights), at the values the forward
 * keeps: fp32 router probabilities and weights, fp32 u and g, h rounded to
 * dtype. Per real row, with w_k, e_k the k-th weight and expert:
 *   dy_k = w_k dout, dh_k = W2[e_k]^T dy_k, du = dh SiLU(g),
 *   dg = dh u SiLU'(g); the shared expert the same with weight 1;
 *   a_k = dh_k . h_k, dl_k = a_k - w_k sum_j a_j (the logit gradient; zero
 *   at unselected experts);
 *   dx = sum_k W13[e_k]^T [du; dg]_k + W13s^T [du; dg]_s + sum_k dl_k W_r[e_k]
 *   dW2[e] = sum dy h^T, dW13[e] = sum [du; dg] x^T over e's rows,
 *   dW_r[e] = sum dl x over e's rows; shared weights over all real rows.
 * The routes and the [up; gate] projection are recomputed inside the call.
 * Arguments as in hi3_moe_forward, plus:
 *   dout             [T, H] dtype.
 *   dx               [T, H] dtype out or NULL; padding rows are not written.
 *   dw_router        [E, H] fp32 out or NULL.
 *   dw_up_gate       [E, 2*I, H] dtype out or NULL ([up; gate] rows).
 *   dw_down          [E, H, I] dtype out or NULL.
 *   dw_shared_up_gate [2*I_shared, H] dtype out or NULL.
 *   dw_shared_down   [H, I_shared] dtype out or NULL.
 *   workspace        at least hi3_moe_backward_workspace_size(...) bytes.
 * A NULL output is not computed. Weight gradients are overwritten (not
 * accumulated); those of experts that no row selects are zero; sums are
 * accumulated in fp32 in a fixed order and rounded once (deterministic).
 * T = 0 zero-fills the requested weight gradients; x, dout and the weights
 * are then not read and may be NULL, and no workspace is needed.
 */
size_t hi3_moe_backward_workspace_size(int64_t T, int32_t H, int32_t E, int32_t K,
                                       int32_t I, int32_t I_shared, int32_t dtype);

int hi3_moe_backward(const void *x, const float *w_router, const void *w_up_gate,
                     const void *w_down, const void *w_shared_up_gate,
                     const void *w_shared_down, const uint8_t *pad_mask, const void *dout,
                     int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                     int32_t I_shared, int32_t dtype, void *dx, float *dw_router,
                     void *dw_up_gate, void *dw_down, void *dw_shared_up_gate,
                     void *dw_shared_down, void *workspace, size_t workspace_bytes,
                     void *hip_stream);

/*
 * hi3_moe_backward with per-stage timing: HI3_NUM_BWD_STAGES + 1 events,
 * recorded as in hi3_moe_forward_instrumented (names:
 * hi3_moe_backward_stage_name: routes, dispatch, slot gathers, the GEMM
 * through the down projection, the recomputed [up; gate] projection with
 * the SwiGLU backward in its epilogue, the GEMM through [up; gate], the
 * logit gradient and dx, the router weight gradient, the two expert weight
 * gradients). For fp32 layers the recompute runs first and is timed with the
 * gathers (its u and g feed the down-projection GEMM's epilogue), and after
 * hi3_moe_forward_train there is no recompute. stage_events must not be NULL.
 */
int hi3_moe_backward_instrumented(const void *x, const float *w_router,
                                  const void *w_up_gate, const void *w_down,
                                  const void *w_shared_up_gate, const void *w_shared_down,
                                  const uint8_t *pad_mask, const void *dout, int64_t T,
                                  int32_t H, int32_t E, int32_t K, int32_t I,
                                  int32_t I_shared, int32_t dtype, void *dx,
                                  float *dw_router, void *dw_up_gate, void *dw_down,
                                  void *dw_shared_up_gate, void *dw_shared_down,
                                  void *workspace, size_t workspace_bytes,
                                  void *hip_stream, void *const *stage_events);

/*
 * Backward of the block entry point hi3_moe_forward_norm_residual
 * (out = h + layer(RMSNorm(h)); model API page, HunyuanImage3Block, a
 * pre-norm layer; the pages' fine-tuning, model-coverage page, "Train"):
 * the layer's gradients at the normalised rows as in hi3_moe_backward, then
 * RMSNorm's, at the forward's fp32 r with the roundings of n and xn passed
 * straight through, plus the residual:
 *   g = dL/dxn (the layer's dx, kept in fp32), dx_norm = r w g - r^3 h s / H
 *   with s = sum over the row of h w g, dh = dout + dx_norm (rounded once),
 *   dnorm_weight = sum over real rows of g * dtype(h r).
 * Arguments as in hi3_moe_backward, plus:
 *   h             [T, H] dtype: the block input (takes the place of x).
 *   norm_weight   [H] dtype, must not be NULL (unless T = 0).
 *   eps           finite, >= 0.
 *   dh            [T, H] dtype out or NULL (takes the place of dx); padding
 *                 rows are not written.
 *   dnorm_weight  [H] dtype out or NULL.
 * Workspace: hi3_moe_backward_workspace_size(...) bytes.
 */
int hi3_moe_backward_norm_residual(const void *h, const void *norm_weight, float eps,
                                   const float *w_router, const void *w_up_gate,
                                   const void *w_down, const void *w_shared_up_gate,
                                   const void *w_shared_down, const uint8_t *pad_mask,
                                   const void *dout, int64_t T, int32_t H, int32_t E,
                                   int32_t K, int32_t I, int32_t I_shared, int32_t dtype,
                                   void *dh, void *dnorm_weight, float *dw_router,
                                   void *dw_up_gate, void *dw_down, void *dw_shared_up_gate,
                                   void *dw_shared_down, void *workspace,
                                   size_t workspace_bytes, void *hip_stream);

/*
 * A training step's pair (the pages' fine-tuning, model-coverage page,
 * "Train"): hi3_moe_forward_train is hi3_moe_forward (same arguments, same
 * out, routes and counts) that also leaves in its workspace the routes, the
 * dispatch maps, u and g (fp32) and h; hi3_moe_backward_after_forward is
 * hi3_moe_backward that takes them from there instead of recomputing the
 * router, the dispatch and the [up; gate] projection. The workspace must be
 * at least hi3_moe_backward_workspace_size(...) bytes for both calls; the
 * second call must get the same workspace, the same x, weights, pad_mask and
 * sizes, with nothing written to any of them in between (the library cannot
 * check this: it keeps no state). Results are bit-identical to
 * hi3_moe_forward and hi3_moe_backward on the same inputs.
 */
int hi3_moe_forward_train(const void *x, const float *w_router, const void *w_up_gate,
                          const void *w_down, const void *w_shared_up_gate,
                          const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                          int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                          int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                          int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                          void *hip_stream);

int hi3_moe_backward_after_forward(const void *x, const float *w_router,
                                   const void *w_up_gate, const void *w_down,
                                   const void *w_shared_up_gate, const void *w_shared_down,
                                   const uint8_t *pad_mask, const void *dout, int64_t T,
                                   int32_t H, int32_t E, int32_t K, int32_t I,
                                   int32_t I_shared, int32_t dtype, void *dx,
                                   float *dw_router, void *dw_up_gate, void *dw_down,
                                   void *dw_shared_up_gate, void *dw_shared_down,
                                   void *workspace, size_t workspace_bytes,
                                   void *hip_stream);

/* Static name of backward stage i (0 <= i < HI3_NUM_BWD_STAGES), else "?". */
const char *hi3_moe_backward_stage_name(int stage);

/*
 * 1 when hi3_moe_forward_overlap (and hi3_moe_forward_instrumented) given a
 * side stream runs the shared expert's GEMMs on it for these sizes, else 0
 * (also for sizes the forward rejects): bf16 and no padding mask.
 * Host-only.
 */
int hi3_moe_forward_shared_on_side(int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                                   int32_t I_shared, int32_t dtype, int32_t has_pad_mask);

/*
 * Measurement probe, not part of the layer: the bf16 matrix-core rate the
 * GPU holds with no memory traffic, reported beside the published dense
 * peak. Enqueues `blocks` blocks of 256 threads; each wave runs iters x 16
 * v_mfma_f32_32x32x16_bf16 in four independent chains on operands read once
 * from `operands` (device, 16-byte aligned, at least 8 KiB of bf16 values:
 * pass values with the statistics of real operands, since how much the
 * operands switch sets the clock the matrix cores hold under load).
 *   out   [blocks * 4] fp32 out (device): one value per wave.
 * Returns the FLOP the launch performs (> 0) or a negative status
 * (HI3_E_NULL, HI3_E_SHAPE for blocks or iters <= 0, HI3_E_UNSUPPORTED for
 * a misaligned pointer, HI3_E_HIP).
 */
int64_t hi3_moe_probe_mfma_bf16(const void *operands, float *out, int32_t blocks,
                                int32_t iters, void *hip_stream);

/* Static name of timed stage i (0 <= i < HI3_NUM_STAGES), else "?". */
const char *hi3_moe_stage_name(int stage);

/* Static description of a status code (host-only). */
const char *hi3_moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* HI3_MOE_H */
