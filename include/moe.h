/*
 * moe.h -- C ABI of libmoe.so: the forward pass of one Mixture-of-Experts
 * layer on one AMD MI355X (gfx950), as hand-written HIP kernels.
 *
 * The layer (page "MoE 模型原理：路由、专家负载、容量、通信与推理成本", wrblog.cn,
 * cited below as [MoE Principles]):
 *   router scores        s_t = W_r x_t + b_r                         (§2.1)
 *   softmax              p_{t,i} = exp(s_{t,i}) / sum_j exp(s_{t,j}) (§2.1)
 *   top-k                S_t = TopK(p_t, k)                          (§2.2)
 *   gates                p~_{t,i} = p_{t,i} / sum_{j in S_t} p_{t,j} (§2.2)
 *   capacity             C = ceil(c * T * k / E)                     (§4.1)
 *   first-come dispatch  token order, per-expert limit C, overflow dropped (§4.2, §4.3)
 *   expert FFN           FFN(x) = W2 sigma(W1 x + b1) + b2           (§1)
 *   combine              y_t = sum_{i in S_t} p~_{t,i} E_i(x_t)      (§2.2, §5)
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument other than `cfg` (a host pointer) is a DEVICE
 *    pointer owned by the caller. The library never allocates, frees,
 *    synchronises or prints; all work is enqueued on `stream` in order.
 *  - Row-major, last index contiguous. x [T,d]; W_r [E,d]; b_r [E];
 *    W1 [E,d_ff,d]; b1 [E,d_ff]; W2 [E,d,d_ff]; b2 [E,d]. W1[e] maps d -> d_ff.
 *  - x, W_r, W1, W2, x_perm, h, y_perm and y have element type cfg->dtype
 *    (MOE_F32 or MOE_BF16, bf16 = the top 16 bits of an IEEE fp32). Biases,
 *    logits, probabilities and gates are fp32 for both dtypes.
 *  - Top-k returns expert ids in descending score order; equal scores go to
 *    the lower expert index. The choice is made on fp32 logits.
 *  - Capacity is granted first-come in token order (a token's own k choices
 *    go to distinct experts, so they never compete). A dropped assignment
 *    contributes nothing; gates are not renormalised after drops; a token
 *    whose every assignment was dropped gets y_t = 0. Two optional rules
 *    change this (cfg->priority, cfg->reroute; see moe_config):
 *    rank-major priority, and moving an overflowing assignment to the
 *    token's next candidate expert instead of dropping it.
 *  - Dispatch layout: rows are expert-major and, within an expert, in token
 *    order, packed from row 0 without padding. rows = sum_e min(count_e, C)
 *    is never read back to the host; buffers indexed by row are sized by
 *    the bound max_rows = min(T*k, E*C) (see moe_max_rows). Entries at and
 *    beyond `rows` are left untouched.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code. Every argument is
 *    checked before the first launch: MOE_ERR_INVALID_ARG, _UNSUPPORTED and
 *    _WORKSPACE enqueue nothing. MOE_ERR_HIP (a launch or event call the HIP
 *    runtime refused) may leave the call's earlier kernels enqueued on
 *    `stream`; its results are then undefined. T == 0 is a valid no-op
 *    returning MOE_OK.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    on the same device (CU count) with the same GEMM block cap (see
 *    moe_set_gemm_max_blocks): the expert GEMMs' tile plan, and with it the
 *    order of some sums, follows the number of persistent blocks.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, bad sizes, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not implemented (shape/dtype combination) */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than moe_workspace_size */
  MOE_ERR_HIP = -4          /* a HIP launch or event call failed */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_ACT_RELU = 0, MOE_ACT_GELU_TANH = 1 };
enum { MOE_MAX_EXPERTS = 1024, MOE_MAX_TOPK = 16 };
/* Order in which arrivals at a full expert are served (moe_config.priority). */
enum { MOE_PRIORITY_TOKEN = 0, MOE_PRIORITY_RANK = 1 };

/* Stage boundaries for moe_layer_forward's optional events. */
enum {
  MOE_STAGE_ROUTE = 0,    /* router GEMM, softmax, top-k, gates, per-tile counts */
  MOE_STAGE_DISPATCH = 1, /* prefix sums, slots, capacity, token permutation */
  MOE_STAGE_GEMM1 = 2,    /* h = sigma(x_perm W1_e^T + b1_e), grouped over experts */
  MOE_STAGE_GEMM2 = 3,    /* y_perm = h W2_e^T + b2_e, grouped over experts */
  MOE_STAGE_COMBINE = 4,  /* gate-weighted gather back to token order */
  MOE_NUM_STAGES = 5
};

/*
 * The layer's shape and behaviour, validated at every entry point
 * ([MoE Principles] §12 lists what must be pinned: expert count and sizes,
 * top-k, capacity, combine rule, overflow behaviour).
 *   T            tokens in the call; the whole call is one routing group.
 *   d, d_ff      hidden and expert-hidden sizes. MOE_BF16 needs both to be
 *                multiples of 64 (else MOE_ERR_UNSUPPORTED).
 *   E, k         experts and experts per token: 1 <= k <= E <= MOE_MAX_EXPERTS,
 *                k <= MOE_MAX_TOPK.
 *   capacity     C >= 1 (from moe_capacity, or any caller choice; C >= T
 *                means nothing is ever dropped).
 *   renormalize  1: gates are the top-k probabilities divided by their sum;
 *                0: gates are the plain softmax probabilities.
 *   dtype        MOE_F32 or MOE_BF16.
 *   act          sigma: MOE_ACT_RELU or MOE_ACT_GELU_TANH
 *                (0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))).
 *   priority     MOE_PRIORITY_TOKEN: arrivals at an expert are served in
 *                token order (t, then the token's rank r).
 *                MOE_PRIORITY_RANK: in rank order (every token's first choice
 *                before any token's second choice, then token order).
 *   reroute      rounds of overflow re-routing R >= 0 ([MoE Principles] §4.3,
 *                second option; ai-master.cc EP engineering answer 001, §一:
 *                overflow goes to the next-best expert or is dropped).
 *                0: an overflowing assignment is dropped. R > 0: capacity is
 *                given out in rounds; round 0 offers the top-k assignments;
 *                before round j every unplaced assignment of a token takes,
 *                in rank order, the token's next candidate (the next expert
 *                in descending score order that the token has not been
 *                offered); arrivals are numbered from the expert's fill at
 *                the round's start, in priority order, and placed while the
 *                number is below C. An assignment served by a candidate is
 *                weighted by that expert's probability (divided by the same
 *                top-k sum when renormalising). The route then returns
 *                n_cand = min(E, k (1 + R)) candidates per token (see
 *                moe_candidates); n_cand must not exceed MOE_MAX_TOPK.
 */
typedef struct moe_config {
  int64_t T;
  int32_t d, d_ff, E, k, capacity, renormalize, dtype, act;
  int32_t priority, reroute;
} moe_config;

/*
 * Optional outputs of moe_layer_forward (device pointers; any may be NULL,
 * in which case that result stays in the workspace).
 *   topk_ids [T,k] int32, topk_gates [T,k] fp32, prob_sum [E] fp32
 *   (sum over tokens of p_{t,i}, for the load-balance statistics of
 *   [MoE Principles] §3.2), expert_counts [E] int32 (before capacity),
 *   expert_offsets [E+1] int32 (after capacity), slot [T,k] int32,
 *   row_of [T,k] int32 (-1 = dropped), row_token [max_rows] int32.
 *   With priority or re-routing (see moe_dispatch_reroute): topk_ids and
 *   topk_gates are [T,n_cand] candidate lists; served_ids [T,k] int32 and
 *   combine_gates [T,k] fp32 are the serving expert (-1 = dropped) and the
 *   combine weight (0 = dropped) of each assignment. Unused otherwise.
 *   h [max_rows,d_ff] (dtype): the first expert GEMM's output
 *   sigma(x W1_e^T + b1_e) per row, kept for the caller (rows >= offsets[E]
 *   untouched); moe_layer_backward ignores it.
 */
typedef struct moe_route_info {
  int32_t *topk_ids;
  float *topk_gates;
  float *prob_sum;
  int32_t *expert_counts;
  int32_t *expert_offsets;
  int32_t *slot;
  int32_t *row_of;
  int32_t *row_token;
  int32_t *served_ids;
  float *combine_gates;
  void *h;
} moe_route_info;

/*
 * C = ceil(c * T * k / E) ([MoE Principles] §4.1; page "Expert Parallelism：
 * 为什么让 Token 去找 Expert，而不是搬运参数？", section "Expert Capacity 和 Token
 * Dropping"), computed exactly from the binary value of c (host only, no GPU).
 * Errors: MOE_ERR_INVALID_ARG if C_out is NULL, T < 0, k < 1, E < 1, c is not
 * finite or c <= 0, or the result exceeds INT32_MAX. T == 0 gives C = 0.
 */
int32_t moe_capacity(int64_t T, int32_t k, int32_t E, double c, int32_t *C_out);

/* Candidates per token returned by moe_route: k, or min(E, k (1 + reroute))
 * with re-routing (host only). */
int32_t moe_candidates(const moe_config *cfg, int32_t *n_cand);

/* max_rows = min(T*k, E*C): the size of every row-indexed buffer (host only). */
int32_t moe_max_rows(const moe_config *cfg, int64_t *rows);

/* Workspace bytes moe_layer_forward needs; the stage entry points need no
 * more than this (host only). */
int32_t moe_workspace_size(const moe_config *cfg, size_t *bytes);

/* Caps the grid of the persistent expert GEMMs (forward and backward) at
 * `blocks` workgroups per launch, on every device; 0 (the default) runs one
 * per CU. For callers that keep CUs free for other work beside the layer,
 * such as an expert-parallel all-to-all pipelined with the expert
 * computation (ai-master.cc EP engineering answer 001, §二, compute-
 * communication overlap). The GEMMs lay out their tiles on the device for
 * whatever grid they get, so results stay within the layer's tolerance at
 * any cap (sums may round differently). Process-wide; applies to launches
 * issued after it returns (host only, no device call).
 * Errors: MOE_ERR_INVALID_ARG if blocks < 0. */
int32_t moe_set_gemm_max_blocks(int32_t blocks);

/*
 * Route ([MoE Principles] §2.1-§2.2; page "MiniMax 面试: MoE gate 与分布式通信",
 * mianshidashi.cn, 深入解析 01: the gate emits scores, top-k ids and weights).
 *   x [T,d], W_r [E,d] (dtype); b_r [E] fp32 or NULL (zero bias).
 *   out topk_ids [T,k] int32, topk_gates [T,k] fp32 (required); with
 *       re-routing [T,n_cand]: the top-k followed by the next candidates in
 *       descending score order, every weight divided by the top-k sum when
 *       renormalising;
 *   out prob_sum [E] fp32 or NULL; out logits [T,E] fp32 or NULL.
 *   ws: at least moe_workspace_size bytes, 256-byte aligned.
 */
int32_t moe_route(const moe_config *cfg, const void *x, const void *W_r, const float *b_r,
                  int32_t *topk_ids, float *topk_gates, float *prob_sum, float *logits,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch ([MoE Principles] §4.2 capacity assignment and §5 dispatch
 * metadata; MiniMax gate/communication page, 深入解析 02 and 06: counting,
 * prefix sum, permutation into a contiguous buffer). Recounts from topk_ids.
 *   in  x [T,d] (dtype), topk_ids [T,k] int32 (each row k distinct ids in [0,E)).
 *   out expert_counts [E] int32: count_e = |{t : e in S_t}| (before capacity).
 *   out expert_offsets [E+1] int32: prefix sums of n_e = min(count_e, C).
 *   out slot [T,k] int32: slot(t,e) = |{t' < t : e in S_t'}|.
 *   out row_of [T,k] int32: offsets[e] + slot if slot < C, else -1.
 *   out row_token [max_rows] int32: the token held by each row.
 *   out x_perm [max_rows,d] (dtype): x_perm[r] = x[row_token[r]] (bit copy).
 * With cfg->priority == MOE_PRIORITY_RANK the slots follow rank order
 * instead (slot = arrivals before it at that expert in rank order).
 * cfg->reroute must be 0 (else MOE_ERR_INVALID_ARG): re-routing also changes
 * the combine weights, which moe_dispatch_reroute returns.
 * Behaviour is undefined if an id is out of range or repeated within a row.
 */
int32_t moe_dispatch(const moe_config *cfg, const void *x, const int32_t *topk_ids,
                     int32_t *expert_counts, int32_t *expert_offsets, int32_t *slot,
                     int32_t *row_of, int32_t *row_token, void *x_perm, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch under any capacity rule of moe_config (priority, re-routing
 * rounds; [MoE Principles] §4.3). For cfg->reroute == 0 and token priority
 * it gives what moe_dispatch gives.
 *   in  x [T,d] (dtype); cand_ids [T,n_cand] int32, each row n_cand distinct
 *       ids in [0,E), best first; cand_gates [T,n_cand] fp32 (moe_route's
 *       outputs).
 *   out expert_counts [E] int32: top-k demand |{t : e in S_t}| (round 0).
 *   out expert_offsets [E+1] int32: prefix sums of the rows each expert
 *       finally holds (at most C).
 *   out slot [T,k] int32: the assignment's arrival number at the expert it
 *       was last offered to (its row within that expert when placed).
 *   out row_of [T,k] int32 (-1 = dropped), row_token [max_rows] int32;
 *       rows within an expert in slot order.
 *   out served_ids [T,k] int32 or NULL: serving expert, -1 if dropped.
 *   out combine_gates [T,k] fp32: cand_gates of the serving candidate, 0 if
 *       dropped (the weights moe_combine takes).
 *   out x_perm [max_rows,d] (dtype) or NULL: x_perm[r] = x[row_token[r]].
 */
int32_t moe_dispatch_reroute(const moe_config *cfg, const void *x, const int32_t *cand_ids,
                             const float *cand_gates, int32_t *expert_counts,
                             int32_t *expert_offsets, int32_t *slot, int32_t *row_of,
                             int32_t *row_token, int32_t *served_ids, float *combine_gates,
                             void *x_perm, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Expert FFN over the expert-contiguous rows as one grouped GEMM per layer
 * ([MoE Principles] §1 FFN; MiniMax gate/communication page, 60-second answer:
 * batched or grouped GEMM per expert).
 *   in  x_perm [max_rows,d] (dtype), expert_offsets [E+1] int32 (device).
 *   in  W1 [E,d_ff,d], W2 [E,d,d_ff] (dtype); b1 [E,d_ff], b2 [E,d] fp32 or NULL.
 *   out h [max_rows,d_ff] (dtype): sigma(x_perm W1_e^T + b1_e), rounded once.
 *   out y_perm [max_rows,d] (dtype): h W2_e^T + b2_e, rounded once.
 */
int32_t moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *expert_offsets,
                       const void *W1, const float *b1, const void *W2, const float *b2,
                       void *h, void *y_perm, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Combine ([MoE Principles] §2.2 output formula and §5 "send outputs back in
 * token order and weight them"):
 *   y_t = sum_{j<k, row_of[t,j] >= 0} topk_gates[t,j] * y_perm[row_of[t,j]],
 *   summed over j = 0..k-1 in fp32 and rounded once to dtype.
 *   in y_perm [max_rows,d] (dtype), row_of [T,k] int32, topk_gates [T,k]
 *   fp32 (with re-routing: moe_dispatch_reroute's combine_gates);
 *   out y [T,d] (dtype).
 */
int32_t moe_combine(const moe_config *cfg, const void *y_perm, const int32_t *row_of,
                    const float *topk_gates, void *y, hipStream_t stream);

/*
 * The whole layer: route -> dispatch -> grouped FFN -> combine
 * ([MoE Principles] §5 data-flow figure, without the all-to-all steps).
 *   x, W_r, W1, W2 (dtype); b_r, b1, b2 fp32 or NULL; out y [T,d] (dtype).
 *   info: optional routing outputs (NULL: none).
 *   ws/ws_bytes: at least moe_workspace_size bytes, 256-byte aligned.
 *   stage_events: NULL, or MOE_NUM_STAGES+1 caller-created hipEvents that
 *   are recorded on `stream` before the first stage and after each stage.
 *   kernel_events: NULL, or 2*MOE_NUM_STAGES caller-created hipEvents:
 *   [2s] when stage s's first kernel starts and [2s+1] when its last kernel
 *   ends, recorded by the kernel dispatches themselves, so each difference
 *   is the stage's kernel time without the launch gap in front of it (a
 *   stage without rows records both on `stream`).
 * The second expert GEMM keeps y_perm in the workspace; when it splits K
 * (few rows, long K) it keeps two fp32 partial sums there instead, which
 * the combine adds before weighting.
 */
int32_t moe_layer_forward(const moe_config *cfg, const void *x, const void *W_r,
                          const float *b_r, const void *W1, const float *b1, const void *W2,
                          const float *b2, void *y, const moe_route_info *info, void *ws,
                          size_t ws_bytes, hipEvent_t *stage_events, hipEvent_t *kernel_events,
                          hipStream_t stream);

/* Bytes of the fixed device array moe_layer_forward_noalloc works in
 * (one copy per GPU the library runs on, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES 268435456

/*
 * moe_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It runs exactly the kernels of
 * moe_layer_forward, in a fixed array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU, and calls no allocator. Arguments and outputs
 * as moe_layer_forward (no stage or kernel events).
 *   Errors: those of moe_layer_forward; MOE_ERR_WORKSPACE when the layer's
 *   moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES (no device call is
 *   made then); MOE_ERR_HIP when the array's address cannot be found.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams, other host threads) race and must be ordered by the
 *   caller. The array keeps the last call's contents; no call relies on them.
 */
int32_t moe_layer_forward_noalloc(const moe_config *cfg, const void *x, const void *W_r,
                                  const float *b_r, const void *W1, const float *b1,
                                  const void *W2, const float *b2, void *y,
                                  const moe_route_info *info, hipStream_t stream);

/* Figures of moe_load_stats, in this order in its stats array. */
enum {
  MOE_STAT_DROPPED = 0,        /* assignments without a row: T k - rows */
  MOE_STAT_OVERFLOW_RATIO = 1, /* dropped / (T k) */
  MOE_STAT_MAX_OVER_MEAN = 2,  /* max_e count_e / mean_e count_e (routed load) */
  MOE_STAT_PADDING_RATIO = 3,  /* E C / rows: a padded [E, C] layout against the rows kept */
  MOE_STAT_LOAD_ENTROPY = 4,   /* -sum_e f_e ln f_e, f_e = count_e / sum count */
  MOE_STAT_KEPT_VARIANCE = 5,  /* population variance over experts of the rows each holds */
  MOE_STAT_AUX_LOSS = 6,       /* aux_alpha E sum_e (count_e / T)(prob_sum_e / T); NaN without prob_sum */
  MOE_STAT_KEPT_ROWS = 7,      /* rows = expert_offsets[E] */
  MOE_NUM_STATS = 8
};

/*
 * Load statistics of one routing step, computed on the device from the
 * dispatch's outputs ([MoE Principles] §3.3: tokens received and dropped
 * per expert, max/mean load; §13: tokens per expert, overflow ratio,
 * padding ratio; §3.2: L_aux; ai-master.cc EP answer 001, follow-up 2:
 * entropy of the expert activation distribution, variance of the tokens
 * each expert processes). One small kernel on `stream`.
 *   in  expert_counts [E] int32 (routed demand, before capacity),
 *       expert_offsets [E+1] int32 (rows each expert holds), prob_sum [E]
 *       fp32 or NULL (moe_route's sum over tokens of p_{t,e}).
 *   out kept [E] int32 or NULL: offsets[e+1] - offsets[e].
 *   out dropped [E] int32 or NULL: max(count_e - kept_e, 0) (the plain rule:
 *       the tokens expert e turned away).
 *   out stats [MOE_NUM_STATS] fp64 (required): see MOE_STAT_*.
 * Sums run in a fixed order: the results are bit-reproducible.
 */
int32_t moe_load_stats(const moe_config *cfg, const int32_t *expert_counts,
                       const int32_t *expert_offsets, const float *prob_sum, double aux_alpha,
                       int32_t *kept, int32_t *dropped, double *stats, hipStream_t stream);

/* Stage boundaries for moe_layer_backward's optional events. */
enum {
  MOE_BWD_STAGE_RECOMPUTE = 0, /* logits, transposed weights, u = x W1^T + b1, Z = dy W2 */
  MOE_BWD_STAGE_ROWS = 1,      /* per-row h, du, dY and combine-weight gradients */
  MOE_BWD_STAGE_DGRAD = 2,     /* dx_perm = du W1_e, grouped */
  MOE_BWD_STAGE_WGRAD = 3,     /* dW1, dW2, db1, db2 */
  MOE_BWD_STAGE_ROUTER = 4,    /* softmax/L_aux backward, dW_r, db_r, dx */
  MOE_BWD_NUM_STAGES = 5
};

/* Workspace bytes moe_layer_backward needs (host only). */
int32_t moe_backward_workspace_size(const moe_config *cfg, size_t *bytes);

/*
 * Backward pass of the layer: gradients of L = <dy, y> + L_aux, L_aux =
 * aux_alpha E sum_i f_i pbar_i ([MoE Principles] §3.2), with the forward's
 * top-k choices and capacity decisions held fixed (a discrete choice has no
 * gradient; a chosen expert receives its gradient through its combine
 * weight, [MoE Principles] §2.4; §9.1 lists the expert and combine backward
 * among the training steps):
 *   dY_r = g_{t,j} dy_t for kept rows; dg_{t,j} = <dy_t, y_perm_r>;
 *   dh = dY W2_e; du = dh * sigma'(u), u = x W1_e^T + b1_e;
 *   dW2_e = dY^T h, db2_e = sum dY; dW1_e = du^T x, db1_e = sum du;
 *   dx_t = sum_j du_r W1_e + ds_t W_r; the router: dp through the
 *   (renormalised) gates plus aux_alpha E f_i / T, ds = softmax backward,
 *   dW_r = ds^T x, db_r = sum_t ds_t.
 * u, h and y_perm's contribution are recomputed from x (nothing of the
 * forward is stored beyond its routing results). bf16 layers round the
 * GEMM operands dY, du (and h, as the forward does) to bf16; all
 * accumulation is fp32.
 *   in  x, W_r, W1, W2, dy [T,d] (dtype); b_r, b1, b2 fp32 or NULL.
 *   in  fwd: the forward's topk_ids, topk_gates, expert_counts,
 *       expert_offsets, row_of and row_token (all required).
 *   out dx [T,d], dW_r [E,d], dW1 [E,d_ff,d], dW2 [E,d,d_ff] fp32 (required);
 *       db_r [E], db1 [E,d_ff], db2 [E,d] fp32 or NULL (not computed).
 *   ws: at least moe_backward_workspace_size bytes, 256-byte aligned.
 *   stage_events: NULL, or MOE_BWD_NUM_STAGES+1 caller-created hipEvents
 *   recorded on `stream` before the first stage and after each stage.
 * Errors as the forward; cfg->reroute != 0 gives MOE_ERR_UNSUPPORTED.
 */
int32_t moe_layer_backward(const moe_config *cfg, const void *x, const void *W_r, const float *b_r,
                           const void *W1, const float *b1, const void *W2, const float *b2,
                           const moe_route_info *fwd, const void *dy, float aux_alpha, float *dx,
                           float *dW_r, float *db_r, float *dW1, float *db1, float *dW2, float *db2,
                           void *ws, size_t ws_bytes, hipEvent_t *stage_events, hipStream_t stream);

/* A static string naming a status code. */
const char *moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
