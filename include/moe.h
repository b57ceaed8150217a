/*
 * moe.h -- C ABI of libmoe: the forward pass of a token-choice Mixture-of-Experts
 * FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer (sources are web pages, cited by title and section):
 *   [MoE-10]  niuwancheng.cn, "10. 混合专家 MoE：总参数与激活参数"
 *   [Hardest] amazingdata.cn, essay "moe-routing-hardest"
 *   [Arch]    wuaizhan.com, "MoE 混合专家架构原理拆解"
 *   [Lesson]  hi-bin.com, "MoE为什么只激活一部分专家"
 *
 *   router logits  z = x . W_g^T (+ optional per-expert logit bias)
 *   gate           softmax over the E experts, or an independent sigmoid per expert
 *   top-k          the k best experts per token (best first, equal scores -> lower id)
 *   weights        renormalised over the k selected (optional), times routed_scaling_factor
 *   capacity       optional: cap = ceil(capacity_factor * T * k / E) assignments per
 *                  expert; later (token, slot) assignments beyond it are dropped and
 *                  contribute 0 (the token passes through the residual only)
 *   dispatch       kept assignments laid out expert-contiguous, in token order
 *   experts        SwiGLU FFN per expert: down( silu(gate(x)) * up(x) ), grouped GEMM
 *   shared expert  optional, always active, weight 1, added to the routed sum
 *   combine        y[t] = sum_j w[t,j] * expert_{idx[t,j]}(x[t]) (+ shared(x[t]))
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronises on these paths.  Every call is asynchronous
 *     on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *   - Row-major, densely packed.  Storage is cfg->dtype for x, the weights, x_perm,
 *     y_perm, y_shared and y; router_bias and topk_w are float32; every index array
 *     is int32.  Arithmetic accumulates in float32 (bf16 MFMA or fp32 FMA).
 *   - Device pointers must be 16-byte aligned.
 *   - The configuration is checked on the host before anything is enqueued: a
 *     non-zero status means nothing was launched.  A failed launch is reported as
 *     MOE_ERR_HIP.  Nothing aborts, prints or throws across the ABI.
 *   - Calls are stateless; concurrent calls are safe unless they share a
 *     workspace or output buffers.
 *
 * Supported range: T >= 1, 1 <= k <= min(E, 16), E <= 1024, H and I multiples of
 * 64, T*k + T < 2^31, n_shared in {0, 1} with I_shared == I when n_shared == 1.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* sizes outside the supported range */
  MOE_ERR_UNSUPPORTED = 3, /* a valid option the library does not implement */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 5,         /* a HIP launch or runtime call failed */
  MOE_ERR_ALIGN = 6,       /* a device pointer is not 16-byte aligned */
  MOE_ERR_SCRATCH = 7      /* moe_forward_noalloc: the layer's workspace exceeds the static scratch */
} moe_status;

/* Gate of [MoE-10] "路由器怎样选专家：top-k 与两种门控": softmax over all experts
 * (Mixtral, Qwen3) or an independent sigmoid per expert (DeepSeek-V3). */
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gate;

/* Storage type of activations and weights; accumulation is always float32. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* The layer's options, named after the config.json fields of [MoE-10]
 * (num_experts_per_tok, moe_intermediate_size, routed_scaling_factor). */
typedef struct {
  int64_t T;                    /* tokens in the batch */
  int64_t H;                    /* hidden size */
  int64_t I;                    /* moe_intermediate_size of a routed expert */
  int64_t E;                    /* routed experts */
  int64_t k;                    /* num_experts_per_tok */
  int32_t gate;                 /* moe_gate */
  int32_t renormalize;          /* 1: selected weights divided by their sum */
  float routed_scaling_factor;  /* multiplies the routed weights (1.0; 2.5 for DeepSeek-V3) */
  float capacity_factor;        /* <= 0: no limit; else cap = ceil(cf*T*k/E) */
  int64_t n_shared;             /* 0 or 1 always-active shared expert */
  int64_t I_shared;             /* its intermediate size (must equal I) */
  int32_t dtype;                /* moe_dtype */
  /* DeepSeek-V3 group-limited selection ([MoE-10] "DeepSeek-V3 的无辅助损失偏置",
   * config n_group / topk_group): the E experts form n_group equal groups; a
   * group's score is the sum of its two best ranking scores; only the
   * topk_group best groups are eligible.  n_group = 0: no grouping. */
  int32_t n_group;              /* 0, or 1..64 dividing E */
  int32_t topk_group;           /* 1..n_group; k <= topk_group * E / n_group */
} moe_config;

/* Weights of one layer.  Layouts are [out, in], used as x @ W^T like the router
 * of [MoE-10] "把一个大 FFN 换成一组小 FFN". */
typedef struct {
  const void *w_router;     /* [E, H] */
  const float *router_bias; /* [E] float32 logit bias, or NULL */
  const void *w_gate;       /* [E, I, H] */
  const void *w_up;         /* [E, I, H] */
  const void *w_down;       /* [E, H, I] */
  const void *ws_gate;      /* [I_shared, H] shared expert, NULL when n_shared == 0 */
  const void *ws_up;        /* [I_shared, H] */
  const void *ws_down;      /* [H, I_shared] */
  /* Selection-only expert bias ([MoE-10] "DeepSeek-V3 的无辅助损失偏置",
   * e_score_correction_bias): experts are ranked by gate score + score_bias,
   * the combine weights use the unbiased scores.  [E] float32 or NULL. */
  const float *score_bias;
} moe_weights;

/* Optional routing outputs of moe_forward; every field may be NULL (then the
 * workspace holds it). */
typedef struct {
  int32_t *topk_idx;     /* [T, k] selected experts, best first */
  float *topk_w;         /* [T, k] combine weights */
  int32_t *counts;       /* [E] demand per expert (assignments before capacity) */
  int32_t *offsets;      /* [E + 1] exclusive scan of the kept load per expert */
  int32_t *row_of_slot;  /* [T, k] row in expert-contiguous order, -1 if dropped */
  int32_t *token_of_row; /* [T*k] token of each kept row; first offsets[E] valid */
  float *scores;         /* [T, E] gate score of every expert (float32), or NULL: not
                          * written.  The input of moe_balance_stats. */
} moe_route_out;

/* Human-readable name of a status code (static string). */
const char *moe_status_str(moe_status s);

/* Host only, touches no GPU: checks cfg against the supported range. */
moe_status moe_validate(const moe_config *cfg);

/* Host only: bytes of device workspace that moe_forward needs; the same size
 * also serves moe_dispatch and moe_expert_ffn. */
moe_status moe_workspace_size(const moe_config *cfg, size_t *bytes);

/* Host only: per-expert capacity, ceil(capacity_factor*T*k/E) computed in double,
 * or -1 when capacity_factor <= 0 (no limit) or cfg is invalid.
 * [MoE-10] "负载不均：路由坍缩与丢 token": capacity = tokens / experts x factor,
 * rounded up in the page's example; "tokens" is read as the T*k assignments. */
int64_t moe_capacity(const moe_config *cfg);

/* Host only: parameters of one MoE FFN layer from its shape.
 * [MoE-10] "总参数和激活参数怎样算": total = E*3*H*I + E*H (router) + shared;
 * active = k*3*H*I + E*H + shared. */
moe_status moe_layer_params(const moe_config *cfg, int64_t *total, int64_t *active);

/* Router GEMM fused with the gate and top-k ([MoE-10] "路由器怎样选专家",
 * [Hardest] routing steps).  Reads x [T,H], w_router [E,H], router_bias [E]
 * (float32, NULL = none); writes topk_idx [T,k] (best first; equal scores ->
 * lower expert id) and topk_w [T,k] (renormalised if cfg->renormalize, times
 * routed_scaling_factor). */
moe_status moe_route(const moe_config *cfg, const void *x, const void *w_router,
                     const float *router_bias, int32_t *topk_idx, float *topk_w,
                     void *stream);

/* moe_route with a selection-only expert bias (score_bias [E] float32 or NULL;
 * see moe_weights.score_bias) and the group limit of cfg->n_group /
 * cfg->topk_group ([MoE-10] "DeepSeek-V3 的无辅助损失偏置").  Ties of ranking
 * scores go to the lower expert id, of group scores to the lower group id.
 * scores: NULL, or [T, E] float32 that receives every expert's gate score
 * (softmax over E, or sigmoid per expert; the bias is not added). */
moe_status moe_route_sel(const moe_config *cfg, const void *x, const void *w_router,
                         const float *router_bias, const float *score_bias, int32_t *topk_idx,
                         float *topk_w, float *scores, void *stream);

/* Load-balancing statistics of one routed batch ([MoE-10] "辅助损失": f_i is the
 * share of the batch routed to expert i, P_i the mean routing probability of
 * expert i, and the balance term is N * sum_i f_i P_i, 1.0 for a perfectly even
 * router; an auxiliary loss is alpha times it).  Inputs: counts [E] (int32, the
 * demand per expert as moe_dispatch writes it) and scores [T, E] (float32, as
 * moe_route_sel writes it).  Outputs, each optional (NULL = not written):
 * score_mean [E] = P_i = sum_t scores[t,i] / T, load_frac [E] = f_i =
 * counts[i] / (T k), balance [1] = E * sum_i f_i P_i.  All float32, summed in a
 * fixed order (deterministic).  ws: at least ceil(T/256) * E * 4 bytes of device
 * scratch (moe_workspace_size() bytes always suffice). */
moe_status moe_balance_stats(const moe_config *cfg, const int32_t *counts, const float *scores,
                             float *score_mean, float *load_frac, float *balance, void *ws,
                             size_t ws_bytes, void *stream);

/* One step of the auxiliary-loss-free balancing ([MoE-10] "DeepSeek-V3 的无辅助
 * 损失偏置"): score_bias[i] += gamma when counts[i] is below the mean load
 * sum(counts) / E, -= gamma when above, unchanged when equal (compared exactly
 * in integers; the add is float32).  counts [E] int32, score_bias [E] float32,
 * updated in place on the device. */
moe_status moe_bias_update(const moe_config *cfg, const int32_t *counts, float gamma,
                           float *score_bias, void *stream);

/* Histogram, stable scan and capacity, then the gather ([MoE-10] simplified
 * Mixtral block: the rows of each expert are collected; "负载不均": overflow is
 * dropped).  Precondition: topk_idx in [0, E).  Writes counts [E] (demand),
 * offsets [E+1] (kept rows per expert, scanned), row_of_slot [T,k] (-1 =
 * dropped), token_of_row [T*k] (first offsets[E] valid) and, when x_perm is not
 * NULL, x_perm [T*k, H] = x[token_of_row[row]] for the first offsets[E] rows.
 * Ranks within an expert follow (token, slot) order, so every output is
 * deterministic.  ws: workspace of at least moe_workspace_size() bytes. */
moe_status moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, const void *x,
                        int32_t *counts, int32_t *offsets, int32_t *row_of_slot,
                        int32_t *token_of_row, void *x_perm, void *ws, size_t ws_bytes,
                        void *stream);

/* Grouped SwiGLU experts ([MoE-10] "把一个大 FFN 换成一组小 FFN": the tokens of
 * one expert go through one batched GEMM).  Rows offsets[e]..offsets[e+1] of
 * x_perm [*, H] go through expert e: y_perm[row] = W_down[e] . (silu(W_gate[e] .
 * x) * (W_up[e] . x)).  offsets [E+1] is a DEVICE array; offsets[E] <= T*k.
 * The shared expert alone is this call with E = 1, I = I_shared, offsets = {0, T}.
 * ws: workspace of at least moe_workspace_size() bytes. */
moe_status moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *offsets,
                          const void *w_gate, const void *w_up, const void *w_down,
                          void *y_perm, void *ws, size_t ws_bytes, void *stream);

/* Deterministic gate-weighted combine ([Lesson] "Router 怎样给 Token 选专家": y_t
 * is the weighted sum of the selected experts' outputs; [MoE-10]
 * "细粒度专家与共享专家": the shared output is added as is).
 * y[t] = sum_{j=0..k-1, row_of_slot[t,j] >= 0} topk_w[t,j] * y_perm[row_of_slot[t,j]]
 *        (+ y_shared[t] when y_shared is not NULL), accumulated in float32 in
 * that fixed order, no atomics.  Dropped slots contribute exactly 0. */
moe_status moe_combine(const moe_config *cfg, const void *y_perm, const int32_t *row_of_slot,
                       const float *topk_w, const void *y_shared, void *y, void *stream);

/* The whole layer: route, dispatch (gather fused into the expert GEMM's A-tile
 * loader), grouped gate/up + SwiGLU, grouped down, combine; the shared expert
 * runs as one more group over all T tokens.  y [T,H] is the FFN output only
 * (the caller adds the residual).  route_out may be NULL; its NULL members are
 * kept in the workspace instead (scores: not computed). */
moe_status moe_forward(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                       moe_route_out *route_out, void *ws, size_t ws_bytes, void *stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments as moe_forward minus the workspace: the library keeps a static
 * device scratch of MOE_STATIC_SCRATCH_BYTES (64 MiB) on every GPU it runs on,
 * held until the process ends, and this call neither allocates nor frees.
 * Returns MOE_ERR_SCRATCH, with nothing launched, when moe_workspace_size(cfg)
 * exceeds it (e.g. the DeepSeek-V3 decode layer, 16 tokens, needs about 3 MB;
 * prefill batches of a few hundred tokens fit).  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Returns MOE_ERR_HIP if
 * the scratch address cannot be obtained on the current device. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
size_t moe_static_scratch_bytes(void);
moe_status moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                               moe_route_out *route_out, void *stream);

/* moe_forward that also records `events` (an array of MOE_STAGE_EVENTS hipEvent_t
 * created by the caller, or NULL) on `stream` around its stages, for timing:
 * [0] before route, [1] after route, [2] after dispatch, [3] after gate/up,
 * [4] after down, [5] after combine.  A NULL entry is not recorded; each recorded
 * event holds the next launch until the previous one has finished, so a caller
 * timing the whole step records only the boundaries it needs. */
#define MOE_STAGE_EVENTS 6
moe_status moe_forward_timed(const moe_config *cfg, const moe_weights *w, const void *x,
                             void *y, moe_route_out *route_out, void *ws, size_t ws_bytes,
                             void *stream, void *const *events);

/* ---- FP8 expert weights for decode ([MoE-10] "推理时：显存按总参数，计算按激活参数":
 * the released DeepSeek-V3 weights are FP8, about one byte per parameter; a
 * small decode batch streams only the touched experts' weights, so one byte per
 * weight halves the streamed bytes).  The page gives no format; the library
 * uses OCP E4M3 codes (bias 7, subnormals, largest finite 448, 0x7F/0xFF NaN)
 * and one float32 scale per 128 x 128 block of each [out, in] weight matrix,
 * weight = E4M3 value x block scale.  Activations stay bf16; products are
 * accumulated in float32 per block and scaled per block. ---- */

typedef struct {
  const uint8_t *w_gate, *w_up, *w_down;    /* codes [E, I, H], [E, I, H], [E, H, I] */
  const float *s_gate, *s_up, *s_down;      /* scales [E, I/128, H/128], [E, I/128, H/128], [E, H/128, I/128] */
  const uint8_t *ws_gate, *ws_up, *ws_down; /* shared expert codes [I, H], [I, H], [H, I]; NULL if n_shared = 0 */
  const float *ss_gate, *ss_up, *ss_down;   /* its scales [I/128, H/128], [I/128, H/128], [H/128, I/128] */
} moe_fp8_experts;

/* Quantise G matrices w [G, N, K] (dtype MOE_BF16 or MOE_F32, device) to E4M3
 * codes [G, N, K] and scales [G, N/128, K/128]: a block's scale is its largest
 * |w| / 448 in float32 (1.0 for an all-zero block) and each weight becomes the
 * E4M3 code nearest to the float32 quotient w / scale, ties to the even code.
 * N and K multiples of 128, G <= 65535. */
moe_status moe_quantize_fp8(const void *w, int32_t dtype, int64_t G, int64_t N, int64_t K,
                            uint8_t *codes, float *scales, void *stream);

/* moe_forward with FP8 routed and shared experts (q) for decode batches: the
 * router (w->w_router, w->router_bias, w->score_bias) and x / y stay bf16;
 * w's expert pointers are not read.  Requires cfg->dtype == MOE_BF16 and
 * T <= 16 (else MOE_ERR_UNSUPPORTED), H and I multiples of 128.  Same
 * workspace as moe_forward. */
moe_status moe_forward_fp8(const moe_config *cfg, const moe_weights *w, const moe_fp8_experts *q,
                           const void *x, void *y, moe_route_out *route_out, void *ws,
                           size_t ws_bytes, void *stream);

/* ---- expert-choice routing ([Hardest], the two routing schools: each expert
 * takes a fixed number of the tokens it wants most; the load is balanced by
 * construction and a token may get no expert) ---- */

/* Optional outputs of moe_forward_ec (each may be NULL: kept in the workspace). */
typedef struct {
  float *scores;         /* [T, E] gate score of every expert for every token */
  int32_t *token_of_row; /* [E * C] chosen tokens, expert-contiguous, ascending token id */
  int32_t *row_of_pair;  /* [T, E] row e*C + j of the pair (t, e), or -1 when e did not take t */
} moe_ec_out;

/* Host only: tokens per expert C = min(T, ceil(cf * T * k / E)) in double, with
 * cf = capacity_factor, read as 1.0 when <= 0 (the token-choice budget of T*k
 * assignments spread evenly); -1 when cfg is invalid. */
int64_t moe_ec_capacity(const moe_config *cfg);

/* Host only: bytes of device workspace that moe_forward_ec needs. */
moe_status moe_ec_workspace_size(const moe_config *cfg, size_t *bytes);

/* Per-expert top-C selection from scores [T, E] (float32): expert e takes the
 * C = moe_ec_capacity(cfg) tokens with the highest scores[t, e], equal scores
 * going to the lower token id (selection exact on the float32 values).  Writes
 * token_of_row [E*C] (expert e's tokens at e*C.., ascending token id) and
 * row_of_pair [T, E] (the row of each chosen pair, -1 elsewhere). */
moe_status moe_route_ec(const moe_config *cfg, const float *scores, int32_t *token_of_row,
                        int32_t *row_of_pair, void *stream);

/* The layer under expert choice: router and gate (cfg->gate; score_bias and
 * expert groups do not apply), per-expert top-C, grouped SwiGLU experts over
 * the E*C chosen rows (the shared expert as one more group over all T tokens),
 * then y[t] = sum over the experts e that took t, in expert order, of
 * scores[t,e] * routed_scaling_factor * expert_e(x_t), accumulated in float32,
 * plus the shared output.  No renormalisation: a token's weights are its raw
 * scores; a token no expert took gets the shared output only (0 without one).
 * ws: at least moe_ec_workspace_size() bytes; eo may be NULL. */
moe_status moe_forward_ec(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                          moe_ec_out *eo, void *ws, size_t ws_bytes, void *stream);

/* ---- calibration (not part of the layer) ----
 * The bf16 MFMA rate the device sustains with no memory traffic: one launch of
 * 2048 workgroups x 4 waves, each wave issuing 4 * iters
 * v_mfma_f32_32x32x16_bf16 on register operands (four independent accumulator
 * chains) and writing one float of its result into sink (device, float32,
 * 8192 entries).  varied = 0: every MFMA multiplies the same two operands;
 * varied = 1: eight operand pairs of hashed bf16 values (sign, exponent 2^-4,
 * mantissa) in turn, chain c taking pair c on even iterations and pair 4 + c
 * on odd ones, so the matrix units toggle as on real data.  *flops (host)
 * receives the launch's floating-point operation count; the caller times the
 * launch (events on `stream`).  1 <= iters <= 2^24 and varied in {0, 1}, else
 * MOE_ERR_SHAPE; MOE_ERR_NULL for a NULL sink or flops. */
moe_status moe_mfma_peak(int64_t iters, int32_t varied, float *sink, int64_t *flops, void *stream);

/* The rate at which the device reads HBM with no arithmetic to speak of: one
 * launch of 4096 workgroups reads `bytes` of buf (device) once, as 32 KiB
 * blocks, block b by workgroup b mod 4096, each block one contiguous sweep of
 * 16-byte non-temporal loads (the fastest read pattern measured: every wave
 * load whole 128-byte lines, not kept in the caches).  sink (device, uint32, 4096 entries) receives in entry w the
 * XOR of every 32-bit word of the blocks w, w + 4096, w + 8192, ... (0 when
 * there are none), so the loads cannot be dropped and the result can be
 * checked.  The caller times the launch (events on `stream`); the buffer
 * should be far larger than the last-level cache (say >= 4 GiB).  bytes a
 * positive multiple of 32768 and at most 2^40, else MOE_ERR_SHAPE;
 * MOE_ERR_NULL / MOE_ERR_ALIGN for a NULL or not 16-byte aligned buf or sink. */
moe_status moe_hbm_read_peak(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
