/*
 * libmoe — one GPU's share of a mixture-of-experts layer on AMD MI355X
 * (gfx950): routing, dispatch into per-expert / per-EP-rank buffers, grouped
 * expert FFN forward and backward, weighted combine, and the backward duals.
 *
 * The problem statement these calls follow is the tutorial chapter
 * "扩展 MoE 模型——迈向分布式训练" (distributed MoE training):
 *   - section "专家并行：在不同设备上分配专家", part 二: the four EP steps
 *     (replicated local gate, send tokens to the expert's device, local
 *     expert compute, return results in sequence order);
 *   - section "All-to-All 通信模式", part 二: N devices, T/N tokens and E/N
 *     experts each, gate g(x), device i sends to device k the set S_ik of its
 *     tokens whose expert lives on k; part 六: variable-size exchanges;
 *   - section "专家并行与数据并行的结合", part 三: backward routes gradients
 *     back to the experts, expert parameter gradients are computed locally;
 *   - section "用于分布式 MoE 的主流框架与库": the knobs a layer takes (top-k
 *     gate with k, ffn experts, model width, number of experts, EP size);
 *   - section "通信优化方法", part 四: pre-allocated, reused buffers.
 * The Piper summary (方法论 1) names expert capacity and the routing table
 * as per-GPU quantities.
 *
 * Conventions for every call below:
 *   - Every tensor argument is a DEVICE pointer owned by the caller,
 *     contiguous and row-major, 16-byte aligned.  The library never
 *     allocates, frees or synchronises; scratch memory is the caller's
 *     `ws` buffer of moe_plan()'s workspace_bytes.
 *   - `stream` is a hipStream_t passed as a plain pointer (NULL = the null
 *     stream).  Each call validates on the host, enqueues its kernels on
 *     that stream and returns; results are valid for later work on it.
 *   - Element type `dtype` (MOE_F32 / MOE_BF16) applies to x, y, weights,
 *     activations and their gradients ("void*" arguments).  Logits, gate
 *     weights and their gradients are always fp32; indices and counts int32;
 *     offsets int64.
 *   - Return value: MOE_OK, or a negative moe_status.  On MOE_ERR_INVALID /
 *     MOE_ERR_UNSUPPORTED nothing was enqueued.  On MOE_ERR_HIP a launch
 *     failed (see moe_last_hip_error()); outputs are then undefined.
 *   - Results are deterministic: no floating-point atomics are used, so two
 *     identical calls give bit-identical outputs.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* bad argument: nothing enqueued          */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside what is implemented   */
  MOE_ERR_HIP = -3           /* a HIP launch failed                     */
} moe_status;

enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Gate weight of the j-th chosen expert e_j of a token with logits l. */
enum {
  MOE_GATE_SOFTMAX_TOPK = 0,        /* g_j = softmax(l)[e_j]                    */
  MOE_GATE_SOFTMAX_TOPK_RENORM = 1, /* g_j = softmax(l)[e_j] / sum_m softmax(l)[e_m] */
  MOE_GATE_TOPK_SOFTMAX = 2         /* g_j = softmax over the k chosen logits   */
};

enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 };

/* Expert e's EP rank: contiguous e / (E/R) (the tutorial's 4-device
 * picture: Dev0 holds E0, E1; Dev1 holds E2, E3); round-robin e % R. */
enum { MOE_PLACE_CONTIGUOUS = 0, MOE_PLACE_ROUND_ROBIN = 1 };

typedef struct {
  int64_t T;                /* tokens, >= 1                                    */
  int64_t d;                /* model width, multiple of 8                      */
  int64_t ffn;              /* routed expert hidden width, multiple of 8       */
  int64_t E;                /* routed experts, 1..64                           */
  int64_t k;                /* experts per token, 1..min(E, 8)                 */
  float capacity_factor;    /* > 0: C = ceil(cf*k*T/E) (double, left to right,
                               capped at T); <= 0: dropless, C = T             */
  int32_t gating;           /* MOE_GATE_*                                      */
  int32_t act;              /* MOE_ACT_*                                       */
  int32_t dtype;            /* MOE_F32 | MOE_BF16                              */
  int32_t ep_ranks;         /* R >= 1, E % R == 0                              */
  int32_t placement;        /* MOE_PLACE_*                                     */
  int64_t n_shared;         /* always-on shared experts (0 if none)            */
  int64_t ffn_shared;       /* hidden width of each shared expert              */
} moe_config;

typedef struct {
  int64_t C;                /* expert capacity                                 */
  int64_t n_max;            /* rows of the permuted buffers: min(T*k, E*C)     */
  size_t workspace_bytes;   /* `ws` size for every call below that takes one   */
} moe_sizes;

/* Row segments of a grouped expert FFN call.  Routed experts: groups = E,
 * offsets = moe_dispatch's expert_offsets, rows_max = n_max, ffn = cfg.ffn,
 * use_placement = 1.  Shared experts: groups = 1, offsets = {0, T},
 * rows_max = T, ffn = n_shared*ffn_shared, use_placement = 0. */
typedef struct {
  int64_t groups;           /* number of row segments, 1..65                    */
  int64_t ffn;              /* hidden width of every group, multiple of 8       */
  int64_t rows_max;         /* rows allocated in the row buffers                */
  const int64_t* offsets;   /* DEVICE [groups+1], ascending, offsets[0] = 0,
                               offsets[groups] <= rows_max: group g owns rows
                               [offsets[g], offsets[g+1])                        */
  int32_t use_placement;    /* 1: group g is send slot g, whose expert (and
                               weight set) follows cfg's placement; 0: group g
                               uses weight set g                                */
  const int64_t* ends;      /* DEVICE [groups] or NULL.  Not NULL: group g owns
                               rows [offsets[g], ends[g]) instead (disjoint
                               sub-ranges, ascending by group, e.g. one token
                               chunk of every expert's segment, from
                               moe_chunk_rows).  Forward and the backward's
                               data gradients only; weight gradients need
                               whole groups (ends = NULL).                     */
} moe_groups;

/* Host only; no GPU is touched.  Sizes every caller-owned buffer up front,
 * following the tutorial's 通信优化方法 四 (pre-allocate and reuse buffers
 * rather than allocating per step): the expert capacity C (Piper 方法论 1
 * names it a per-GPU model input; C = ceil(cf*k*T/E), dropless C = T), the
 * rows n_max = min(T*k, E*C) of the permuted buffers (the all-to-all send
 * buffer of All-to-All 二, which holds at most every kept (token, expert)
 * pair), and the workspace every call below may use.
 * Errors: MOE_ERR_INVALID (null pointer, non-positive sizes, k > E,
 * E % R != 0, unknown enum), MOE_ERR_UNSUPPORTED (E > 64, k > 8, d or ffn
 * not a multiple of 8, T*k >= 2^31, or a row of an expert GEMM operand --
 * d, or the m*ffn columns of [A | B] (m = 2 for SwiGLU, 1 for GELU), or
 * m*n_shared*ffn_shared -- wider than 8388352 bytes, the most a 256-row tile
 * of one GEMM buffer resource may span). */
int moe_plan(const moe_config* cfg, moe_sizes* out);

/* Gate GEMM, softmax and top-k routing (tutorial: 专家并行 二 step 1, the
 * replicated router; 框架: top-k gate).
 *   x [T, d] dtype; w_router [d, E] dtype; bias [E] fp32 or NULL (added to
 *   the logits before softmax and selection).
 *   logits [T, E] fp32: l = x W_r + b, fp32 accumulation.
 *   topk_idx [T, k] int32: per token, experts ordered by (logit descending,
 *   index ascending), first k — equal logits go to the lower index.
 *   topk_w [T, k] fp32: gate weights per cfg->gating.
 *   ws: caller workspace of moe_plan's workspace_bytes, 16-byte aligned;
 *   required for bf16 (the call may write a re-packed copy of w_router
 *   there: more than 16 experts or d above 4096), may be NULL for fp32.
 * Errors: MOE_ERR_INVALID for a null required pointer or a misaligned x / ws. */
int moe_route(const moe_config* cfg, const void* x, const void* w_router,
              const float* bias, float* logits, int32_t* topk_idx,
              float* topk_w, void* ws, void* stream);

/* Capacity, counts, offsets, EP send layout and permutation (tutorial:
 * All-to-All 二/六, send sets S_ik of variable size; Piper 方法论 1:
 * capacity).  pos(t, j) = number of tokens t' < t that chose expert
 * e = topk_idx[t, j]; the assignment is kept iff pos < C (overflow dropped in
 * token order).  Send slots list the experts by (EP rank, local index); an
 * expert's segment lists its kept tokens in ascending order.
 *   raw_counts [E] int32: tokens that chose e;  expert_counts [E] int32:
 *     kept, min(raw, C);
 *   expert_offsets [E+1] int64: segment start of send slot s (slot order);
 *   send_counts [R] int32 / send_offsets [R+1] int64: rows per EP rank;
 *   row_of [T*k] int32: row of assignment (t, j), -1 if dropped;
 *   assign_of_row [n_max] int32: t*k + j of each row (rows >= n untouched);
 *   x_perm [n_max, d] dtype: x_perm[row_of[t*k+j]] = x[t] (exact copy) —
 *     the all-to-all send buffer, segment q = rows of EP rank q.  NULL (with
 *     x NULL too) computes the layout only; moe_permute copies later.
 *   ws: moe_plan's workspace. */
int moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                 void* x_perm, int32_t* row_of, int32_t* assign_of_row,
                 int32_t* raw_counts, int32_t* expert_counts,
                 int64_t* expert_offsets, int32_t* send_counts,
                 int64_t* send_offsets, void* ws, void* stream);

/* The row copy of moe_dispatch alone: x_perm[row_of[t*k+j]] = x[t] for every
 * kept (t, j) of cfg->T tokens.  row_of holds rows of the whole x_perm, so a
 * caller can copy one token chunk [t0, t1) by passing x + t0*d,
 * row_of + t0*k and a config with T = t1 - t0 (moe_dispatch with x_perm NULL
 * having laid out the whole batch): the tutorial's 通信优化方法 三 overlap of
 * communication with computation, here a bandwidth kernel beside the expert
 * GEMMs of another chunk (FlowMoE notes, 关键设计: pipelining over token
 * chunks).  Errors: MOE_ERR_INVALID for a null or misaligned pointer. */
int moe_permute(const moe_config* cfg, const void* x, const int32_t* row_of,
                void* x_perm, void* stream);

/* Rows of token chunks in the dispatch layout.  The kept rows of each expert
 * are its first C choosers in token order, so the tokens of chunk r,
 * [token_bounds[r], token_bounds[r+1]), hold a contiguous sub-range of every
 * expert's segment.  Writes chunk_rows [chunks+1, E] int64 (DEVICE): row r,
 * slot s = the first row of chunk r in send slot s (row 0 = the segments'
 * starts, row `chunks` = their ends), so chunk r's moe_groups table is
 * offsets = chunk_rows + r*E, ends = chunk_rows + (r+1)*E.
 *   topk_idx, row_of, expert_offsets: moe_route's and moe_dispatch's;
 *   token_bounds: HOST [chunks+1], ascending, 0 first and cfg->T last.
 * Deterministic (integer atomic minimums).  Errors: MOE_ERR_INVALID for a
 * null pointer or bad bounds, MOE_ERR_UNSUPPORTED for more than 16 chunks. */
int moe_chunk_rows(const moe_config* cfg, const int32_t* topk_idx,
                   const int32_t* row_of, const int64_t* expert_offsets,
                   int64_t chunks, const int64_t* token_bounds,
                   int64_t* chunk_rows, void* stream);

/* moe_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * moe_dispatch minus `ws`.  Its scratch (per-block expert counts and bases,
 * the experts' first rows) is a static device array of 2 MiB + 512 bytes
 * inside the library, one per GPU, held until the process ends; the call
 * allocates nothing.  Limits: cfg->T <= 2^20 tokens (MOE_ERR_UNSUPPORTED
 * beyond).  `stream` must belong to the calling thread's current device.
 * Calls that overlap in time on one GPU (on different streams) share that
 * scratch and race: order them on one stream. */
int moe_dispatch_noalloc(const moe_config* cfg, const void* x,
                         const int32_t* topk_idx, void* x_perm,
                         int32_t* row_of, int32_t* assign_of_row,
                         int32_t* raw_counts, int32_t* expert_counts,
                         int64_t* expert_offsets, int32_t* send_counts,
                         int64_t* send_offsets, void* stream);

/* Grouped expert FFN forward (tutorial: 专家并行 二 step 3, local experts;
 * 框架: ffn experts), MFMA with fp32 accumulation.
 *   x_rows [rows_max, d]; weights per expert:
 *     GELU:   w_in = W1 [E', d, ffn], w_out = W2 [E', ffn, d], w_up NULL;
 *     SwiGLU: w_in = W_gate, w_up = W_up [E', d, ffn], w_out = W_down.
 *   act_saved: what the backward multiplies dL/dh by (the derivatives of
 *     the activation at this forward's pre-activations, so that
 *     moe_expert_ffn_bwd does not evaluate the activation again):
 *     GELU [rows_max, ffn]: GELU'(Z) = Phi(Z) + Z phi(Z) with Z = x W1;
 *     SwiGLU [rows_max, 2*ffn]: dh/dA = B s (1 + A (1 - s)) in columns
 *     [0, ffn) and dh/dB = silu(A) in [ffn, 2*ffn), with A = x W_gate,
 *     B = x W_up, s = sigmoid(A).  Rounded to dtype like the other outputs.
 *   h [rows_max, ffn]: GELU(Z) (exact erf form) or silu(A) * B.
 *   y_rows [rows_max, d]: h W_out.  Rows outside the segments are untouched. */
int moe_expert_ffn_fwd(const moe_config* cfg, const moe_groups* grp,
                       const void* x_rows, const void* w_in, const void* w_up,
                       const void* w_out, void* act_saved, void* h,
                       void* y_rows, void* stream);

/* Fused forward of the routed experts (tutorial: 用于分布式 MoE 的主流框架与库
 * 二, Tutel's fused kernels: gate, routing, expert compute and combine
 * merged to cut launches and traffic).  For a forward-only pass:
 *   - GEMM-1 reads each row's activation straight from the token rows,
 *     x[assign_of_row[r] / k], so the dispatch copy (moe_dispatch with x_perm
 *     NULL) is not needed, and writes only h (no saved A | B or Z);
 *   - GEMM-2 writes row r's output, scaled by its gate weight
 *     topk_w[assign_of_row[r]], to row assign_of_row[r] = t*k + j of y_tok
 *     [T*k, d]: the un-permuted, weighted rows that moe_combine_fused sums.
 * The backward needs the unweighted y_perm (for d_topk_w) and x_perm (for
 * the weight gradients), so training uses moe_expert_ffn_fwd.
 *   grp: the routed table (groups = E, use_placement, no ends);
 *   x [T, d], assign_of_row [n_max], topk_w [T, k] (moe_route's,
 *   moe_dispatch's); h [rows_max, ffn]; y_tok [T*k, d] (rows of dropped
 *   assignments untouched).
 * Errors: MOE_ERR_INVALID for a null or misaligned pointer or another group
 * table, MOE_ERR_UNSUPPORTED for fp32 or T*d*2 > 0x7FFF0000 bytes. */
int moe_expert_ffn_fwd_fused(const moe_config* cfg, const moe_groups* grp,
                             const void* x, const int32_t* assign_of_row,
                             const float* topk_w, const void* w_in,
                             const void* w_up, const void* w_out, void* h,
                             void* y_tok, void* stream);

/* Combine of moe_expert_ffn_fwd_fused's weighted token-major rows:
 *   y[t] = sum over kept j (row_of[t*k+j] >= 0) of y_tok[t*k+j]
 *          (+ y_shared[t] if not NULL), fp32 accumulation in j order.
 * Errors: MOE_ERR_INVALID for a null or misaligned pointer. */
int moe_combine_fused(const moe_config* cfg, const void* y_tok,
                      const int32_t* row_of, const void* y_shared, void* y,
                      void* stream);

/* The two halves of moe_expert_ffn_bwd, for callers that pipeline token
 * chunks: moe_expert_ffn_bwd_data computes dL/d act (into ws) and dx_rows for
 * the group table's rows (sub-ranges allowed: grp->ends), and
 * moe_expert_ffn_bwd_weights the weight gradients over whole groups (ends
 * NULL) from the dL/d act that data calls covering every row left in ws.
 * Nothing else may use ws in between.  These two read the weights as given
 * (no transposed copy in ws), whatever the rows per weight set.  Arguments,
 * results and errors as in moe_expert_ffn_bwd. */
int moe_expert_ffn_bwd_data(const moe_config* cfg, const moe_groups* grp,
                            const void* w_in, const void* w_up,
                            const void* w_out, const void* act_saved,
                            const void* dy_rows, void* dx_rows, void* ws,
                            void* stream);
int moe_expert_ffn_bwd_weights(const moe_config* cfg, const moe_groups* grp,
                               const void* x_rows, const void* h,
                               const void* dy_rows, void* dw_in, void* dw_up,
                               void* dw_out, void* ws, void* stream);

/* Grouped expert FFN backward (tutorial: 专家并行与数据并行的结合 三.3:
 * gradients routed back to the experts, parameter gradients computed
 * locally).  dy_rows [rows_max, d] is dL/d y_rows.
 *   dx_rows [rows_max, d] = dL/d x_rows;
 *   dw_in, dw_up, dw_out: same shapes and dtype as w_in, w_up, w_out;
 *   weight sets with no rows get exact zeros.
 *   ws: moe_plan's workspace (holds dL/dZ or dL/d[A|B] in dtype, then the
 *       fp32 partials of weight gradients split over their rows; in bf16
 *       with at least 2000 (1 + m) / m rows per weight set on average, m = 2
 *       for SwiGLU else 1, then also a transposed copy of the three weight
 *       tensors, made in this call, that both dgrads read; moe_plan sizes
 *       the workspace for it and the call does without it when a table's
 *       copy would not fit).
 * Errors: MOE_ERR_INVALID also when the group table would need more
 *   workspace than moe_plan's workspace_bytes for cfg (a table with more
 *   groups, rows or hidden width than the routed or shared tables above), or
 *   has sub-range ends (the weight gradients need whole groups). */
int moe_expert_ffn_bwd(const moe_config* cfg, const moe_groups* grp,
                       const void* x_rows, const void* w_in, const void* w_up,
                       const void* w_out, const void* act_saved, const void* h,
                       const void* dy_rows, void* dx_rows, void* dw_in,
                       void* dw_up, void* dw_out, void* ws, void* stream);

/* Weighted combine (tutorial: 专家并行 二 step 4, results returned in
 * sequence order; 流水线并行 三: outputs merged).
 *   y[t] = sum over kept j of topk_w[t, j] * y_perm[row_of[t*k+j]]
 *          (+ y_shared[t] if y_shared != NULL), fp32 accumulation.
 *   A token with every choice dropped gets y = 0 (+ shared). */
int moe_combine(const moe_config* cfg, const void* y_perm,
                const int32_t* row_of, const float* topk_w,
                const void* y_shared, void* y, void* stream);

/* Combine backward (tutorial: 专家并行与数据并行的结合 三.3: in the
 * backward pass the output gradient is sent back to the device of each
 * chosen expert; 专家并行 二 step 4 is the forward merge this reverses).
 * The chain rule of the weighted sum in moe_combine gives:
 *   dy_perm[row_of[t*k+j]] = topk_w[t, j] * dy[t]   (the expert's upstream
 *     gradient, written in the send-buffer layout);
 *   d_topk_w[t, j] = <dy[t], y_perm[row_of[t*k+j]]> (0 if dropped), the
 *     gate weight's gradient, fp32 accumulation.
 * Rows of dy_perm outside the kept rows are untouched.
 * Errors: MOE_ERR_INVALID for a null pointer or a misaligned dy / y_perm /
 * dy_perm. */
int moe_combine_bwd(const moe_config* cfg, const void* dy, const void* y_perm,
                    const int32_t* row_of, const float* topk_w, void* dy_perm,
                    float* d_topk_w, void* stream);

/* Router backward (tutorial: 专家并行与数据并行的结合 三.4, router
 * gradients).  dlogits [T, E] fp32 through the gate-weight Jacobian:
 *   SOFTMAX_TOPK: dl = p (dp - <p, dp>), dp[e_j] = d_topk_w[t, j], else 0;
 *   RENORM / TOPK_SOFTMAX: dl[e_j] = g_j (dg_j - sum_m g_m dg_m), 0 elsewhere;
 *   plus dlogits_add [T, E] fp32 when not NULL: another gradient of the
 *   logits, such as moe_aux_loss_bwd's, so that dlogits, dw_router and the
 *   router term of moe_dispatch_bwd carry it too.
 * dw_router [d, E] dtype = x^T dlogits (deterministic two-stage reduction).
 * The bias gets no gradient.  ws: moe_plan's workspace. */
int moe_route_bwd(const moe_config* cfg, const void* x, const float* logits,
                  const int32_t* topk_idx, const float* d_topk_w,
                  const float* dlogits_add, float* dlogits, void* dw_router,
                  void* ws, void* stream);

/* Auxiliary load-balancing loss (tutorial: 用于分布式 MoE 的主流框架与库 一,
 * DeepSpeed's moe block and its loss_coef, the load-balancing loss
 * coefficient; 实践 七.3: the logged auxiliary loss should be near 0 with
 * experts chosen about equally often).  The pages give no formula; the one
 * computed is
 *   loss = coef * E * sum_e f_e P_e,
 * f_e = raw_counts[e] / (T k), the share of the routing choices on expert e
 * (moe_dispatch's raw counts, before capacity), P_e = the mean over tokens
 * of softmax(logits[t])[e].  Equal choice counts give loss = coef.
 *   logits [T, E] fp32 (moe_route's), raw_counts [E] int32;
 *   loss: DEVICE pointer to one fp32, written;
 *   ws: moe_plan's workspace (the per-workgroup partial sums, fixed order,
 *   so the loss is deterministic).
 * Errors: MOE_ERR_INVALID for a null pointer, a NaN coef or a misaligned ws. */
int moe_aux_loss(const moe_config* cfg, const float* logits,
                 const int32_t* raw_counts, float coef, float* loss, void* ws,
                 void* stream);

/* Gradient of moe_aux_loss's loss (upstream gradient 1) with respect to the
 * logits, f held constant (it changes only where the top-k does):
 *   dlogits_aux[t, e] = coef * E / T * p[t, e] * (f_e - sum_m f_m p[t, m]),
 * p = softmax(logits[t]); [T, E] fp32, written.  Pass it to moe_route_bwd as
 * dlogits_add.  Errors: MOE_ERR_INVALID for a null pointer or a NaN coef. */
int moe_aux_loss_bwd(const moe_config* cfg, const float* logits,
                     const int32_t* raw_counts, float coef, float* dlogits_aux,
                     void* stream);

/* Dispatch backward (tutorial: 专家并行与数据并行的结合 三.3: the input
 * gradients computed on the experts' devices return to each token's device
 * and sequence order, reversing 专家并行 二 step 2; 三.4: the router's own
 * gradient path).  Un-permute and sum, with the router's dx fused:
 *   dx[t] = sum over kept j of dx_perm[row_of[t*k+j]]
 *           + sum_e dlogits[t, e] * w_router[:, e]
 *           (+ dx_add[t] if dx_add != NULL, e.g. the shared experts' dx),
 *   fp32 accumulation, stored in dtype.  A token with every choice dropped
 *   gets only the router (and dx_add) terms.
 * Errors: MOE_ERR_INVALID for a null required pointer or a misaligned
 * dx_perm / dx / dx_add. */
int moe_dispatch_bwd(const moe_config* cfg, const void* dx_perm,
                     const int32_t* row_of, const float* dlogits,
                     const void* w_router, const void* dx_add, void* dx,
                     void* stream);

const char* moe_status_string(int status);
/* hipError_t of the last MOE_ERR_HIP on the calling thread (0 if none). */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_MOE_H */
