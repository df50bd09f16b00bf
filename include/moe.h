/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer-forward library
 * (libmoe.so).
 *
 * The forward pass of one DeepSeekMoE layer, in the order the calls below
 * run it:
 *   router GEMM and scores  -> moe_route
 *   group-limited top-k     -> moe_route
 *   dispatch                -> moe_permute
 *   SwiGLU experts          -> moe_grouped_ffn (routed experts, shared expert)
 *   combine                 -> moe_combine
 *   load statistics         -> moe_load_stats (batch), moe_seq_load_stats
 *                              (per sequence), moe_group_load_stats (per
 *                              expert group / device)
 *   all of the above        -> moe_layer_forward
 *
 * Sources (web pages, cited by title and section):
 *   [EVO]   "DeepSeek MoE：从v1到v3的演进" (wln20.github.io)
 *   [GLR]   "DeepSeek-V3的Group-Limited Expert Routing与负载均衡优化实践" (mhpn.cn)
 *   [BUILD] "从零构建DeepSeekMoE：揭秘混合专家模型中的负载均衡与专家协同机制"
 *   [TECH]  "DeepSeek-V3技术解密：DeepSeekMoE架构如何重塑AI模型效能边界"
 *
 * Conventions shared by every call:
 *   - Every array pointer is a DEVICE pointer, allocated and owned by the
 *     caller; the library allocates no device memory and keeps no pointer
 *     after a call returns.  Only `cfg`, `weights` (the struct itself),
 *     `aux` (the struct itself), `bytes` and `stage_events` are host memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the host.  Results are ready when the
 *     stream's work up to that point has completed.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-MOE_OK return nothing was enqueued (MOE_ERR_HIP excepted: a launch
 *     failed part-way, and output contents are unspecified).
 *   - Row-major layouts, element strides as stated; weights are stored
 *     "out x in" (the reduction dimension contiguous).
 *   - Calls that share a workspace must not overlap in time; independent
 *     calls on different streams need their own workspaces.
 *   - Outputs are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics on any output path).
 *   - A call enqueues only kernel launches (and the requested event records)
 *     on `stream`; buffers are cleared by kernels, not memset.  Calls can
 *     therefore be captured into a HIP graph and replayed; each replay
 *     reproduces the eager call bit for bit.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size or inconsistent cfg */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
  MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required */
  MOE_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
  MOE_ERR_TOO_LARGE = 5    /* moe_layer_forward_noalloc: needs more than the
                              fixed scratch (MOE_NOALLOC_SCRATCH_BYTES) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layout of the expert weight matrices (w13, w2, ws13, ws2).  Each matrix
 * is R rows (output features) by K columns (input features).
 *   MOE_LAYOUT_ROWS:  row-major, element (r, c) at r*K + c.  fp32 weights.
 *   MOE_LAYOUT_TILED: blocks of 16 rows x 32 columns (1 KiB in bf16); the
 *     block of rows [16i, 16i+16) and columns [32j, 32j+32) starts at element
 *     (i*(K/32) + j)*512, and inside it the 16-byte chunk number l (0..63)
 *     holds row 16i + l%16, columns 32j + 8*(l/16) .. +7.  bf16 weights; R a
 *     multiple of 16, K of 32.  Same size as row-major; moe_pack_weights
 *     converts.  (Each chunk is one lane's MFMA fragment, so the kernels load
 *     weights as contiguous KiBs.) */
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILED = 1 } moe_layout;

/* Score function.  SIGMOID: s = 1/(1+e^-l), each expert independent
 * ([EVO] §DeepSeek-v3).  SOFTMAX: s = softmax over the N logits ([EVO]
 * §ST-MoE p_i(x); §DeepSeek-v1/v2 gate).  Both are computed in fp32 with
 * every rounding step fixed, so a score is reproducible bit for bit: the
 * exponential is Cody-Waite reduction plus a degree-7 Taylor series; the
 * softmax takes E_e = e^(l_e - m) with m the largest logit (E_e = 0 when
 * l_e - m < -64), S = the pairwise sum of E over 256 slots (slot e >= N
 * holds 0; each node adds its lower half's sum to its upper half's), and
 * s_e = E_e / S correctly rounded. */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

typedef struct {
  int32_t T;           /* tokens in the batch (>= 0)                            */
  int32_t H;           /* hidden size; multiple of 64                           */
  int32_t N;           /* routed experts; 1..256, multiple of 4                 */
  int32_t k;           /* experts chosen per token; 0..min(64, candidates)      */
  int32_t n_groups;    /* expert groups ([GLR] §1); 1 = no group limit          */
  int32_t topk_groups; /* groups kept per token ([GLR] §1, §3)                  */
  int32_t group_topn;  /* keys summed into a group's score: 1 or 2              */
  int32_t score_fn;    /* moe_score_fn                                          */
  int32_t norm_topk;   /* 1: gates divided by the sum of the k chosen scores    */
  float route_scale;   /* gate multiplier (1.0, or 2.5 for V3-shaped layers)    */
  int32_t capacity;    /* per-expert capacity C; 0 = unlimited ([EVO] §GShard)  */
  int32_t I;           /* routed expert intermediate size; multiple of 64       */
  int32_t n_shared;    /* always-on shared experts ([EVO] §DeepSeek-v1)         */
  int32_t I_shared;    /* intermediate size of one shared expert                */
  int32_t act_dtype;   /* moe_dtype of x, expert activations and out            */
  int32_t w_dtype;     /* moe_dtype of expert weights (must equal act_dtype)    */
  int32_t router_dtype;/* moe_dtype of the router weight W_g                    */
  int32_t group_capacity; /* device-level token dropping ([EVO] §DeepSeek-v2):
                           * each of the n_groups expert groups (devices) keeps
                           * at most this many assignments, dropping its
                           * lowest-scored ones; 0 = off, -1 = the average
                           * group load ceil(T*k / n_groups).  Exclusive with
                           * `capacity`.                                        */
  int32_t w_layout;    /* moe_layout of the expert weights: MOE_LAYOUT_TILED for
                        * bf16, MOE_LAYOUT_ROWS for fp32 (else UNSUPPORTED)  */
} moe_cfg;

/* Layer weights (device pointers); the expert matrices in cfg->w_layout:
 *   w_router [N, H]              router_dtype, row-major
 *   w13      [N, 2*I, H]         per expert: rows [0,I) gate, rows [I,2I) up
 *   w2       [N, H, I]           per expert: down projection
 *   ws13     [2*n_shared*I_shared, H]  the shared experts packed as one of
 *            width n_shared*I_shared: gate rows of every shared expert, then
 *            their up rows, in the same expert order
 *   ws2      [H, n_shared*I_shared]    their down columns, same order
 * Packing the shared experts side by side is exactly their sum, since each
 * intermediate unit of a SwiGLU expert contributes independently. */
typedef struct {
  const void* w_router;
  const void* w13;
  const void* w2;
  const void* ws13; /* NULL iff n_shared == 0 */
  const void* ws2;  /* NULL iff n_shared == 0 */
} moe_weights;

/* Stages of moe_layer_forward, for optional per-stage events. */
enum {
  MOE_STAGE_ROUTER_GEMM = 0, /* logits                                        */
  MOE_STAGE_ROUTE = 1,       /* scores, group limit, top-k, gates, lse        */
  MOE_STAGE_DISPATCH = 2,    /* histogram, scan, capacity, permutation        */
  MOE_STAGE_FFN_GATE_UP = 3, /* SwiGLU first half (routed + shared)           */
  MOE_STAGE_FFN_DOWN = 4,    /* down projection (routed + shared)             */
  MOE_STAGE_COMBINE = 5,     /* gate-weighted combine                         */
  MOE_STAGE_STATS = 6,       /* f, P, L_B, z                                  */
  MOE_N_STAGES = 7
};

/* Optional outputs of moe_layer_forward; any member may be NULL (the value
 * then lives in the workspace only).  Sizes:
 *   logits [T,N] f32, topk_idx/topk_gate/topk_score [T,k], token_lse [T] f32,
 *   counts [N] i32 (before capacity), offsets [N+1] i32 (after capacity),
 *   row_token [T*k] i32 (first offsets[N] valid), inv_row [T,k] i32
 *   (-1 = dropped), n_dropped [2] i32 = {dropped assignments, tokens with
 *   every assignment dropped}, f [N], P [N], scalars [3] f32 = {L_B, z, z_sq}.
 * stage_events: host array of MOE_N_STAGES+1 hipEvent_t created by the
 * caller; event i is recorded on the stream before stage i and event
 * MOE_N_STAGES after the last stage.  NULL = no events.  A failed event
 * record returns MOE_ERR_HIP like a failed launch. */
typedef struct {
  float* logits;
  int32_t* topk_idx;
  float* topk_gate;
  float* topk_score;
  float* token_lse;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* inv_row;
  int32_t* n_dropped;
  float* f;
  float* P;
  float* scalars;
  void** stage_events;
} moe_aux;

/* Convert n_mat row-major matrices of rows x cols (consecutive in src) to
 * MOE_LAYOUT_TILED in dst: a one-time step when weights are loaded.
 * dtype must be MOE_BF16 (else MOE_ERR_UNSUPPORTED), rows a multiple of 16
 * and cols of 32 (else MOE_ERR_UNSUPPORTED); src and dst are device buffers
 * of n_mat*rows*cols elements that must not overlap (MOE_ERR_INVALID_ARG).
 * Example: w13 of a layer is n_mat = N, rows = 2*I, cols = H; w2 is N, H, I;
 * ws13 is 1, 2*n_shared*I_shared, H; ws2 is 1, H, n_shared*I_shared. */
moe_status moe_pack_weights(int64_t n_mat, int32_t rows, int32_t cols, int32_t dtype,
                            const void* src, void* dst, void* stream);

/* Bytes of workspace moe_layer_forward needs for cfg; also enough for any
 * single granular call below with the same cfg.  Returns MOE_ERR_INVALID_ARG
 * or MOE_ERR_UNSUPPORTED for a cfg the library rejects. */
moe_status moe_workspace_size(const moe_cfg* cfg, size_t* bytes);

/* Router GEMM, scores, group-limited top-k and gates ([EVO] §DeepSeek-v3:
 * sigmoid score, selection on s + b, gate from the unbiased s; [GLR] §1, §3:
 * score groups, keep the best topk_groups, choose top-k among their experts).
 *   x        [T,H] act_dtype, or NULL: then `logits` is an INPUT [T,N] f32
 *            and the router GEMM is skipped
 *   w_router [N,H] router_dtype (ignored when x == NULL)
 *   logits   [T,N] f32: written when x != NULL (fp32-accumulated x.W_g^T,
 *            [TECH] §四.2 keeps the router in fp32).  With bf16 x the
 *            weight is first written to the workspace as bf16 pieces that
 *            sum to it exactly (three for an fp32 weight); each bf16 x bf16
 *            product is exact in fp32, so only the order of the fp32
 *            additions differs from an fp32 GEMM.
 *   bias     [N] f32 or NULL: added to the score for selection only
 *   topk_idx [T,k] i32: chosen experts, slot j = j-th largest key; ties go
 *            to the lower expert (and group) index
 *   topk_gate [T,k] f32: s (divided by the sum of the k chosen s when
 *            norm_topk) times route_scale
 *   topk_score [T,k] f32: unbiased s of the chosen expert
 *   token_lse [T] f32: log sum_e exp(l_e), or NULL
 * Selection keys: sigmoid -> fl32(s + b) with s from the library's fp32
 * sigmoid (Cody-Waite reduction, degree-7 Taylor series, correctly rounded
 * add and divide); softmax -> fl32(l + b).  Group score = fl32 sum of the
 * group's group_topn largest keys.  group_topn = 1 is DeepSeek-v2's
 * device-limited routing ([EVO] §DeepSeek-v2): with one group per device,
 * the kept groups are exactly the devices met first when walking the
 * experts from the highest key down, so a token reaches at most
 * topk_groups devices.  Workspace: moe_workspace_size bytes suffice; with
 * x != NULL the router GEMM's partial sums and weight pieces live there
 * (MOE_ERR_WORKSPACE if ws is NULL or smaller), with x == NULL none is
 * used. */
moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router,
                     float* logits, const float* bias, int32_t* topk_idx,
                     float* topk_gate, float* topk_score, float* token_lse,
                     void* ws, size_t ws_bytes, void* stream);

/* Dispatch ([EVO] §GShard expert capacity; §DeepSeek-v2 device-level
 * dropping, lowest-scored tokens first): per-expert counts, optional
 * dropping, permutation.  Rows are grouped by expert (ascending), ascending
 * token order inside an expert.
 *   capacity C > 0: an expert keeps its C assignments of highest topk_score;
 *   group_capacity: each group of N/n_groups consecutive experts keeps its
 *   cap highest-scored assignments (cap = group_capacity, or the average
 *   group load ceil(T*k/n_groups) for -1).
 * Order among equal scores: lower token first, then lower expert.  The
 * decision uses topk_score exactly as given (fp32).
 *   topk_idx, topk_score [T,k]; x [T,H] act_dtype or NULL
 *   counts [N] i32 (before dropping), offsets [N+1] i32 (after dropping),
 *   row_token [T*k] i32, inv_row [T,k] i32 (-1 = dropped),
 *   x_perm [T*k, H] act_dtype or NULL: x_perm[r] = x[row_token[r]] for
 *   r < offsets[N]; n_dropped [2] i32 or NULL: dropped assignments, tokens
 *   with every assignment dropped.
 * Dropping needs T < 2^24 (MOE_ERR_UNSUPPORTED otherwise). */
moe_status moe_permute(const moe_cfg* cfg, const int32_t* topk_idx,
                       const float* topk_score, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* row_token, int32_t* inv_row,
                       void* x_perm, int32_t* n_dropped, void* ws,
                       size_t ws_bytes, void* stream);

/* Grouped SwiGLU experts over row segments ([EVO] §DeepSeek-v1 fine-grained
 * experts; the expert's form is SwiGLU: y = Wd (silu(Wg a) * (Wu a))).
 * Segment s covers rows [seg_offsets[s], seg_offsets[s+1]) and uses
 *   w13 + s*2*inter*H ([2*inter, H]: gate rows then up rows) and
 *   w2  + s*H*inter   ([H, inter]).
 *   seg_offsets [n_segments+1] i32 DEVICE, non-decreasing, from 0;
 *            NULL = one segment of max_rows rows
 *   max_rows  upper bound on seg_offsets[n_segments] (sizes y and the
 *            workspace); rows beyond seg_offsets[n_segments] are untouched
 *   a        activations; row r of the problem reads a[row_index[r]] when
 *            row_index != NULL, else a[r]; [*, H] act_dtype
 *   y        [max_rows, H] act_dtype output
 * act_dtype == w_dtype == bf16: bf16 MFMA, fp32 accumulate, the SwiGLU
 * product rounded to bf16 once.  f32: fp32 arithmetic throughout.
 * Workspace: moe_grouped_ffn_workspace_size. */
moe_status moe_grouped_ffn(const moe_cfg* cfg, int32_t n_segments,
                           const int32_t* seg_offsets, int32_t max_rows,
                           int32_t inter, const void* a,
                           const int32_t* row_index, const void* w13,
                           const void* w2, void* y, void* ws, size_t ws_bytes,
                           void* stream);
moe_status moe_grouped_ffn_workspace_size(const moe_cfg* cfg, int32_t max_rows,
                                          int32_t inter, size_t* bytes);

/* Combine ([BUILD] §2.2: shared output plus routed output; [EVO] §GShard:
 * a dropped assignment contributes nothing, the token keeps its residual
 * outside the layer):
 *   out[t] = y_shared[t] + sum_{j<k, inv_row[t,j] >= 0} gate[t,j] * y_perm[inv_row[t,j]]
 * summed in fp32 in slot order, rounded once to act_dtype.
 *   y_perm [*, H], y_shared [T,H] or NULL, out [T,H] (act_dtype). */
moe_status moe_combine(const moe_cfg* cfg, const void* y_perm,
                       const int32_t* inv_row, const float* topk_gate,
                       const void* y_shared, void* out, void* stream);

/* Load statistics ([EVO] §ST-MoE): f_e = counts_e / (k T);
 * P_e = sum_t s[t,e] / sum_t sum_e' s[t,e'] (the expert's share of all
 * score mass, all N experts, no bias); L_B = N sum_e f_e P_e;
 * z = (1/T) sum_t LSE(l_t); z_sq = (1/T) sum_t LSE(l_t)^2.
 *   counts [N] i32, token_lse [T] f32, logits [T,N] f32 ->
 *   f [N] f32, P [N] f32, scalars [3] f32 = {L_B, z, z_sq}.
 * Reductions are accumulated in fp64 in a fixed order. */
moe_status moe_load_stats(const moe_cfg* cfg, const int32_t* counts,
                          const float* token_lse, const float* logits, float* f,
                          float* P, float* scalars, void* ws, size_t ws_bytes,
                          void* stream);

/* Sequence-wise load statistics ([EVO] §DeepSeek-v3, sequence-wise balance
 * loss; the pages print no formula, so these are moe_load_stats's f, P and
 * L_B computed over the tokens of one sequence instead of the batch):
 * sequence q covers tokens [cu_seqlens[q], cu_seqlens[q+1]); its counts come
 * from topk_idx (before any dropping).
 *   cu_seqlens [n_seq+1] i32 DEVICE, non-decreasing from 0 to T (values are
 *            clamped to [0, T]; outputs for other inputs are unspecified);
 *   topk_idx [T,k] i32, token_lse [T] f32 (needed for softmax), logits [T,N]
 *   -> f_seq [n_seq,N] f32, P_seq [n_seq,N] f32, L_seq [n_seq] f32, and
 *   L_mean [1] f32 or NULL: mean of L_seq over the non-empty sequences
 *   (0 when there are none).  An empty sequence has f = P = 0, L = 0.
 * fp64 accumulation in a fixed order.  Workspace:
 * moe_seq_load_stats_workspace_size. */
moe_status moe_seq_load_stats(const moe_cfg* cfg, int32_t n_seq, const int32_t* cu_seqlens,
                              const int32_t* topk_idx, const float* token_lse,
                              const float* logits, float* f_seq, float* P_seq, float* L_seq,
                              float* L_mean, void* ws, size_t ws_bytes, void* stream);
moe_status moe_seq_load_stats_workspace_size(const moe_cfg* cfg, int32_t n_seq, size_t* bytes);

/* Device-level load statistics ([EVO] §DeepSeek-v1, device-level balance
 * loss; no formula printed): the cfg's n_groups groups of consecutive
 * experts stand for devices; F_g = sum of f over the group (its share of
 * the assignments), P_g = sum of P (its share of the score mass), L_dev =
 * n_groups * sum_g F_g P_g (1 when balanced; the expert-level L_B when every
 * group holds one expert).
 *   f, P [N] f32 (moe_load_stats outputs) -> F_group [n_groups] f32 or NULL,
 *   P_group [n_groups] f32 or NULL, L_dev [1] f32 or NULL.  No workspace. */
moe_status moe_group_load_stats(const moe_cfg* cfg, const float* f, const float* P,
                                float* F_group, float* P_group, float* L_dev, void* stream);

/* Auxiliary-loss-free bias update ([EVO] §DeepSeek-v3): with c the
 * per-expert counts and cbar their mean, b_e <- b_e + u * sign(cbar - c_e),
 * sign(0) = 0.  bias [N] f32 updated in place. */
moe_status moe_bias_update(const moe_cfg* cfg, const int32_t* counts,
                           float* bias, float u, void* stream);

/* The whole layer ([BUILD] §2.2, the layer's forward pass: the shared
 * experts' output plus the gate-weighted outputs of the routed experts the
 * router picked; [EVO] §DeepSeek-v3 and [GLR] §1, §3 for the routing):
 *   out [T,H] = shared(x) + sum of gated routed experts, the calls above
 * run in order (router GEMM, route, dispatch, grouped SwiGLU for the routed
 * and shared experts, combine, load statistics) on one stream.
 * x [T,H] act_dtype; bias [N] f32 or NULL; aux NULL or as above.
 * Workspace: moe_workspace_size(cfg); MOE_ERR_WORKSPACE if ws is NULL or
 * smaller.  Errors as for the granular calls, all detected before any
 * launch. */
moe_status moe_layer_forward(const moe_cfg* cfg, const moe_weights* weights,
                             const void* x, const float* bias, void* out,
                             const moe_aux* aux, void* ws, size_t ws_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * moe_layer_forward without a workspace argument.  Its scratch is one fixed
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held until the process ends; the call itself allocates nothing.
 * Arguments, outputs and errors as moe_layer_forward, plus
 * MOE_ERR_TOO_LARGE when moe_workspace_size(cfg) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. a V3-shaped layer up to about
 * 250 tokens, hidden 2048 / 64 experts up to about 1200), checked before
 * anything is enqueued.  The first call on a GPU looks up the array's device
 * address with that GPU current (make it outside any graph capture).  Every
 * call on one GPU uses the same scratch: calls that overlap in time on one
 * GPU (other streams, other host threads) race and give undefined results;
 * calls in stream order are safe, since each call clears what it
 * accumulates into. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_cfg* cfg, const moe_weights* weights,
                                     const void* x, const float* bias, void* out,
                                     const moe_aux* aux, void* stream);

/* Diagnostic (a property of the hardware, not a step of the method): the
 * SIMD each wave of a large-tile-shaped workgroup (512 threads, one per CU)
 * runs on.  simd [n_workgroups*8] i32 DEVICE receives, for wave w of
 * workgroup g, its SIMD number 0..3 at simd[8g + w].  The prefill GEMM
 * kernels run fastest when waves w and w + 4 share a SIMD (their results do
 * not depend on it).  n_workgroups < 0, or simd NULL with n_workgroups > 0:
 * MOE_ERR_INVALID_ARG. */
moe_status moe_probe_wave_simd(int32_t n_workgroups, int32_t* simd, void* stream);

/* Static string for a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
