/*
 * moe_oracle.h -- plain, slow, single-threaded CPU definition of one
 * DeepSeekMoE layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the parity reference.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or constant generator with the HIP
 * library under routing_expert_ffn_sigmoid_amd/csrc, and neither includes
 * the other.
 *
 * Sources (web pages, cited by title and section):
 *   [EVO]   "DeepSeek MoE：从v1到v3的演进" (wln20.github.io)
 *   [GLR]   "DeepSeek-V3的Group-Limited Expert Routing与负载均衡优化实践" (mhpn.cn)
 *   [BUILD] "从零构建DeepSeekMoE：揭秘混合专家模型中的负载均衡与专家协同机制"
 *           (opc.csdn.net)
 *   [TECH]  "DeepSeek-V3技术解密：DeepSeekMoE架构如何重塑AI模型效能边界"
 *
 * Precision: every floating-point result is computed in fp64, except the
 * quantities that decide an integer (expert choice, group choice, capacity
 * drop order).  Those are taken in fp32, the router precision [TECH] section
 * "四、开发者实践指南" item 2 keeps, with the fp32 sigmoid defined below.
 *
 * Typed inputs: arrays marked (typed) are fp32 (ORC_F32) or raw bfloat16
 * bit patterns (ORC_BF16, uint16).  A bf16 value is widened to fp32 exactly.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1

/* fp32 sigmoid used for expert scores.  Definition (shared by the spec of
 * both implementations, written independently in each):
 *   x  = clamp(-l, -87, 87)
 *   n  = round-half-even(fl32(x * log2(e)))
 *   r  = fma(-n, LN2_HI, x); r = fma(-n, LN2_LO, r)   (Cody & Waite split)
 *   p  = Taylor polynomial of e^r to degree 7, Horner with fma
 *   E  = p * 2^n (exact scaling)
 *   s  = 1 / (1 + E), correctly rounded fp32 add and divide.
 * NaN logits are outside the supported domain. */
float orc_sigmoid32(float l);
void orc_sigmoid32_array(const float* in, float* out, int64_t n);

/* fp32 softmax over one token's N logits (N <= 256), the score the v1/v2 gate
 * takes and the drop order of device-level dropping is decided on ([EVO]
 * §ST-MoE p_i(x); §DeepSeek-v2 device-level token dropping).  Definition
 * (written independently on each side):
 *   m   = the largest logit
 *   E_e = the exponential of the sigmoid above applied to fl32(l_e - m),
 *         except E_e = 0 when fl32(l_e - m) < -64
 *   S   = pairwise sum of E over 256 slots (slots e >= N hold 0): the sum of
 *         slots [a, b) is sum[a, (a+b)/2) + sum[(a+b)/2, b), down to single
 *         slots, each + one correctly rounded fp32 add
 *   s_e = E_e / S, correctly rounded fp32 divide.
 * Returns -1 when N is outside 1..256. */
int orc_softmax32(int N, const float* logits, float* s);

/* Router logits l[t,e] = sum_h x[t,h] * Wg[e,h]  ([EVO] §ST-MoE z-loss: the
 * router's per-expert logits; [BUILD] §5.2 router is a linear layer).
 * x (typed) [T,H], wg (typed) [N,H]; out [T,N] fp64. */
void orc_router_logits(int T, int H, int N, const void* x, int x_dtype,
                       const void* wg, int wg_dtype, double* out);

typedef struct {
  int T, N, k;
  int n_groups;     /* 1 = no group limit */
  int topk_groups;  /* groups kept */
  int group_topn;   /* keys summed into a group score (1 or 2) */
  int score_fn;     /* ORC_SOFTMAX or ORC_SIGMOID */
  int norm_topk;    /* 1: gates divided by the sum of the selected scores */
  double route_scale;
} orc_route_cfg;

/* Score, select and gate every token.  logits [T,N] fp32 (the values the
 * selection is made on), bias [N] fp32 or NULL.
 * Outputs: topk_idx [T,k], topk_gate [T,k] fp64, topk_score [T,k] fp32
 * (unbiased score of the chosen expert), lse [T] fp64 (log-sum-exp of the
 * logits), kept_groups [T,n_groups] (1 = kept) or NULL.
 * Returns 0, or -1 on an invalid configuration. */
int orc_route(const orc_route_cfg* cfg, const float* logits, const float* bias,
              int32_t* topk_idx, double* topk_gate, float* topk_score,
              double* lse, uint8_t* kept_groups);

/* Dispatch: per-expert counts, optional capacity drop, permutation.
 * capacity 0 = unlimited.  Outputs: counts [N] (before capacity),
 * offsets [N+1] (after capacity), row_token [T*k] (first offsets[N] used),
 * inv_row [T*k] (-1 = dropped), drop_stats[2] = {dropped assignments,
 * tokens with every assignment dropped}.  Returns 0 or -1. */
int orc_dispatch(int T, int N, int k, int capacity, const int32_t* topk_idx,
                 const float* topk_score, int32_t* counts, int32_t* offsets,
                 int32_t* row_token, int32_t* inv_row, int64_t* drop_stats);

/* Dispatch with device-level token dropping: the N experts form G equal
 * groups (devices); a group holding more than group_cap assignments keeps
 * the group_cap highest-scoring ones (ties: lower token, then lower expert).
 * Outputs as orc_dispatch (counts before dropping).  Returns 0 or -1. */
int orc_dispatch_grouped(int T, int N, int k, int G, int group_cap, const int32_t* topk_idx,
                         const float* topk_score, int32_t* counts, int32_t* offsets,
                         int32_t* row_token, int32_t* inv_row, int64_t* drop_stats);

/* One SwiGLU expert on one row: y = Wd (silu(Wg x) * (Wu x)).
 * w13 (typed) [2I,H]: rows [0,I) gate, rows [I,2I) up; w2 (typed) [H,I]. */
void orc_swiglu_row(int H, int I, const void* x_row, int x_dtype,
                    const void* w13, const void* w2, int w_dtype, double* y);

/* Full layer output for one token:
 *   out = sum_{s<n_shared} SharedExpert_s(x) + sum_{j<k, kept} gate_j E_{e_j}(x)
 * w13_sel[j]/w2_sel[j]: weights of the expert in slot j, NULL = dropped slot.
 * ws13 (typed) [2*n_shared*I_sh, H] packs the shared experts' gate rows
 * (expert s at rows [s*I_sh,(s+1)*I_sh)) then their up rows (expert s at
 * rows [n_shared*I_sh + s*I_sh, ...)); ws2 (typed) [H, n_shared*I_sh]
 * packs their down columns the same way.  Each shared expert is evaluated
 * on its own. */
void orc_token_output(int H, int k, int I, int n_shared, int I_sh,
                      const void* x_row, int x_dtype,
                      const void* const* w13_sel, const void* const* w2_sel,
                      const double* gates, const void* ws13, const void* ws2,
                      int w_dtype, double* out);

/* Combine ([BUILD] §2.2 shared + routed; [EVO] §GShard dropped slots add
 * nothing): out[t] = y_sh[t] + sum_{j<k, inv_row[t,j] >= 0} gate[t,j] *
 * y[inv_row[t,j]].  y (typed) [*,H], y_sh (typed) [T,H] or NULL,
 * gate [T,k] fp64; out [T,H] fp64. */
void orc_combine(int T, int H, int k, const void* y, const void* y_sh, int dtype,
                 const int32_t* inv_row, const double* gate, double* out);

/* Load statistics ([EVO] §ST-MoE): f_e = c_e/(k T),
 * P_e = sum_t s[t,e] / sum_t sum_e' s[t,e'], L_B = N sum_e f_e P_e,
 * z = (1/T) sum_t LSE(l_t), z_sq = (1/T) sum_t LSE(l_t)^2.
 * scalars[3] = {L_B, z, z_sq}. */
void orc_load_stats(int T, int N, int k, int score_fn, const float* logits,
                    const int32_t* counts, double* f, double* P,
                    double* scalars);

/* Sequence-wise statistics: orc_load_stats's f, P and L_B over the tokens
 * [cu_seqlens[q], cu_seqlens[q+1]) of each sequence q (counts from
 * topk_idx).  f_seq, P_seq [n_seq, N]; L_seq [n_seq]; L_mean = mean of L_seq
 * over non-empty sequences.  cu_seqlens: n_seq+1 non-decreasing values from
 * 0 to T.  Returns 0 or -1. */
int orc_seq_load_stats(int T, int N, int k, int score_fn, int n_seq, const int32_t* cu_seqlens,
                       const int32_t* topk_idx, const float* logits, double* f_seq,
                       double* P_seq, double* L_seq, double* L_mean);

/* Device-level statistics over G equal expert groups: F_g = sum f, P_g =
 * sum P over the group, L_dev = G * sum_g F_g P_g.  Returns 0 or -1. */
int orc_group_load_stats(int N, int G, const double* f, const double* P, double* F_g,
                         double* P_g, double* L_dev);

/* Auxiliary-loss-free bias update ([EVO] §DeepSeek-v3):
 * e_i = mean(c) - c_i ; b_i <- b_i + u * sign(e_i), sign(0) = 0.
 * Returned in fp32 (the bias is an fp32 tensor). */
void orc_bias_update(int N, const int32_t* counts, const float* bias_in,
                     float u, float* bias_out);

#ifdef __cplusplus
}
#endif
#endif
