/*
 * moe_oracle.c -- the CPU parity reference for one DeepSeekMoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).  Plain loops, one thread,
 * no blocking, no fusion, no reordering beyond the definitions cited at each
 * function.  Build: gcc -std=c11 -O2 -ffp-contract=off (no fast-math), so
 * every fp32 operation below is one IEEE-754 operation.
 *
 * Parity pins: every function here is pinned by tests in tests/test_oracle_*.py
 * (closed forms, invariants, brute force, special cases); the SwiGLU form of
 * the expert is a definition the pages do not print ("parity unpinned" as to
 * the choice of SwiGLU itself; its arithmetic is pinned against fp64 matmuls).
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

static float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* element i of a typed array, widened exactly */
static double typed_at(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_BF16) return (double)bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

/* A value with its index; ordering = value descending, then index ascending.
 * This is the tie rule for every selection the method makes. */
typedef struct {
  float v;
  int i;
} vi_t;

static int vi_cmp(const void* a, const void* b) {
  const vi_t* x = (const vi_t*)a;
  const vi_t* y = (const vi_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->i < y->i) ? -1 : (x->i > y->i);
}

/* ---------------------------------------------------------------- sigmoid */

/* e^x in fp32 for x in [-87, 87]: Cody & Waite reduction x = n ln2 + r with
 * the two-part ln 2 of fdlibm's single-precision exponential, then the
 * degree-7 Taylor series of e^r (|r| <= ln2/2, truncation < 2^-27). */
static float exp32_cw(float x) {
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e4p-1f;
  const float ln2_lo = 0x1.7f7d1cp-20f;
  float n = rintf(x * log2e);
  float r = fmaf(-n, ln2_hi, x);
  r = fmaf(-n, ln2_lo, r);
  /* sum_{j=0..7} r^j / j!, highest power first */
  float p = 1.0f / 5040.0f;
  p = fmaf(p, r, 1.0f / 720.0f);
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

/* s = 1/(1+e^-l): the v3 gate turns each logit into an independent score in
 * (0,1) ([EVO] §DeepSeek-v3, sigmoid gating). */
float orc_sigmoid32(float l) {
  float x = -l;
  x = fminf(fmaxf(x, -87.0f), 87.0f);
  float e = exp32_cw(x);
  return 1.0f / (1.0f + e);
}

void orc_sigmoid32_array(const float* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sigmoid32(in[i]);
}

/* ---------------------------------------------------------------- softmax */

/* Sum of slots [a, b) of v by recursive halving: the left half's sum plus
 * the right half's, one fp32 add per node. */
static float pairwise_sum32(const float* v, int a, int b) {
  if (b - a == 1) return v[a];
  const int mid = a + (b - a) / 2;
  return pairwise_sum32(v, a, mid) + pairwise_sum32(v, mid, b);
}

/* p_i = e^{l_i} / sum_j e^{l_j} over the token's logits ([EVO] §ST-MoE), in
 * fp32 with every step fixed (see moe_oracle.h): shifted by the largest
 * logit, terms more than 64 below it set to 0, the sum a pairwise tree over
 * 256 slots. */
int orc_softmax32(int N, const float* logits, float* s) {
  if (N < 1 || N > 256) return -1;
  float m = logits[0];
  for (int e = 1; e < N; ++e)
    if (logits[e] > m) m = logits[e];
  float E[256];
  for (int e = 0; e < 256; ++e) E[e] = 0.0f;
  for (int e = 0; e < N; ++e) {
    const float x = logits[e] - m;
    E[e] = (x < -64.0f) ? 0.0f : exp32_cw(x);
  }
  const float S = pairwise_sum32(E, 0, 256);
  for (int e = 0; e < N; ++e) s[e] = E[e] / S;
  return 0;
}

/* ---------------------------------------------------------------- logits */

void orc_router_logits(int T, int H, int N, const void* x, int x_dtype,
                       const void* wg, int wg_dtype, double* out) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < N; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += typed_at(x, x_dtype, (int64_t)t * H + h) *
               typed_at(wg, wg_dtype, (int64_t)e * H + h);
      out[(int64_t)t * N + e] = acc;
    }
}

/* ---------------------------------------------------------------- routing */

/* Per token ([EVO] §DeepSeek-v3; [GLR] §1 and §3):
 *  1. score s_e: sigmoid(l_e) (v3) or softmax over all N logits (v1/v2);
 *  2. selection key: s_e + b_e for sigmoid (bias steers selection only);
 *     for softmax the key is the logit itself (+ b_e if given), which orders
 *     experts exactly as the softmax probability does;
 *  3. with n_groups > 1: group score = sum of the group's group_topn largest
 *     keys, keep the topk_groups best groups, experts of other groups are
 *     not candidates;
 *  4. the k largest keys among candidates, in descending order (slot order);
 *  5. gate_j = s of the chosen expert (unbiased), divided by the sum of the
 *     k chosen scores when norm_topk, times route_scale. */
int orc_route(const orc_route_cfg* c, const float* logits, const float* bias,
              int32_t* topk_idx, double* topk_gate, float* topk_score,
              double* lse, uint8_t* kept_groups) {
  const int N = c->N, k = c->k, G = c->n_groups;
  if (N <= 0 || k < 0 || G <= 0 || N % G != 0) return -1;
  const int gs = N / G;
  if (c->topk_groups < 1 || c->topk_groups > G) return -1;
  if (k > c->topk_groups * gs) return -1;
  if (G > 1 && (c->group_topn < 1 || c->group_topn > gs)) return -1;
  if (c->score_fn != ORC_SIGMOID && N > 256) return -1; /* orc_softmax32's domain */

  vi_t* ek = (vi_t*)malloc(sizeof(vi_t) * N);
  vi_t* gk = (vi_t*)malloc(sizeof(vi_t) * G);
  vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * gs);
  float* s32 = (float*)malloc(sizeof(float) * N);
  double* s64 = (double*)malloc(sizeof(double) * N);
  uint8_t* keep = (uint8_t*)malloc(G);

  for (int t = 0; t < c->T; ++t) {
    const float* l = logits + (int64_t)t * N;

    /* log-sum-exp of the logits (used by the z-loss) */
    double m = -INFINITY;
    for (int e = 0; e < N; ++e) m = fmax(m, (double)l[e]);
    double se = 0.0;
    for (int e = 0; e < N; ++e) se += exp((double)l[e] - m);
    lse[t] = m + log(se);

    /* 1. scores (fp32: they decide drops, and the gate is taken from them) */
    if (c->score_fn == ORC_SIGMOID) {
      for (int e = 0; e < N; ++e) s32[e] = orc_sigmoid32(l[e]);
    } else {
      orc_softmax32(N, l, s32);
    }
    for (int e = 0; e < N; ++e) s64[e] = (double)s32[e];
    /* 2. keys */
    for (int e = 0; e < N; ++e) {
      float b = bias ? bias[e] : 0.0f;
      float base = (c->score_fn == ORC_SIGMOID) ? s32[e] : l[e];
      ek[e].v = base + b;
      ek[e].i = e;
    }
    /* 3. group limit */
    for (int q = 0; q < G; ++q) keep[q] = 1;
    if (G > 1) {
      for (int q = 0; q < G; ++q) {
        memcpy(tmp, ek + (int64_t)q * gs, sizeof(vi_t) * gs);
        qsort(tmp, gs, sizeof(vi_t), vi_cmp);
        float g = tmp[0].v;
        for (int j = 1; j < c->group_topn; ++j) g = g + tmp[j].v;
        gk[q].v = g;
        gk[q].i = q;
      }
      qsort(gk, G, sizeof(vi_t), vi_cmp);
      for (int q = 0; q < G; ++q) keep[q] = 0;
      for (int j = 0; j < c->topk_groups; ++j) keep[gk[j].i] = 1;
    }
    if (kept_groups)
      for (int q = 0; q < G; ++q) kept_groups[(int64_t)t * G + q] = keep[q];

    /* 4. top-k among candidates */
    int nc = 0;
    for (int e = 0; e < N; ++e)
      if (keep[e / gs]) ek[nc++] = ek[e];
    qsort(ek, nc, sizeof(vi_t), vi_cmp);

    /* 5. gates */
    double ssum = 0.0;
    for (int j = 0; j < k; ++j) ssum += s64[ek[j].i];
    for (int j = 0; j < k; ++j) {
      int e = ek[j].i;
      double g = s64[e];
      if (c->norm_topk) g = g / ssum;
      topk_idx[(int64_t)t * k + j] = e;
      topk_gate[(int64_t)t * k + j] = g * c->route_scale;
      topk_score[(int64_t)t * k + j] = s32[e];
    }
  }
  free(ek);
  free(gk);
  free(tmp);
  free(s32);
  free(s64);
  free(keep);
  return 0;
}

/* ---------------------------------------------------------------- dispatch */

/* Group every (token, slot) assignment by expert ([EVO] §GShard: experts
 * receive the tokens routed to them; expert capacity).  With capacity C > 0
 * an expert keeps at most C assignments: the ones with the highest unbiased
 * score, lower token index first among equal scores; the rest are dropped
 * and the token reaches the next layer through the residual ([EVO] §GShard
 * expert capacity; §DeepSeek-v2 drops the lowest-scored tokens first).
 * Rows are laid out expert by expert, ascending token order inside an
 * expert. */
int orc_dispatch(int T, int N, int k, int capacity, const int32_t* topk_idx,
                 const float* topk_score, int32_t* counts, int32_t* offsets,
                 int32_t* row_token, int32_t* inv_row, int64_t* drop_stats) {
  if (T < 0 || N <= 0 || k < 0 || capacity < 0) return -1;
  const int64_t A = (int64_t)T * k;
  for (int e = 0; e < N; ++e) counts[e] = 0;
  for (int64_t a = 0; a < A; ++a) {
    int e = topk_idx[a];
    if (e < 0 || e >= N) return -1;
    counts[e]++;
  }
  for (int64_t a = 0; a < A; ++a) inv_row[a] = -1;

  /* kept flag per assignment */
  uint8_t* kept = (uint8_t*)malloc(A > 0 ? A : 1);
  for (int64_t a = 0; a < A; ++a) kept[a] = 1;
  vi_t* cand = (vi_t*)malloc(sizeof(vi_t) * (T > 0 ? T : 1));
  int64_t* slot_of = (int64_t*)malloc(sizeof(int64_t) * (T > 0 ? T : 1));
  int64_t dropped = 0;
  if (capacity > 0) {
    for (int e = 0; e < N; ++e) {
      if (counts[e] <= capacity) continue;
      /* this expert's assignments in token order; a token picks an expert
         at most once, so the token index identifies the assignment */
      int n = 0;
      for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
          if (topk_idx[(int64_t)t * k + j] == e) {
            cand[n].v = topk_score[(int64_t)t * k + j];
            cand[n].i = t;
            slot_of[t] = (int64_t)t * k + j;
            ++n;
          }
      qsort(cand, n, sizeof(vi_t), vi_cmp);
      for (int r = capacity; r < n; ++r) {
        kept[slot_of[cand[r].i]] = 0;
        ++dropped;
      }
    }
  }
  offsets[0] = 0;
  for (int e = 0; e < N; ++e) {
    int ke = (capacity > 0 && counts[e] > capacity) ? capacity : counts[e];
    offsets[e + 1] = offsets[e] + ke;
  }
  for (int e = 0; e < N; ++e) {
    int r = offsets[e];
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {
        int64_t a = (int64_t)t * k + j;
        if (topk_idx[a] == e && kept[a]) {
          row_token[r] = t;
          inv_row[a] = r;
          ++r;
        }
      }
  }
  int64_t all_dropped = 0;
  for (int t = 0; t < T && k > 0; ++t) {
    int any = 0;
    for (int j = 0; j < k; ++j) any |= kept[(int64_t)t * k + j];
    if (!any) ++all_dropped;
  }
  drop_stats[0] = dropped;
  drop_stats[1] = all_dropped;
  free(kept);
  free(cand);
  free(slot_of);
  return 0;
}

/* Device-level token drop ([EVO] §DeepSeek-v2, device-level token dropping):
 * experts are split into G equal groups (one group per device); a group
 * whose assignments exceed `group_cap` keeps the group_cap assignments with
 * the highest scores and drops the rest.  Order among equal scores: lower
 * token first, then lower expert.  Rows are laid out expert by expert, token
 * order inside an expert, as in orc_dispatch. */
typedef struct {
  float s;
  int t, e;
  int64_t slot;
} drop_cand_t;

static int drop_cand_cmp(const void* a, const void* b) {
  const drop_cand_t* x = (const drop_cand_t*)a;
  const drop_cand_t* y = (const drop_cand_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  if (x->t != y->t) return x->t < y->t ? -1 : 1;
  return (x->e < y->e) ? -1 : (x->e > y->e);
}

int orc_dispatch_grouped(int T, int N, int k, int G, int group_cap, const int32_t* topk_idx,
                         const float* topk_score, int32_t* counts, int32_t* offsets,
                         int32_t* row_token, int32_t* inv_row, int64_t* drop_stats) {
  if (T < 0 || N <= 0 || k < 0 || G <= 0 || N % G != 0 || group_cap <= 0) return -1;
  const int gs = N / G;
  const int64_t A = (int64_t)T * k;
  for (int e = 0; e < N; ++e) counts[e] = 0;
  for (int64_t a = 0; a < A; ++a) {
    int e = topk_idx[a];
    if (e < 0 || e >= N) return -1;
    counts[e]++;
  }
  uint8_t* kept = (uint8_t*)malloc(A > 0 ? A : 1);
  for (int64_t a = 0; a < A; ++a) kept[a] = 1;
  drop_cand_t* cand = (drop_cand_t*)malloc(sizeof(drop_cand_t) * (A > 0 ? A : 1));
  int64_t dropped = 0;
  for (int g = 0; g < G; ++g) {
    int64_t n = 0;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {
        const int64_t a = (int64_t)t * k + j;
        const int e = topk_idx[a];
        if (e / gs != g) continue;
        cand[n].s = topk_score[a];
        cand[n].t = t;
        cand[n].e = e;
        cand[n].slot = a;
        ++n;
      }
    if (n <= group_cap) continue;
    qsort(cand, (size_t)n, sizeof(drop_cand_t), drop_cand_cmp);
    for (int64_t r = group_cap; r < n; ++r) {
      kept[cand[r].slot] = 0;
      ++dropped;
    }
  }
  for (int64_t a = 0; a < A; ++a) inv_row[a] = -1;
  offsets[0] = 0;
  int r = 0;
  for (int e = 0; e < N; ++e) {
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {
        const int64_t a = (int64_t)t * k + j;
        if (topk_idx[a] == e && kept[a]) {
          row_token[r] = t;
          inv_row[a] = r;
          ++r;
        }
      }
    offsets[e + 1] = r;
  }
  int64_t all_dropped = 0;
  for (int t = 0; t < T && k > 0; ++t) {
    int any = 0;
    for (int j = 0; j < k; ++j) any |= kept[(int64_t)t * k + j];
    if (!any) ++all_dropped;
  }
  drop_stats[0] = dropped;
  drop_stats[1] = all_dropped;
  free(kept);
  free(cand);
  return 0;
}

/* ---------------------------------------------------------------- experts */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert on one row, with the gate/up/down weights addressed through
 * strides so that one member of a packed set of experts can be evaluated on
 * its own.  gate row i = w13[(g0 + i) * H], up row i = w13[(u0 + i) * H],
 * down element (o, i) = w2[o * ld2 + d0 + i]. */
static void swiglu_row_strided(int H, int I, const void* x, int x_dtype,
                               const void* w13, int64_t g0, int64_t u0,
                               const void* w2, int64_t ld2, int64_t d0,
                               int w_dtype, double* y_acc, double scale) {
  double* h = (double*)malloc(sizeof(double) * (I > 0 ? I : 1));
  for (int i = 0; i < I; ++i) {
    double a = 0.0, u = 0.0;
    for (int c = 0; c < H; ++c) {
      double xv = typed_at(x, x_dtype, c);
      a += typed_at(w13, w_dtype, (g0 + i) * H + c) * xv;
      u += typed_at(w13, w_dtype, (u0 + i) * H + c) * xv;
    }
    h[i] = silu(a) * u;
  }
  for (int o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += typed_at(w2, w_dtype, o * ld2 + d0 + i) * h[i];
    y_acc[o] += scale * acc;
  }
  free(h);
}

void orc_swiglu_row(int H, int I, const void* x_row, int x_dtype,
                    const void* w13, const void* w2, int w_dtype, double* y) {
  for (int o = 0; o < H; ++o) y[o] = 0.0;
  swiglu_row_strided(H, I, x_row, x_dtype, w13, 0, I, w2, I, 0, w_dtype, y, 1.0);
}

/* Layer output = always-on shared experts, each with weight 1, plus the
 * gate-weighted routed experts ([BUILD] §2.2 layer forward; [EVO]
 * §DeepSeek-v1 shared-expert isolation).  The residual is not part of the
 * layer's output. */
void orc_token_output(int H, int k, int I, int n_shared, int I_sh,
                      const void* x_row, int x_dtype,
                      const void* const* w13_sel, const void* const* w2_sel,
                      const double* gates, const void* ws13, const void* ws2,
                      int w_dtype, double* out) {
  for (int o = 0; o < H; ++o) out[o] = 0.0;
  const int64_t Ish_all = (int64_t)n_shared * I_sh;
  for (int s = 0; s < n_shared; ++s)
    swiglu_row_strided(H, I_sh, x_row, x_dtype, ws13, (int64_t)s * I_sh,
                       Ish_all + (int64_t)s * I_sh, ws2, Ish_all,
                       (int64_t)s * I_sh, w_dtype, out, 1.0);
  for (int j = 0; j < k; ++j) {
    if (!w13_sel[j]) continue; /* dropped slot contributes nothing */
    swiglu_row_strided(H, I, x_row, x_dtype, w13_sel[j], 0, I, w2_sel[j], I, 0,
                       w_dtype, out, gates[j]);
  }
}

void orc_combine(int T, int H, int k, const void* y, const void* y_sh, int dtype,
                 const int32_t* inv_row, const double* gate, double* out) {
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      double acc = y_sh ? typed_at(y_sh, dtype, (int64_t)t * H + h) : 0.0;
      for (int j = 0; j < k; ++j) {
        int r = inv_row[(int64_t)t * k + j];
        if (r < 0) continue;
        acc += gate[(int64_t)t * k + j] * typed_at(y, dtype, (int64_t)r * H + h);
      }
      out[(int64_t)t * H + h] = acc;
    }
}

/* ---------------------------------------------------------------- stats */

void orc_load_stats(int T, int N, int k, int score_fn, const float* logits,
                    const int32_t* counts, double* f, double* P,
                    double* scalars) {
  double* col = (double*)calloc(N, sizeof(double));
  double z = 0.0, z2 = 0.0;
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * N;
    double m = -INFINITY;
    for (int e = 0; e < N; ++e) m = fmax(m, (double)l[e]);
    double se = 0.0;
    for (int e = 0; e < N; ++e) se += exp((double)l[e] - m);
    double lse = m + log(se);
    z += lse;
    z2 += lse * lse;
    for (int e = 0; e < N; ++e) {
      double s = (score_fn == ORC_SIGMOID) ? (double)orc_sigmoid32(l[e])
                                           : exp((double)l[e] - m) / se;
      col[e] += s;
    }
  }
  double tot = 0.0;
  for (int e = 0; e < N; ++e) tot += col[e];
  double lb = 0.0;
  for (int e = 0; e < N; ++e) {
    f[e] = (T > 0 && k > 0) ? (double)counts[e] / ((double)k * T) : 0.0;
    P[e] = tot > 0.0 ? col[e] / tot : 0.0;
    lb += f[e] * P[e];
  }
  scalars[0] = N * lb;
  scalars[1] = T > 0 ? z / T : 0.0;
  scalars[2] = T > 0 ? z2 / T : 0.0;
  free(col);
}

/* Sequence-wise balance statistics ([EVO] §DeepSeek-v3, sequence-wise
 * balance loss: the expert-level statistics of [EVO] §ST-MoE taken over the
 * tokens of one sequence instead of the whole batch).  Sequence q covers
 * tokens [cu_seqlens[q], cu_seqlens[q+1]); its counts come from topk_idx.
 * L_mean = mean of L_seq over the non-empty sequences (0 if none). */
int orc_seq_load_stats(int T, int N, int k, int score_fn, int n_seq, const int32_t* cu_seqlens,
                       const int32_t* topk_idx, const float* logits, double* f_seq,
                       double* P_seq, double* L_seq, double* L_mean) {
  if (T < 0 || N <= 0 || k < 0 || n_seq < 0) return -1;
  if (n_seq > 0 && (cu_seqlens[0] != 0 || cu_seqlens[n_seq] != T)) return -1;
  for (int q = 0; q < n_seq; ++q)
    if (cu_seqlens[q + 1] < cu_seqlens[q]) return -1;
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * N);
  double sum = 0.0;
  int nonempty = 0;
  for (int q = 0; q < n_seq; ++q) {
    const int a = cu_seqlens[q], b = cu_seqlens[q + 1];
    for (int e = 0; e < N; ++e) counts[e] = 0;
    for (int64_t i = (int64_t)a * k; i < (int64_t)b * k; ++i) {
      const int e = topk_idx[i];
      if (e < 0 || e >= N) {
        free(counts);
        return -1;
      }
      counts[e]++;
    }
    double sc[3];
    orc_load_stats(b - a, N, k, score_fn, logits + (int64_t)a * N, counts, f_seq + (int64_t)q * N,
                   P_seq + (int64_t)q * N, sc);
    L_seq[q] = sc[0];
    if (b > a) {
      sum += sc[0];
      ++nonempty;
    }
  }
  *L_mean = nonempty > 0 ? sum / nonempty : 0.0;
  free(counts);
  return 0;
}

/* Device-level balance statistics ([EVO] §DeepSeek-v1, device-level balance
 * loss: the experts split into G groups, one per device, balanced at group
 * granularity).  F_g = sum of f over the group's experts (share of the
 * assignments), P_g = sum of P (share of the score mass), L_dev =
 * G * sum_g F_g P_g, which is 1 for a uniform load and, with one expert per
 * group, the expert-level L_B. */
int orc_group_load_stats(int N, int G, const double* f, const double* P, double* F_g,
                         double* P_g, double* L_dev) {
  if (N <= 0 || G <= 0 || N % G != 0) return -1;
  const int gs = N / G;
  double l = 0.0;
  for (int g = 0; g < G; ++g) {
    double a = 0.0, b = 0.0;
    for (int e = g * gs; e < (g + 1) * gs; ++e) {
      a += f[e];
      b += P[e];
    }
    F_g[g] = a;
    P_g[g] = b;
    l += a * b;
  }
  *L_dev = G * l;
  return 0;
}

/* ---------------------------------------------------------------- bias */

void orc_bias_update(int N, const int32_t* counts, const float* bias_in,
                     float u, float* bias_out) {
  double mean = 0.0;
  for (int e = 0; e < N; ++e) mean += counts[e];
  mean /= N;
  for (int e = 0; e < N; ++e) {
    double err = mean - counts[e];
    float step = (err > 0) ? u : (err < 0 ? -u : 0.0f);
    bias_out[e] = bias_in[e] + step;
  }
}
