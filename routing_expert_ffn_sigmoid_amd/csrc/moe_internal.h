// moe_internal.h -- device helpers and kernel-launcher declarations shared by
// the translation units of libmoe.so (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits in global memory
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two fp32 values rounded to bf16 (nearest even; NaN stays NaN) and packed,
// `lo` in the low half: one v_cvt_pk_bf16_f32 on gfx950, which matched the
// integer rounding (add 0x7fff plus the kept lsb, NaN quieted) bit for bit on
// 2^25 random pairs of bit patterns plus ties, denormals and infinities.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_hw v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Wave-wide butterfly reductions (64 lanes).
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger
// integer); -0 is folded onto +0 so the two compare equal, as floats do.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------ fp32 exponential
// e^x for x in [-87, 87], defined exactly so that every score a selection or
// a drop is decided on is reproducible bit for bit:
//   n = rne(fl32(x * log2 e));
//   r = fma(-n, ln2_hi, x); r = fma(-n, ln2_lo, r)     (Cody & Waite, with
//       fdlibm's two-part ln 2);
//   p = sum_{j<=7} r^j/j! by fma Horner; E = p * 2^n.
// For |x| <= 87 the result is a normal fp32 number.
__device__ __forceinline__ float exp32_cw(float x) {
#pragma clang fp contract(off)
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e4p-1f, x);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 1.0f / 5040.0f;
  p = __builtin_fmaf(p, r, 1.0f / 720.0f);
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, static_cast<int>(n));
}

// fp32 sigmoid s = 1 / (1 + exp32_cw(clamp(-l, -87, 87))), correctly rounded
// add and divide.  The clamp keeps every result a normal fp32 number (s
// saturates at sigma(-87) below l = -87).
__device__ __forceinline__ float sigmoid_score(float l) {
#pragma clang fp contract(off)
  const float x = __builtin_fminf(__builtin_fmaxf(-l, -87.0f), 87.0f);
  const float d = 1.0f + exp32_cw(x);
  return 1.0f / d;
}

// Softmax numerator of a logit l given the token's largest logit m:
// exp32_cw(l - m), and exactly 0 when l - m < -64 (such a term is below
// 2^-92 of the largest one, and the quotient by the sum, at most 256, stays a
// normal fp32 number for every term that is kept).
__device__ __forceinline__ float softmax_numerator(float l, float m) {
#pragma clang fp contract(off)
  const float x = l - m;
  return x < -64.0f ? 0.0f : exp32_cw(x);
}

// Sum over the 64 lanes by recursive halving in index order: after the step
// with offset o every lane holds the sum of its aligned block of 2o lanes,
// formed as (lower half) + (upper half).  With lane L holding the sum of
// entries 4L .. 4L+3 as (e0 + e1) + (e2 + e3), the result is the pairwise
// sum of 256 entries (a binary tree over index halves), the same on every
// lane.
__device__ __forceinline__ float wave_sum_pairwise_f32(float v) {
#pragma unroll
  for (int o = 1; o <= 32; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ------------------------------------------------------------------ launchers
// Every launcher enqueues on `st` and returns hipGetLastError().

// Router GEMM plan: the kernel, its K splits and the workspace it needs.
//   bf16 path (x bf16, H % 32 == 0): the router weight is first written to
//   the workspace as np bf16 pieces in the tiled fragment layout (np = 3
//   exact pieces of an fp32 weight, np = 1 for a bf16 weight), then a bf16
//   MFMA GEMM accumulates x * piece in fp32.
//   fp32 path (otherwise): fp32 MFMA straight from x and the weight.
// Logit partials part[s][t][e] = sum over split s of x[t,h] * wg[e,h] go to
// the workspace when splits > 1 (the route kernel adds them in split order),
// else straight to the logits.
struct RouterPlan {
  int bf16;            // 1: bf16 MFMA over weight pieces, 0: fp32 MFMA
  int np;              // weight pieces (bf16 path)
  int npad;            // N rounded up to 16 (rows of each piece)
  int splits;          // K splits
  int kchunk;          // K elements per split
  size_t part_bytes;   // workspace: partials at offset 0 (0 when splits == 1)
  size_t piece_off;    // workspace: pieces at this offset
  size_t ws_bytes;     // total workspace
};
RouterPlan router_plan(int T, int H, int N, int x_dtype, int wg_dtype);
// Enqueues the router GEMM; *part_out receives the partials (or the logits
// when splits == 1) for RouteParams.  ws holds plan.ws_bytes bytes.
hipError_t launch_router_gemm(const RouterPlan& rp, const void* x, int x_dtype, const void* wg,
                              int wg_dtype, float* logits, void* ws, int T, int H, int N,
                              const float** part_out, hipStream_t st);

// Tokens per dispatch block: the dispatch kernels count and rank each
// expert's assignments per block of this many tokens.
constexpr int kDispatchTokPerBlock = 256;

struct RouteParams {
  const float* part;  // [splits][T][N] logit partials (or the logits, splits = 1)
  int splits;
  float* logits;      // [T][N] out (may equal part when splits == 1)
  const float* bias;  // [N] or null
  int32_t* topk_idx;
  float* topk_gate;
  float* topk_score;
  float* token_lse;   // may be null
  // when not null: [ceil(T / kDispatchTokPerBlock)][N] per-block expert
  // counts, zero on entry; the route kernel adds its selections (integer
  // adds, so the counts do not depend on their order) and dispatch then
  // skips its counting pass
  int32_t* block_counts;
  int T, N, k, n_groups, topk_groups, group_topn, score_fn, norm_topk;
  float route_scale;
};
hipError_t launch_route(const RouteParams& p, hipStream_t st);

// Dropping policy of one dispatch: per-expert capacity, or a cap per group
// of n_groups consecutive experts (device-level dropping); at most one set.
struct DropPolicy {
  int capacity;   // per expert, 0 = none
  int n_groups;   // groups for group_cap
  int group_cap;  // per group, 0 = none (already resolved, > 0 when set)
  bool any() const { return capacity > 0 || group_cap > 0; }
};

struct DispatchWs {
  int32_t* block_counts;  // [nb][N]
  int32_t* block_base;    // [nb][N]
  int32_t* pre_off;       // [N]
  uint64_t* cand_key;     // [T*k] (dropping only)
  int32_t* cand_slot;     // [T*k] (dropping only)
  uint64_t* group_tau;    // [n_groups] (group dropping only)
  int32_t* kept;          // [N] (group dropping only)
};
int dispatch_blocks(int T);
size_t dispatch_ws_bytes(int T, int N, int k, const DropPolicy& d);
DispatchWs dispatch_ws_carve(void* ws, int T, int N, int k, const DropPolicy& d);
// zero the per-block counts the fused route kernel accumulates into
hipError_t launch_zero_block_counts(const DispatchWs& w, int T, int N, hipStream_t st);
// counts_ready: w.block_counts already holds the per-block counts of
// topk_idx (route kernel with RouteParams::block_counts)
hipError_t launch_dispatch(const int32_t* topk_idx, const float* topk_score, int T, int N,
                           int k, const DropPolicy& d, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, int32_t* inv_row, int32_t* n_dropped,
                           const DispatchWs& w, hipStream_t st, bool counts_ready = false);
hipError_t launch_permute(const void* x, int elem_bytes, int H, const int32_t* row_token,
                          const int32_t* offsets, int N, int max_rows, void* x_perm,
                          hipStream_t st);

// One problem group of the grouped SwiGLU GEMM.
struct FfnGroup {
  const void* A;            // activations [*, lda]
  int64_t lda;
  const int32_t* row_index; // optional gather: problem row r reads A[row_index[r]]
  const int32_t* seg_off;   // [nseg+1] device, or null = one segment of `rows`
  int32_t nseg;
  int32_t rows;             // used when seg_off == null
  const void* W;            // weights, segment s at W + s * w_stride (elements)
  int64_t w_stride;
  void* Out;                // [*, ldo]
  int64_t ldo;
  int32_t K;                // reduction length
  int32_t n_out;            // output columns (h cols in the gate/up phase)
  int32_t up_off;           // gate/up phase: row offset of the up half (= inter)
  uint32_t a_bytes;         // bytes addressable from A (buffer bound; 0 = unknown)
  uint32_t w_bytes;         // bytes of one segment's weights (buffer bound; 0 = unknown)
  uint32_t o_bytes;         // bytes addressable from Out (buffer bound; 0 = unknown)
};
// phase 0: gate/up + SwiGLU -> h;  phase 1: down projection -> y.
// `rows_hint`: expected rows per segment (chooses the tile height).
hipError_t launch_ffn_bf16(const FfnGroup* groups, int ngroups, int phase, int rows_hint,
                           hipStream_t st);
hipError_t launch_ffn_f32(const FfnGroup& g, int phase, int max_rows, hipStream_t st);
// SIMD of each wave of n_workgroups large-tile-shaped workgroups: simd[8g + w]
hipError_t launch_wave_simd_probe(int32_t* simd, int n_workgroups, hipStream_t st);

hipError_t launch_combine(const void* y_perm, const int32_t* inv_row, const float* gate,
                          const void* y_shared, void* out, int T, int H, int k,
                          int act_dtype, hipStream_t st);

int stats_blocks(int T);
size_t stats_ws_bytes(int T, int N);
hipError_t launch_stats(const int32_t* counts, const float* lse, const float* logits, int T,
                        int N, int k, int score_fn, float* f, float* P, float* scalars,
                        void* ws, hipStream_t st);
hipError_t launch_pack_tiled(const void* src, void* dst, int64_t n_mat, int R, int K,
                             hipStream_t st);
size_t seq_stats_ws_bytes(int T, int N, int n_seq);
hipError_t launch_seq_stats(const int32_t* cu, int n_seq, const int32_t* topk_idx,
                            const float* lse, const float* logits, int T, int N, int k,
                            int score_fn, float* f_seq, float* P_seq, float* L_seq,
                            float* L_mean, void* ws, hipStream_t st);
hipError_t launch_group_stats(const float* f, const float* P, int N, int G, float* F_g,
                              float* P_g, float* L_dev, hipStream_t st);
hipError_t launch_bias_update(const int32_t* counts, float* bias, int N, float u,
                              hipStream_t st);

}  // namespace moe
