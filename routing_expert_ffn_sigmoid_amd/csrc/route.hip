// route.hip -- router GEMM (fp32 MFMA) and per-token scoring, group-limited
// top-k and gates (one wavefront per token).
//
// Sources: "DeepSeek MoE：从v1到v3的演进" §DeepSeek-v3 (sigmoid score, bias
// used for selection only, gate from the unbiased score) and §ST-MoE (z-loss
// log-sum-exp); "DeepSeek-V3的Group-Limited Expert Routing与负载均衡优化实践"
// §1 and §3 (score the groups, keep the best ones, mask the rest, choose the
// top-k experts); "DeepSeek-V3技术解密…" §四.2 (router kept in fp32).
#include "moe_internal.h"

namespace moe {

// ============================================================ router GEMM
// logits partials part[s][t][e] = sum_{h in split s} x[t,h] * wg[e,h], fp32
// MFMA 16x16x4 with fp32 accumulation.  A wave owns 32 tokens x 64 experts
// (2 x 4 blocks of 16x16); a workgroup of 4 waves owns 32 tokens x 256
// experts.  Each lane reads 4 consecutive k of its row per 16-k chunk; the
// four MFMAs of a chunk use element i of those 4, so A and B see the same
// k permutation and the sum is over the same k set.

template <typename T>
__device__ __forceinline__ void load4_f32(const T* p, float out[4]);
template <>
__device__ __forceinline__ void load4_f32<float>(const float* p, float out[4]) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  out[0] = v.x;
  out[1] = v.y;
  out[2] = v.z;
  out[3] = v.w;
}
template <>
__device__ __forceinline__ void load4_f32<bf16_t>(const bf16_t* p, float out[4]) {
  u32x2 v = *reinterpret_cast<const u32x2*>(p);
  out[0] = __uint_as_float(v.x << 16);
  out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16);
  out[3] = __uint_as_float(v.y & 0xffff0000u);
}

template <typename XT, typename WT>
__global__ __launch_bounds__(256) void router_gemm_kernel(const XT* __restrict__ x,
                                                          const WT* __restrict__ wg,
                                                          float* __restrict__ part, int T,
                                                          int H, int N, int kchunk) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32;
  const int e0 = blockIdx.y * 256 + wave * 64;
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int kend = min(H, kbeg + kchunk);
  if (e0 >= N) return;  // whole wave beyond the experts (uniform)

  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 4;
  const XT* xrow[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    int t = min(t0 + mb * 16 + r16, T - 1);
    xrow[mb] = x + static_cast<int64_t>(t) * H + kq;
  }
  const WT* wrow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    int e = min(e0 + nb * 16 + r16, N - 1);
    wrow[nb] = wg + static_cast<int64_t>(e) * H + kq;
  }
  f32x4 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = kbeg; k < kend; k += 16) {
    float a[2][4], b[4][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) load4_f32<XT>(xrow[mb] + k, a[mb]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) load4_f32<WT>(wrow[nb] + k, b[nb]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] =
              __builtin_amdgcn_mfma_f32_16x16x4f32(a[mb][i], b[nb][i], acc[mb][nb], 0, 0, 0);
  }
  // D layout: lane holds rows 4*(lane/16)+i, column lane%16 of each block.
  float* out = part + static_cast<int64_t>(split) * T * N;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      int e = e0 + nb * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int t = t0 + mb * 16 + (lane >> 4) * 4 + i;
        if (t < T && e < N) out[static_cast<int64_t>(t) * N + e] = acc[mb][nb][i];
      }
    }
}

int router_splits(int T, int H, int N) {
  const int tiles = ((T + 31) / 32) * ((N + 255) / 256);
  if (tiles <= 0) return 1;
  int s = (1024 + tiles - 1) / tiles;
  const int smax = H / 64 < 32 ? H / 64 : 32;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_router_gemm(const void* x, int x_dtype, const void* wg, int wg_dtype,
                              float* part, int T, int H, int N, int splits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  int kchunk = (H + splits - 1) / splits;
  kchunk = (kchunk + 15) / 16 * 16;
  dim3 grid((T + 31) / 32, (N + 255) / 256, splits);
  if (x_dtype == MOE_BF16 && wg_dtype == MOE_F32)
    router_gemm_kernel<bf16_t, float><<<grid, 256, 0, st>>>(
        static_cast<const bf16_t*>(x), static_cast<const float*>(wg), part, T, H, N, kchunk);
  else if (x_dtype == MOE_BF16 && wg_dtype == MOE_BF16)
    router_gemm_kernel<bf16_t, bf16_t><<<grid, 256, 0, st>>>(
        static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(wg), part, T, H, N, kchunk);
  else if (x_dtype == MOE_F32 && wg_dtype == MOE_F32)
    router_gemm_kernel<float, float><<<grid, 256, 0, st>>>(
        static_cast<const float*>(x), static_cast<const float*>(wg), part, T, H, N, kchunk);
  else
    router_gemm_kernel<float, bf16_t><<<grid, 256, 0, st>>>(
        static_cast<const float*>(x), static_cast<const bf16_t*>(wg), part, T, H, N, kchunk);
  return hipGetLastError();
}

// ============================================================ route kernel
// One wavefront per token; lane L holds experts 4L..4L+3.  A group of gs
// experts spans gs/4 consecutive lanes.  Selection compares 64-bit keys
// (order-preserving fp32 bits << 32 | ~expert), so one max decides both the
// larger key and, on equal keys, the lower expert index.
__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;  // whole wave (uniform)
  const int N = p.N;
  const int e0 = lane * 4;
  const bool valid = e0 < N;  // N is a multiple of 4

  float l[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    for (int s = 0; s < p.splits; ++s) {
      f32x4 v = *reinterpret_cast<const f32x4*>(p.part + (static_cast<int64_t>(s) * p.T + t) * N + e0);
      l[0] += v.x;
      l[1] += v.y;
      l[2] += v.z;
      l[3] += v.w;
    }
    *reinterpret_cast<f32x4*>(p.logits + static_cast<int64_t>(t) * N + e0) =
        f32x4{l[0], l[1], l[2], l[3]};
  }

  // log-sum-exp over the N logits
  float m = valid ? fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])) : -INFINITY;
  m = wave_max_f32(m);
  float se = 0.f;
  if (valid) se = __expf(l[0] - m) + __expf(l[1] - m) + __expf(l[2] - m) + __expf(l[3] - m);
  se = wave_sum_f32(se);
  const float lse = m + __logf(se);

  // scores and selection keys
  float s[4];
  uint32_t ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (p.score_fn == MOE_SCORE_SIGMOID) {
      s[r] = sigmoid_score(l[r]);
    } else {
      s[r] = __expf(l[r] - m) / se;
    }
    float b = (valid && p.bias) ? p.bias[e0 + r] : 0.0f;
    float base = (p.score_fn == MOE_SCORE_SIGMOID) ? s[r] : l[r];
    float key = base + b;
    ok[r] = valid ? f32_order_key(key) : 0u;
  }

  // group limit
  if (p.n_groups > 1) {
    const int L = (N / p.n_groups) / 4;  // lanes per group
    const int q = lane / L;              // this lane's group (valid lanes)
    // local top-2 of the lane's 4 keys
    uint32_t a1 = 0, a2 = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t v = ok[r];
      if (v > a1) {
        a2 = a1;
        a1 = v;
      } else if (v > a2) {
        a2 = v;
      }
    }
    // merge the top-2 pairs of the group's L lanes
    uint32_t g1 = 0, g2 = 0;
    for (int i = 0; i < L; ++i) {
      int src = q * L + i;
      if (src > 63) src = 63;
      uint32_t b1 = __shfl(a1, src, kWave);
      uint32_t b2 = __shfl(a2, src, kWave);
      uint32_t hi = g1 > b1 ? g1 : b1;
      uint32_t lo1 = g1 > b1 ? b1 : g1;
      uint32_t lo2 = g2 > b2 ? g2 : b2;
      g1 = hi;
      g2 = lo1 > lo2 ? lo1 : lo2;
    }
    float gs_val = f32_from_order_key(g1);
    if (p.group_topn == 2) gs_val = gs_val + f32_from_order_key(g2);
    // rank of this lane's group among all groups (ties: lower group first)
    int rank = 0;
    for (int j = 0; j < p.n_groups; ++j) {
      float gj = __uint_as_float(
          __builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(gs_val)), j * L));
      rank += (gj > gs_val) || (gj == gs_val && j < q);
    }
    if (!valid || rank >= p.topk_groups) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ok[r] = 0u;
    }
  }

  // top-k by repeated wave-wide maximum
  uint64_t pk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    pk[r] = ok[r] ? ((static_cast<uint64_t>(ok[r]) << 32) | (0xffffffffu - static_cast<uint32_t>(e0 + r)))
                  : 0ull;
  int my_idx = 0;
  float my_s = 0.f;
  for (int j = 0; j < p.k; ++j) {
    uint64_t best = pk[0];
#pragma unroll
    for (int r = 1; r < 4; ++r) best = pk[r] > best ? pk[r] : best;
    best = wave_max_u64(best);
    const int ew = __builtin_amdgcn_readfirstlane(
        static_cast<int>(0xffffffffu - static_cast<uint32_t>(best)));
    float cand = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (e0 + r == ew) {
        cand = s[r];
        pk[r] = 0ull;
      }
    }
    const float sw = __uint_as_float(
        __builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(cand)), (ew >> 2) & 63));
    if (lane == j) {
      my_idx = ew;
      my_s = sw;
    }
  }
  // gates: sum of the chosen scores in slot order
  float ssum = 0.f;
  for (int j = 0; j < p.k; ++j)
    ssum += __uint_as_float(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(my_s)), j));
  if (lane < p.k) {
    float g = p.norm_topk ? my_s / ssum : my_s;
    const int64_t o = static_cast<int64_t>(t) * p.k + lane;
    p.topk_idx[o] = my_idx;
    p.topk_gate[o] = g * p.route_scale;
    p.topk_score[o] = my_s;
  }
  if (lane == 0 && p.token_lse) p.token_lse[t] = lse;
}

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  route_kernel<<<(p.T + 3) / 4, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe
