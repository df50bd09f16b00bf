// combine_stats.hip -- gate-weighted combine, load statistics and the
// auxiliary-loss-free bias update.
//
// Sources: "从零构建DeepSeekMoE…" §2.2 (output = shared experts + routed
// experts); "DeepSeek MoE：从v1到v3的演进" §GShard (a dropped token adds
// nothing here and keeps its residual outside the layer), §ST-MoE (f_i,
// P_i, L_B = N sum f_i P_i, z-loss) and §DeepSeek-v3 (bias update by the
// sign of the load error).
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- combine
// out[t] = y_shared[t] + sum_j gate[t,j] * y_perm[inv_row[t,j]], fp32 sum in
// slot order, one rounding.  One thread per 8 (bf16) or 4 (fp32) elements.
__global__ __launch_bounds__(256) void combine_bf16_kernel(const bf16_t* __restrict__ y_perm,
                                                           const int32_t* __restrict__ inv_row,
                                                           const float* __restrict__ gate,
                                                           const bf16_t* __restrict__ y_sh,
                                                           bf16_t* __restrict__ out, int T, int H,
                                                           int k) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8];
  if (y_sh) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(y_sh + static_cast<int64_t>(t) * H + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __uint_as_float(w[i] << 16);
      acc[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int r = inv_row[static_cast<int64_t>(t) * k + j];
    if (r < 0) continue;
    const float gj = gate[static_cast<int64_t>(t) * k + j];
    const u32x4 v = *reinterpret_cast<const u32x4*>(y_perm + static_cast<int64_t>(r) * H + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(gj, __uint_as_float(w[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(gj, __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  }
  u32x4 o;
  o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
  o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
  o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
  o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
  *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(t) * H + c) = o;
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ y_perm,
                                                          const int32_t* __restrict__ inv_row,
                                                          const float* __restrict__ gate,
                                                          const float* __restrict__ y_sh,
                                                          float* __restrict__ out, int T, int H,
                                                          int k) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  f32x4 acc = y_sh ? *reinterpret_cast<const f32x4*>(y_sh + static_cast<int64_t>(t) * H + c)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int r = inv_row[static_cast<int64_t>(t) * k + j];
    if (r < 0) continue;
    const float gj = gate[static_cast<int64_t>(t) * k + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(y_perm + static_cast<int64_t>(r) * H + c);
    acc.x = fmaf(gj, v.x, acc.x);
    acc.y = fmaf(gj, v.y, acc.y);
    acc.z = fmaf(gj, v.z, acc.z);
    acc.w = fmaf(gj, v.w, acc.w);
  }
  *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(t) * H + c) = acc;
}

hipError_t launch_combine(const void* y_perm, const int32_t* inv_row, const float* gate,
                          const void* y_shared, void* out, int T, int H, int k, int act_dtype,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (act_dtype == MOE_BF16) {
    dim3 grid((H / 8 + 255) / 256, T);
    combine_bf16_kernel<<<grid, 256, 0, st>>>(
        static_cast<const bf16_t*>(y_perm), inv_row, gate,
        static_cast<const bf16_t*>(y_shared), static_cast<bf16_t*>(out), T, H, k);
  } else {
    dim3 grid((H / 4 + 255) / 256, T);
    combine_f32_kernel<<<grid, 256, 0, st>>>(static_cast<const float*>(y_perm), inv_row, gate,
                                             static_cast<const float*>(y_shared),
                                             static_cast<float*>(out), T, H, k);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- stats
constexpr int kStatsMaxBlocks = 256;

int stats_blocks(int T) {
  int b = (T + 63) / 64;
  if (b > kStatsMaxBlocks) b = kStatsMaxBlocks;
  if (b < 1) b = 1;
  return b;
}

size_t stats_ws_bytes(int T, int N) {
  return static_cast<size_t>(stats_blocks(T)) * (N + 2) * sizeof(double);
}

// Block b sums tokens [b*chunk, (b+1)*chunk): thread e < N accumulates the
// scores of expert e; wave 0 also sums lse and lse^2.  part: [blocks][N+2].
__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ lse, int T,
                                                            int N, int score_fn, int chunk,
                                                            double* __restrict__ part) {
  const int b = blockIdx.x;
  const int t0 = b * chunk;
  const int t1 = min(T, t0 + chunk);
  double* out = part + static_cast<int64_t>(b) * (N + 2);
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    double acc = 0.0;
    for (int t = t0; t < t1; ++t) {
      const float l = logits[static_cast<int64_t>(t) * N + e];
      const float s = score_fn == MOE_SCORE_SIGMOID ? sigmoid_score(l) : __expf(l - lse[t]);
      acc += static_cast<double>(s);
    }
    out[e] = acc;
  }
  if (threadIdx.x < 64) {
    double z = 0.0, z2 = 0.0;
    for (int t = t0 + threadIdx.x; t < t1; t += 64) {
      const double v = lse[t];
      z += v;
      z2 += v * v;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      z += __shfl_xor(z, o, kWave);
      z2 += __shfl_xor(z2, o, kWave);
    }
    if (threadIdx.x == 0) {
      out[N] = z;
      out[N + 1] = z2;
    }
  }
}

__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void stats_final_kernel(const double* __restrict__ part,
                                                          int nblk, const int32_t* __restrict__ counts,
                                                          int T, int N, int k, float* __restrict__ f,
                                                          float* __restrict__ P,
                                                          float* __restrict__ scalars) {
  __shared__ double sh[4];
  const int e = threadIdx.x;
  double col = 0.0;
  if (e < N)
    for (int b = 0; b < nblk; ++b) col += part[static_cast<int64_t>(b) * (N + 2) + e];
  const double tot = block_sum_f64(col, sh);
  const double fe = (e < N && T > 0 && k > 0) ? static_cast<double>(counts[e]) / (static_cast<double>(k) * T) : 0.0;
  const double pe = (e < N && tot > 0.0) ? col / tot : 0.0;
  const double lb = block_sum_f64(fe * pe, sh);
  if (e < N) {
    if (f) f[e] = static_cast<float>(fe);
    if (P) P[e] = static_cast<float>(pe);
  }
  if (e == 0 && scalars) {
    double z = 0.0, z2 = 0.0;
    for (int b = 0; b < nblk; ++b) {
      z += part[static_cast<int64_t>(b) * (N + 2) + N];
      z2 += part[static_cast<int64_t>(b) * (N + 2) + N + 1];
    }
    scalars[0] = static_cast<float>(N * lb);
    scalars[1] = T > 0 ? static_cast<float>(z / T) : 0.f;
    scalars[2] = T > 0 ? static_cast<float>(z2 / T) : 0.f;
  }
}

hipError_t launch_stats(const int32_t* counts, const float* lse, const float* logits, int T,
                        int N, int k, int score_fn, float* f, float* P, float* scalars, void* ws,
                        hipStream_t st) {
  const int nblk = stats_blocks(T);
  const int chunk = T > 0 ? (T + nblk - 1) / nblk : 0;
  double* part = static_cast<double*>(ws);
  stats_partial_kernel<<<nblk, 256, 0, st>>>(logits, lse, T, N, score_fn, chunk, part);
  stats_final_kernel<<<1, 256, 0, st>>>(part, nblk, counts, T, N, k, f, P, scalars);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bias
// b_e += u * sign(mean(c) - c_e); the sign is taken exactly in integers as
// sign(sum(c) - N c_e).
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          float* __restrict__ bias, int N,
                                                          float u) {
  __shared__ long long sh[4];
  long long c = threadIdx.x < N ? counts[threadIdx.x] : 0;
  long long s = c;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  const long long tot = sh[0] + sh[1] + sh[2] + sh[3];
  if (threadIdx.x < N) {
    const long long d = tot - static_cast<long long>(N) * c;
    const float step = d > 0 ? u : (d < 0 ? -u : 0.0f);
    bias[threadIdx.x] = bias[threadIdx.x] + step;
  }
}

hipError_t launch_bias_update(const int32_t* counts, float* bias, int N, float u,
                              hipStream_t st) {
  bias_update_kernel<<<1, 256, 0, st>>>(counts, bias, N, u);
  return hipGetLastError();
}

}  // namespace moe
