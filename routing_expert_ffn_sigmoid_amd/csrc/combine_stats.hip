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
// Rows of y_perm are read once and out is written once: both carry the
// non-temporal hint (V3 prefill combine 0.235 -> 0.195 ms, 6.0 TB/s).
constexpr int kCombineSlots = 8;  // row loads in flight per thread
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
  // slots in groups of kCombineSlots: row indices and gates first, then all
  // the group's row loads in flight together, then the sums in slot order
  for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
    int r[kCombineSlots];
    float g[kCombineSlots];
    u32x4 v[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      const int j = j0 + u;
      r[u] = j < k ? inv_row[static_cast<int64_t>(t) * k + j] : -1;
      g[u] = j < k ? gate[static_cast<int64_t>(t) * k + j] : 0.f;
    }
    // a dropped slot re-reads a kept row of the group (ignored below), so
    // the loads carry no condition and all go out together; rows are
    // token-uniform, so these branches do not diverge
    int any = -1;
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) any = r[u] >= 0 ? r[u] : any;
    if (any < 0) continue;
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u)
      v[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(y_perm + static_cast<int64_t>(r[u] >= 0 ? r[u] : any) * H + c));
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      if (r[u] < 0) continue;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(g[u], __uint_as_float(w[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(g[u], __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
      }
    }
  }
  u32x4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + static_cast<int64_t>(t) * H + c));
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
  for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
    int r[kCombineSlots];
    float g[kCombineSlots];
    f32x4 v[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      const int j = j0 + u;
      r[u] = j < k ? inv_row[static_cast<int64_t>(t) * k + j] : -1;
      g[u] = j < k ? gate[static_cast<int64_t>(t) * k + j] : 0.f;
    }
    // a dropped slot re-reads a kept row of the group (ignored below), so
    // the loads carry no condition and all go out together; rows are
    // token-uniform, so these branches do not diverge
    int any = -1;
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) any = r[u] >= 0 ? r[u] : any;
    if (any < 0) continue;
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u)
      v[u] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(y_perm + static_cast<int64_t>(r[u] >= 0 ? r[u] : any) * H + c));
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      if (r[u] < 0) continue;
      acc.x = fmaf(g[u], v[u].x, acc.x);
      acc.y = fmaf(g[u], v[u].y, acc.y);
      acc.z = fmaf(g[u], v[u].z, acc.z);
      acc.w = fmaf(g[u], v[u].w, acc.w);
    }
  }
  __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + static_cast<int64_t>(t) * H + c));
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
constexpr int kStatsLoads = 32;  // loads one thread keeps in flight in the statistics kernels

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
  auto score = [&](float l, int t) {
    return score_fn == MOE_SCORE_SIGMOID ? sigmoid_score(l) : __expf(l - lse[t]);
  };
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    // tokens in ascending order; kStatsLoads logit loads in flight at a time
    // (the launch is short and latency-bound: few rounds of memory latency)
    double acc = 0.0;
    int t = t0;
    for (; t + kStatsLoads <= t1; t += kStatsLoads) {
      float l[kStatsLoads];
#pragma unroll
      for (int u = 0; u < kStatsLoads; ++u) l[u] = logits[static_cast<int64_t>(t + u) * N + e];
#pragma unroll
      for (int u = 0; u < kStatsLoads; ++u) acc += static_cast<double>(score(l[u], t + u));
    }
    for (; t < t1; ++t) acc += static_cast<double>(score(logits[static_cast<int64_t>(t) * N + e], t));
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
  // column sums in block order, kStatsLoads partial loads in flight at a time
  double col = 0.0;
  if (e < N) {
    int b = 0;
    for (; b + kStatsLoads <= nblk; b += kStatsLoads) {
      double v[kStatsLoads];
#pragma unroll
      for (int u = 0; u < kStatsLoads; ++u) v[u] = part[static_cast<int64_t>(b + u) * (N + 2) + e];
#pragma unroll
      for (int u = 0; u < kStatsLoads; ++u) col += v[u];
    }
    for (; b < nblk; ++b) col += part[static_cast<int64_t>(b) * (N + 2) + e];
  }
  // lse sums: lane l of wave 0 takes blocks l, l + 64, ...
  double z = 0.0, z2 = 0.0;
  if (threadIdx.x < 64) {
    for (int b = threadIdx.x; b < nblk; b += 64) {
      z += part[static_cast<int64_t>(b) * (N + 2) + N];
      z2 += part[static_cast<int64_t>(b) * (N + 2) + N + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      z += __shfl_xor(z, o, kWave);
      z2 += __shfl_xor(z2, o, kWave);
    }
  }
  const double tot = block_sum_f64(col, sh);
  const double fe = (e < N && T > 0 && k > 0) ? static_cast<double>(counts[e]) / (static_cast<double>(k) * T) : 0.0;
  const double pe = (e < N && tot > 0.0) ? col / tot : 0.0;
  const double lb = block_sum_f64(fe * pe, sh);
  if (e < N) {
    if (f) f[e] = static_cast<float>(fe);
    if (P) P[e] = static_cast<float>(pe);
  }
  if (e == 0 && scalars) {
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

// ------------------------------------------------- sequence-wise stats
// The load statistics above, per sequence ("DeepSeek MoE：从v1到v3的演进"
// §DeepSeek-v3, sequence-wise balance loss).  Sequence q covers tokens
// [cu[q], cu[q+1]) (clamped to [0, T], so any input stays in bounds); it is
// cut into chunks of kSeqChunk tokens, each chunk summed by one workgroup
// (fp64, token order), the chunks of a sequence reduced in order.
constexpr int kSeqChunk = 64;

size_t seq_stats_ws_bytes(int T, int N, int n_seq) {
  const size_t chunks = static_cast<size_t>((T + kSeqChunk - 1) / kSeqChunk) + n_seq;
  const size_t a = ((static_cast<size_t>(n_seq) + 1) * sizeof(int32_t) + 255) & ~size_t(255);
  const size_t b = (chunks * N * sizeof(double) + 255) & ~size_t(255);
  return a + b + chunks * N * sizeof(int32_t) + 256;
}

__device__ __forceinline__ int clamp_tok(int v, int T) { return v < 0 ? 0 : (v > T ? T : v); }

// chunk_start[q] = chunks of the sequences before q; chunk_start[n_seq] = total
__global__ __launch_bounds__(256) void seq_chunks_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                         int T, int32_t* __restrict__ chunk_start) {
  __shared__ int sh[256];
  int running = 0;
  for (int q0 = 0; q0 < n_seq; q0 += 256) {
    const int q = q0 + threadIdx.x;
    int c = 0;
    if (q < n_seq) {
      const int a = clamp_tok(cu[q], T), b = clamp_tok(cu[q + 1], T);
      c = b > a ? (b - a + kSeqChunk - 1) / kSeqChunk : 0;
    }
    sh[threadIdx.x] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
      __syncthreads();
      sh[threadIdx.x] += v;
      __syncthreads();
    }
    if (q < n_seq) chunk_start[q] = running + sh[threadIdx.x] - c;
    running += sh[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) chunk_start[n_seq] = running;
}

__global__ __launch_bounds__(256) void seq_partial_kernel(
    const int32_t* __restrict__ cu, int n_seq, int T, int N, int k, int score_fn,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ logits, const float* __restrict__ lse, double* __restrict__ part,
    int32_t* __restrict__ pcnt) {
  __shared__ int hist[256];
  const int b = blockIdx.x;
  if (b >= chunk_start[n_seq]) return;  // uniform
  // the last sequence whose first chunk is <= b owns chunk b
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_start[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int a = clamp_tok(cu[lo], T), e_end = clamp_tok(cu[lo + 1], T);
  const int t0 = a + (b - chunk_start[lo]) * kSeqChunk;
  const int t1 = min(e_end, t0 + kSeqChunk);
  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < (t1 - t0) * k; i += blockDim.x) {
    const int e = topk_idx[static_cast<int64_t>(t0) * k + i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) atomicAdd(&hist[e], 1);  // integer
  }
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    double acc = 0.0;
    for (int t = t0; t < t1; ++t) {
      const float l = logits[static_cast<int64_t>(t) * N + e];
      const float sc = score_fn == MOE_SCORE_SIGMOID ? sigmoid_score(l) : __expf(l - lse[t]);
      acc += static_cast<double>(sc);
    }
    part[static_cast<int64_t>(b) * N + e] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) pcnt[static_cast<int64_t>(b) * N + e] = hist[e];
}

__global__ __launch_bounds__(256) void seq_final_kernel(
    const int32_t* __restrict__ cu, int n_seq, int T, int N, int k, int max_chunks,
    const int32_t* __restrict__ chunk_start, const double* __restrict__ part,
    const int32_t* __restrict__ pcnt, float* __restrict__ f_seq, float* __restrict__ P_seq,
    float* __restrict__ L_seq) {
  __shared__ double sh[4];
  const int q = blockIdx.x;
  const int e = threadIdx.x;
  const int Tq = max(0, clamp_tok(cu[q + 1], T) - clamp_tok(cu[q], T));
  double col = 0.0;
  long long cnt = 0;
  // chunk ids beyond the partials written (only for overlapping, invalid
  // boundaries) are not read
  const int c_end = min(chunk_start[q + 1], max_chunks);
  if (e < N)
    for (int c = chunk_start[q]; c < c_end; ++c) {
      col += part[static_cast<int64_t>(c) * N + e];
      cnt += pcnt[static_cast<int64_t>(c) * N + e];
    }
  const double tot = block_sum_f64(col, sh);
  const double fe = (e < N && Tq > 0 && k > 0) ? static_cast<double>(cnt) / (static_cast<double>(k) * Tq) : 0.0;
  const double pe = (e < N && tot > 0.0) ? col / tot : 0.0;
  const double lb = block_sum_f64(fe * pe, sh);
  if (e < N) {
    f_seq[static_cast<int64_t>(q) * N + e] = static_cast<float>(fe);
    P_seq[static_cast<int64_t>(q) * N + e] = static_cast<float>(pe);
  }
  if (e == 0) L_seq[q] = static_cast<float>(N * lb);
}

// mean of L_seq over the non-empty sequences (0 when there are none)
__global__ __launch_bounds__(256) void seq_mean_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                       int T, const float* __restrict__ L_seq,
                                                       float* __restrict__ L_mean) {
  __shared__ double sh[4];
  double sum = 0.0, cnt = 0.0;
  for (int q = threadIdx.x; q < n_seq; q += blockDim.x)
    if (clamp_tok(cu[q + 1], T) > clamp_tok(cu[q], T)) {
      sum += L_seq[q];
      cnt += 1.0;
    }
  sum = block_sum_f64(sum, sh);
  cnt = block_sum_f64(cnt, sh);
  if (threadIdx.x == 0) L_mean[0] = cnt > 0.0 ? static_cast<float>(sum / cnt) : 0.f;
}

hipError_t launch_seq_stats(const int32_t* cu, int n_seq, const int32_t* topk_idx,
                            const float* lse, const float* logits, int T, int N, int k,
                            int score_fn, float* f_seq, float* P_seq, float* L_seq,
                            float* L_mean, void* ws, hipStream_t st) {
  const int chunks = (T + kSeqChunk - 1) / kSeqChunk + n_seq;
  char* p = static_cast<char*>(ws);
  int32_t* chunk_start = reinterpret_cast<int32_t*>(p);
  p += ((static_cast<size_t>(n_seq) + 1) * sizeof(int32_t) + 255) & ~size_t(255);
  double* part = reinterpret_cast<double*>(p);
  p += (static_cast<size_t>(chunks) * N * sizeof(double) + 255) & ~size_t(255);
  int32_t* pcnt = reinterpret_cast<int32_t*>(p);
  if (n_seq > 0) {
    seq_chunks_kernel<<<1, 256, 0, st>>>(cu, n_seq, T, chunk_start);
    if (chunks > 0)
      seq_partial_kernel<<<chunks, 256, 0, st>>>(cu, n_seq, T, N, k, score_fn, chunk_start,
                                                 topk_idx, logits, lse, part, pcnt);
    seq_final_kernel<<<n_seq, 256, 0, st>>>(cu, n_seq, T, N, k, chunks, chunk_start, part, pcnt,
                                            f_seq, P_seq, L_seq);
  }
  if (L_mean) seq_mean_kernel<<<1, 256, 0, st>>>(cu, n_seq, T, L_seq, L_mean);
  return hipGetLastError();
}

// ------------------------------------------------- device-level stats
// "DeepSeek MoE：从v1到v3的演进" §DeepSeek-v1, device-level balance loss: the
// expert statistics summed over each of G groups of consecutive experts
// (one group per device); L_dev = G sum_g F_g P_g.
__global__ __launch_bounds__(256) void group_stats_kernel(const float* __restrict__ f,
                                                          const float* __restrict__ P, int N,
                                                          int G, float* __restrict__ F_g,
                                                          float* __restrict__ P_g,
                                                          float* __restrict__ L_dev) {
  __shared__ double sh[4];
  const int g = threadIdx.x;
  const int gs = N / G;
  double a = 0.0, b = 0.0;
  if (g < G)
    for (int e = g * gs; e < (g + 1) * gs; ++e) {
      a += f[e];
      b += P[e];
    }
  if (g < G) {
    if (F_g) F_g[g] = static_cast<float>(a);
    if (P_g) P_g[g] = static_cast<float>(b);
  }
  const double l = block_sum_f64(g < G ? a * b : 0.0, sh);
  if (g == 0 && L_dev) L_dev[0] = static_cast<float>(G * l);
}

hipError_t launch_group_stats(const float* f, const float* P, int N, int G, float* F_g,
                              float* P_g, float* L_dev, hipStream_t st) {
  group_stats_kernel<<<1, 256, 0, st>>>(f, P, N, G, F_g, P_g, L_dev);
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
