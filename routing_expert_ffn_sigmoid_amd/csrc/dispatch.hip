// dispatch.hip -- per-expert histogram, prefix sums, capacity drop and the
// token permutation, all deterministic (no order-dependent atomics).
//
// Sources: "DeepSeek MoE：从v1到v3的演进" §GShard (tokens are sent to the
// experts that own them; expert capacity; overflow passes through the
// residual) and §DeepSeek-v2 (device-level dropping: a device over the
// average load drops its lowest-scored tokens).
//
// Dropping order: a 64-bit key per assignment, higher is kept first:
// order key of the fp32 score (bits 63..32), then the lower token (bits
// 31..8, T < 2^24), then the lower expert (bits 7..0, N <= 256).  Keys are
// distinct, so "the C largest keys" is a set of exactly C assignments.
//
// Rows are laid out expert by expert, ascending token order inside an
// expert.  A token's rank inside its expert comes from LDS bit masks: wave w
// of a block ORs bit `lane` into mask[w][e] for each expert its token chose;
// OR is order-independent, and popcounts of the masks below a lane give the
// number of earlier tokens of the block that chose e.
#include "moe_internal.h"

namespace moe {

constexpr int kTokPerBlock = kDispatchTokPerBlock;  // 4 waves x 64 tokens

int dispatch_blocks(int T) { return (T + kTokPerBlock - 1) / kTokPerBlock; }

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t dispatch_ws_bytes(int T, int N, int k, const DropPolicy& d) {
  const size_t nb = dispatch_blocks(T);
  size_t b = 0;
  b += align256(nb * N * sizeof(int32_t));  // block_counts
  b += align256(nb * N * sizeof(int32_t));  // block_base
  b += align256(N * sizeof(int32_t));       // pre_off
  if (d.any()) {
    b += align256(static_cast<size_t>(T) * k * sizeof(uint64_t));
    b += align256(static_cast<size_t>(T) * k * sizeof(int32_t));
  }
  if (d.group_cap > 0) {
    b += align256(static_cast<size_t>(d.n_groups) * sizeof(uint64_t));
    b += align256(N * sizeof(int32_t));
  }
  return b;
}

DispatchWs dispatch_ws_carve(void* ws, int T, int N, int k, const DropPolicy& d) {
  const size_t nb = dispatch_blocks(T);
  char* p = static_cast<char*>(ws);
  DispatchWs w{};
  w.block_counts = reinterpret_cast<int32_t*>(p);
  p += align256(nb * N * sizeof(int32_t));
  w.block_base = reinterpret_cast<int32_t*>(p);
  p += align256(nb * N * sizeof(int32_t));
  w.pre_off = reinterpret_cast<int32_t*>(p);
  p += align256(N * sizeof(int32_t));
  if (d.any()) {
    w.cand_key = reinterpret_cast<uint64_t*>(p);
    p += align256(static_cast<size_t>(T) * k * sizeof(uint64_t));
    w.cand_slot = reinterpret_cast<int32_t*>(p);
    p += align256(static_cast<size_t>(T) * k * sizeof(int32_t));
  }
  if (d.group_cap > 0) {
    w.group_tau = reinterpret_cast<uint64_t*>(p);
    p += align256(static_cast<size_t>(d.n_groups) * sizeof(uint64_t));
    w.kept = reinterpret_cast<int32_t*>(p);
  }
  return w;
}

__device__ __forceinline__ uint64_t drop_key(float s, int t, int e) {
  return (static_cast<uint64_t>(f32_order_key(s)) << 32) |
         (static_cast<uint64_t>(0xFFFFFFu - static_cast<uint32_t>(t)) << 8) |
         static_cast<uint64_t>(0xFFu - static_cast<uint32_t>(e));
}

// Build mask[w][e] for this block's tokens.  masks: [4][N] in LDS.
__device__ __forceinline__ void build_masks(unsigned long long* masks,
                                            const int32_t* __restrict__ topk_idx, int T,
                                            int N, int k) {
  for (int i = threadIdx.x; i < 4 * N; i += blockDim.x) masks[i] = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[static_cast<int64_t>(t) * k + j];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N))
        atomicOr(&masks[w * N + e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ topk_idx,
                                                             int T, int N, int k,
                                                             int32_t* __restrict__ block_counts) {
  extern __shared__ unsigned long long masks[];
  build_masks(masks, topk_idx, T, N, k);
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) c += __popcll(masks[w * N + e]);
    block_counts[static_cast<int64_t>(blockIdx.x) * N + e] = c;
  }
}

// Inclusive scan of one value per thread over a 256-thread block.
__device__ __forceinline__ int block_scan_incl(int v, int* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int a = threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
    __syncthreads();
    sh[threadIdx.x] += a;
    __syncthreads();
  }
  int r = sh[threadIdx.x];
  __syncthreads();
  return r;
}

// One block of 256 threads; thread e owns expert e (N <= 256).
__global__ __launch_bounds__(256) void dispatch_scan_kernel(const int32_t* __restrict__ block_counts,
                                                            int nb, int N, int capacity,
                                                            int32_t* __restrict__ block_base,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ pre_off,
                                                            int32_t* __restrict__ n_dropped) {
  __shared__ int sh[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N) {
    // eight blocks' counts are loaded before they are added, so their
    // loads overlap instead of one latency per block
    for (int b0 = 0; b0 < nb; b0 += 8) {
      int c8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c8[j] = b0 + j < nb ? block_counts[static_cast<int64_t>(b0 + j) * N + e] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b0 + j < nb) block_base[static_cast<int64_t>(b0 + j) * N + e] = run;
        run += c8[j];
      }
    }
  }
  const int c_e = e < N ? run : 0;
  const int kept = (capacity > 0 && c_e > capacity) ? capacity : c_e;
  const int incl_c = block_scan_incl(c_e, sh);
  const int incl_k = block_scan_incl(kept, sh);
  const int drop_tot = block_scan_incl(c_e - kept, sh);
  if (e < N) {
    counts[e] = c_e;
    pre_off[e] = incl_c - c_e;
    offsets[e] = incl_k - kept;
  }
  if (e == N - 1) {
    offsets[N] = incl_k;
    if (n_dropped) {
      n_dropped[0] = drop_tot;
      n_dropped[1] = 0;
    }
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_score, int T, int N,
    int k, int capacity, bool all_candidates, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pre_off, int32_t* __restrict__ row_token,
    int32_t* __restrict__ inv_row, uint64_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_slot) {
  extern __shared__ unsigned long long masks[];
  build_masks(masks, topk_idx, T, N, k);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int64_t slot = static_cast<int64_t>(t) * k + j;
    const int e = topk_idx[slot];
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(N)) {  // outside the contract
      inv_row[slot] = -1;
      continue;
    }
    int rank = block_base[static_cast<int64_t>(blockIdx.x) * N + e];
    for (int w2 = 0; w2 < w; ++w2) rank += __popcll(masks[w2 * N + e]);
    rank += __popcll(masks[w * N + e] & below);
    if (!all_candidates && (capacity == 0 || counts[e] <= capacity)) {
      const int row = offsets[e] + rank;
      inv_row[slot] = row;
      row_token[row] = t;
    } else {
      // candidates of an expert sit in token order at pre_off[e] + rank
      const int pos = pre_off[e] + rank;
      cand_key[pos] = drop_key(topk_score[slot], t, e);
      cand_slot[pos] = static_cast<int32_t>(slot);
    }
  }
}

// The `need`-th largest of n distinct 64-bit keys, by an 8-bit radix select
// over the whole workgroup (result in every thread).
constexpr int kCapThreads = 1024;

__device__ uint64_t radix_select_key(const uint64_t* __restrict__ keys, int n, int need) {
  __shared__ int hist[256];
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_need;
  __shared__ int sh_done;
  if (threadIdx.x == 0) {
    sh_prefix = 0ull;
    sh_need = need;
    sh_done = 0;
  }
  for (int d = 7; d >= 0; --d) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const uint64_t prefix = sh_prefix;
    const int hs = 8 * (d + 1);
    const int lane = threadIdx.x & 63;
    // batches of 8 keys per thread, loaded before they are counted, so 8
    // loads are in flight instead of one (uniform trip count)
    constexpr int kB = 8;
    for (int i0 = 0; i0 < n; i0 += kB * static_cast<int>(blockDim.x)) {
      uint64_t kb[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = i0 + j * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x);
        kb[j] = i < n ? keys[i] : 0ull;
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = i0 + j * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x);
        const uint64_t key = kb[j];
        const bool match = i < n && ((d == 7) || ((key >> hs) == (prefix >> hs)));
        const int dg = static_cast<int>((key >> (8 * d)) & 255);
        // The top digits of one expert's keys (its scores' exponent) fall
        // into one or two bins: lanes sharing the first pending lane's digit
        // add their count with one atomic, up to four rounds, the rest one
        // each.
        uint64_t act = __ballot(match);
        for (int it = 0; it < 4 && act != 0ull; ++it) {
          const int lead = __ffsll(static_cast<unsigned long long>(act)) - 1;
          const int ld = __shfl(dg, lead);
          const uint64_t same = __ballot(match && dg == ld) & act;
          if (lane == lead) atomicAdd(&hist[ld], __popcll(same));
          act &= ~same;
        }
        if ((act >> lane) & 1ull) atomicAdd(&hist[dg], 1);
      }
    }
    __syncthreads();
    // The digit whose bin holds the left-th largest matching key: wave 0
    // takes the bins in descending order, four per lane (lane l: 255 - 4l
    // down to 252 - 4l), forms the running count over lanes, and the first
    // lane whose running count reaches `left` finds the digit in its bins.
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      const int left = sh_need;  // >= 1 and at most the matching keys
      int h[4];
      int own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[255 - 4 * l - q];
        own += h[q];
      }
      int incl = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (l >= o) incl += t;
      }
      const uint64_t reach = __ballot(incl >= left);
      if (l == __ffsll(static_cast<unsigned long long>(reach)) - 1) {
        int cum = incl - own;
        int digit = 252 - 4 * l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + h[q] >= left) {
            digit = 255 - 4 * l - q;
            break;
          }
          cum += h[q];
        }
        sh_need = left - cum;
        sh_prefix = prefix | (static_cast<uint64_t>(digit) << (8 * d));
        // every key of the bin is needed: the prefix with zero lower digits
        // is the threshold (keys are distinct, those below the bin are not
        // kept)
        sh_done = (left - cum == hist[digit]) ? 1 : 0;
      }
    }
    __syncthreads();
    if (sh_done) break;  // uniform
  }
  const uint64_t tau = sh_prefix;
  __syncthreads();
  return tau;
}

// Rows for one expert's candidates (token order): keys >= tau are kept and
// numbered from base_row in token order, the others are dropped.
__device__ void assign_kept_rows(const uint64_t* __restrict__ keys,
                                 const int32_t* __restrict__ slots, int c, uint64_t tau,
                                 int base_row, int k, int32_t* __restrict__ row_token,
                                 int32_t* __restrict__ inv_row) {
  constexpr int kWaves = kCapThreads / 64;
  __shared__ int wave_kept[kWaves];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int running = 0;
  // the next chunk's key and slot are loaded while this chunk is ranked
  uint64_t key_n = threadIdx.x < static_cast<unsigned>(c) ? keys[threadIdx.x] : 0ull;
  int slot_n = threadIdx.x < static_cast<unsigned>(c) ? slots[threadIdx.x] : 0;
  for (int c0 = 0; c0 < c; c0 += kCapThreads) {
    const int i = c0 + threadIdx.x;
    const uint64_t key = key_n;
    const int slot = slot_n;
    const int inext = i + kCapThreads;
    if (inext < c) {
      key_n = keys[inext];
      slot_n = slots[inext];
    }
    const bool keep = i < c && key >= tau;
    // rank inside the chunk: kept lanes of earlier waves, then of lower
    // lanes of this wave (ballot and popcount)
    const uint64_t m = __ballot(keep);
    if (lane == 0) wave_kept[w] = __popcll(m);
    __syncthreads();
    int before = 0, chunk_total = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const int x = wave_kept[v];
      before += v < w ? x : 0;
      chunk_total += x;
    }
    const int excl = before + __popcll(m & ((1ull << lane) - 1ull));
    if (i < c) {
      if (keep) {
        const int row = base_row + running + excl;
        inv_row[slot] = row;
        row_token[row] = slot / k;
      } else {
        inv_row[slot] = -1;
      }
    }
    running += chunk_total;
    __syncthreads();  // wave_kept is rewritten by the next chunk
  }
}

// Per-expert capacity: one workgroup per expert over capacity keeps its
// `capacity` largest keys.
__global__ __launch_bounds__(kCapThreads) void capacity_select_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pre_off, const uint64_t* __restrict__ cand_key,
    const int32_t* __restrict__ cand_slot, int k, int capacity,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row) {
  const int e = blockIdx.x;
  const int c = counts[e];
  if (c <= capacity) return;  // uniform
  const uint64_t* keys = cand_key + pre_off[e];
  const uint64_t tau = radix_select_key(keys, c, capacity);
  assign_kept_rows(keys, cand_slot + pre_off[e], c, tau, offsets[e], k, row_token, inv_row);
}

// Device-level dropping, step 1: one workgroup per group of gs experts.  The
// group's candidates are contiguous (experts in order); a group over its cap
// finds the cap-th largest key, and every expert of the group counts its
// candidates at or above it.
__global__ __launch_bounds__(kCapThreads) void group_select_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ pre_off,
    const uint64_t* __restrict__ cand_key, int gs, int group_cap,
    uint64_t* __restrict__ group_tau, int32_t* __restrict__ kept) {
  __shared__ int kc[256];
  const int g = blockIdx.x;
  const int e0 = g * gs;
  const int begin = pre_off[e0];
  const int end = pre_off[e0 + gs - 1] + counts[e0 + gs - 1];
  const int n = end - begin;
  uint64_t tau = 0ull;
  if (n > group_cap) tau = radix_select_key(cand_key + begin, n, group_cap);  // uniform branch
  for (int i = threadIdx.x; i < gs; i += blockDim.x) kc[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t key = cand_key[begin + i];
    if (key >= tau) atomicAdd(&kc[0xFF - static_cast<int>(key & 0xFF) - e0], 1);  // integer: order-free
  }
  __syncthreads();
  for (int i = threadIdx.x; i < gs; i += blockDim.x) kept[e0 + i] = kc[i];
  if (threadIdx.x == 0) group_tau[g] = tau;
}

// Step 2 (one workgroup of 256, thread e = expert e): row offsets from the
// kept counts, and the dropped-assignment count.
__global__ __launch_bounds__(256) void kept_scan_kernel(const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ kept, int N,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ n_dropped) {
  __shared__ int sh[256];
  const int e = threadIdx.x;
  const int ke = e < N ? kept[e] : 0;
  const int de = e < N ? counts[e] - ke : 0;
  const int incl = block_scan_incl(ke, sh);
  const int drop_tot = block_scan_incl(de, sh);
  if (e < N) offsets[e] = incl - ke;
  if (e == N - 1) {
    offsets[N] = incl;
    if (n_dropped) {
      n_dropped[0] = drop_tot;
      n_dropped[1] = 0;
    }
  }
}

// Step 3: one workgroup per expert numbers its kept candidates.
__global__ __launch_bounds__(kCapThreads) void group_assign_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pre_off, const uint64_t* __restrict__ cand_key,
    const int32_t* __restrict__ cand_slot, const uint64_t* __restrict__ group_tau, int gs, int k,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row) {
  const int e = blockIdx.x;
  const int c = counts[e];
  if (c == 0) return;  // uniform
  assign_kept_rows(cand_key + pre_off[e], cand_slot + pre_off[e], c, group_tau[e / gs],
                   offsets[e], k, row_token, inv_row);
}

__global__ __launch_bounds__(256) void count_all_dropped_kernel(const int32_t* __restrict__ inv_row,
                                                                int T, int k,
                                                                int32_t* __restrict__ n_dropped) {
  __shared__ int sh[4];
  const int t = blockIdx.x * 256 + threadIdx.x;
  int flag = 0;
  if (t < T) {
    flag = 1;
    for (int j = 0; j < k; ++j) flag &= (inv_row[static_cast<int64_t>(t) * k + j] < 0);
  }
  int s = flag;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tot = sh[0] + sh[1] + sh[2] + sh[3];
    if (tot) atomicAdd(&n_dropped[1], tot);  // integer sum: order-independent
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_zero_block_counts(const DispatchWs& w, int T, int N, hipStream_t st) {
  const int nb = dispatch_blocks(T);
  if (nb > 0) fill_i32_kernel<<<(nb * N + 255) / 256, 256, 0, st>>>(w.block_counts, nb * N, 0);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* topk_idx, const float* topk_score, int T, int N,
                           int k, const DropPolicy& d, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, int32_t* inv_row, int32_t* n_dropped,
                           const DispatchWs& w, hipStream_t st, bool counts_ready) {
  const int nb = dispatch_blocks(T);
  const size_t lds = 4 * N * sizeof(unsigned long long);
  const bool grouped = d.group_cap > 0;
  if (counts_ready) {
    // per-block counts were added up by the route kernel
  } else if (nb > 0 && k > 0) {
    dispatch_count_kernel<<<nb, 256, lds, st>>>(topk_idx, T, N, k, w.block_counts);
  } else if (nb > 0) {
    fill_i32_kernel<<<(nb * N + 255) / 256, 256, 0, st>>>(w.block_counts, nb * N, 0);
  }
  // with group dropping the offsets and drop counts written here are
  // provisional (no drops); kept_scan_kernel overwrites them
  dispatch_scan_kernel<<<1, 256, 0, st>>>(w.block_counts, nb, N, grouped ? 0 : d.capacity,
                                          w.block_base, counts, offsets, w.pre_off, n_dropped);
  if (nb > 0 && k > 0) {
    dispatch_scatter_kernel<<<nb, 256, lds, st>>>(
        topk_idx, topk_score, T, N, k, grouped ? 0 : d.capacity, grouped, w.block_base, counts,
        offsets, w.pre_off, row_token, inv_row, w.cand_key, w.cand_slot);
    if (grouped) {
      const int gs = N / d.n_groups;
      group_select_kernel<<<d.n_groups, kCapThreads, 0, st>>>(counts, w.pre_off, w.cand_key, gs,
                                                               d.group_cap, w.group_tau, w.kept);
      kept_scan_kernel<<<1, 256, 0, st>>>(counts, w.kept, N, offsets, n_dropped);
      group_assign_kernel<<<N, kCapThreads, 0, st>>>(counts, offsets, w.pre_off, w.cand_key,
                                                     w.cand_slot, w.group_tau, gs, k, row_token,
                                                     inv_row);
    } else if (d.capacity > 0) {
      capacity_select_kernel<<<N, kCapThreads, 0, st>>>(counts, offsets, w.pre_off, w.cand_key,
                                                        w.cand_slot, k, d.capacity, row_token,
                                                        inv_row);
    }
    if (d.any() && n_dropped)
      count_all_dropped_kernel<<<(T + 255) / 256, 256, 0, st>>>(inv_row, T, k, n_dropped);
  }
  return hipGetLastError();
}

// x_perm[r] = x[row_token[r]] for r < offsets[N]; one wave per row, 16-byte
// vectors.
__global__ __launch_bounds__(256) void permute_kernel(const char* __restrict__ x,
                                                      int64_t row_bytes,
                                                      const int32_t* __restrict__ row_token,
                                                      const int32_t* __restrict__ offsets,
                                                      int N, char* __restrict__ x_perm) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= offsets[N]) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<int64_t>(row_token[r]) * row_bytes);
  u32x4* dst = reinterpret_cast<u32x4*>(x_perm + static_cast<int64_t>(r) * row_bytes);
  const int nv = static_cast<int>(row_bytes / 16);
  for (int i = lane; i < nv; i += 64) dst[i] = src[i];
}

hipError_t launch_permute(const void* x, int elem_bytes, int H, const int32_t* row_token,
                          const int32_t* offsets, int N, int max_rows, void* x_perm,
                          hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  permute_kernel<<<(max_rows + 3) / 4, 256, 0, st>>>(
      static_cast<const char*>(x), static_cast<int64_t>(H) * elem_bytes, row_token, offsets, N,
      static_cast<char*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
