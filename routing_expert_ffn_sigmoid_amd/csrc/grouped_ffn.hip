// grouped_ffn.hip -- grouped SwiGLU expert GEMMs over variable-size row
// segments (the routed experts) plus extra groups (the shared expert), in one
// persistent launch per phase.
//
// Sources: "DeepSeek MoE：从v1到v3的演进" §DeepSeek-v1 (fine-grained routed
// experts; isolated shared experts every token passes through);
// "从零构建DeepSeekMoE…" §2.2 (layer output = shared experts + routed
// experts).  The expert form is SwiGLU: h = silu(Wg a) * (Wu a), y = Wd h.
//
// bf16 path (gfx950 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//  * workgroup = 4 waves; a wave computes all BM rows of the tile times 64
//    weight rows (4 blocks of 16).  In the gate/up phase a wave's blocks are
//    gate columns c..c+31 and the up columns c..c+31, so the SwiGLU product
//    is formed in registers and h is rounded to bf16 once.
//  * activations (shared by the 4 waves) are staged through LDS, double
//    buffered, 16-byte chunks XOR-swizzled by row so MFMA fragment reads hit
//    distinct banks; the weights (used by one wave only) stream from global
//    memory straight into registers, PF steps ahead.
//  * M-blocks of 16 rows past the end of a segment are skipped, so a
//    segment's last tile costs what its rows need (to 16 rows).
//  * persistent grid: each XCD (workgroup id mod 8) walks a contiguous eighth
//    of the tile list, so tiles that share an expert's weights (consecutive
//    m-tiles of one n-tile) and its activations (consecutive n-tiles) meet in
//    that XCD's L2.
#include "moe_internal.h"

namespace moe {

constexpr int kBK = 64;        // k per pipeline step (8 chunks of 16 bytes)
constexpr int kThreads = 256;  // 4 waves
constexpr int kMaxSegs = 1024; // flat segments over all groups per launch

struct FfnLaunch {
  FfnGroup g[2];
  int ngroups;
  int nt[2];  // n-tiles per group
};

__device__ __forceinline__ int seg_begin(const FfnGroup& g, int s) {
  return g.seg_off ? g.seg_off[s] : 0;
}
__device__ __forceinline__ int seg_end(const FfnGroup& g, int s) {
  return g.seg_off ? g.seg_off[s + 1] : g.rows;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Exclusive prefix of `cnt` tiles per flat segment into tstart[0..n].
template <int BM>
__device__ void build_tile_starts(const FfnLaunch& a, int nsegT, int* tstart, int* tmp) {
  const int tid = threadIdx.x;
  // each thread owns 4 consecutive segments
  int local[4];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid * 4 + j;
    int c = 0;
    if (i < nsegT) {
      const int grp = (a.ngroups > 1 && i >= a.g[0].nseg) ? 1 : 0;
      const FfnGroup& g = grp ? a.g[1] : a.g[0];
      const int s = grp ? i - a.g[0].nseg : i;
      const int rows = seg_end(g, s) - seg_begin(g, s);
      c = ((rows + BM - 1) / BM) * (grp ? a.nt[1] : a.nt[0]);
    }
    sum += c;
    local[j] = sum;
  }
  tmp[tid] = sum;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  const int base = tmp[tid] - sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid * 4 + j;
    if (i < nsegT) tstart[i + 1] = base + local[j];
  }
  if (tid == 0) tstart[0] = 0;
  __syncthreads();
}

template <int MB, int PF, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void ffn_bf16_kernel(FfnLaunch a) {
  constexpr int BM = 16 * MB;
  constexpr int APASS = (BM * 8 + kThreads - 1) / kThreads;  // 16-byte A loads per thread
  constexpr int NSLOT = PF + 1;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * kBK];
  __shared__ int tstart[kMaxSegs + 1];
  __shared__ int tmp[kThreads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nsegT = a.g[0].nseg + (a.ngroups > 1 ? a.g[1].nseg : 0);
  build_tile_starts<BM>(a, nsegT, tstart, tmp);
  const int total = tstart[nsegT];

  const int nxcd = 8;
  const int per = gridDim.x / nxcd;
  const int xcd = blockIdx.x % nxcd;
  const int slot = blockIdx.x / nxcd;
  const int lo = static_cast<int>((static_cast<int64_t>(total) * xcd) / nxcd);
  const int hi = static_cast<int>((static_cast<int64_t>(total) * (xcd + 1)) / nxcd);

  for (int L = lo + slot; L < hi; L += per) {
    // ---- decode the tile
    int i0 = 0, i1 = nsegT;
    while (i1 - i0 > 1) {
      const int mid = (i0 + i1) >> 1;
      if (tstart[mid] <= L) i0 = mid;
      else i1 = mid;
    }
    const int grp = (a.ngroups > 1 && i0 >= a.g[0].nseg) ? 1 : 0;
    const FfnGroup& g = grp ? a.g[1] : a.g[0];
    const int s = grp ? i0 - a.g[0].nseg : i0;
    const int r0 = seg_begin(g, s);
    const int rows = seg_end(g, s) - r0;
    const int mtc = (rows + BM - 1) / BM;
    const int local = L - tstart[i0];
    const int nt = local / mtc;
    const int mt = local - nt * mtc;
    const int mrow0 = r0 + mt * BM;
    const int mv = min(BM, rows - mt * BM);
    const int nmb = (mv + 15) >> 4;
    const int K = g.K;
    const int nk = K / kBK;

    // ---- activation loader: thread -> (row, 16-byte chunk)
    const bf16_t* A = static_cast<const bf16_t*>(g.A);
    const bf16_t* aptr[APASS];
    bool aval[APASS];
    int aoff[APASS];
#pragma unroll
    for (int p = 0; p < APASS; ++p) {
      const int row = (tid >> 3) + 32 * p;
      const int ch = tid & 7;
      aval[p] = (row < BM) && (row < mv);
      int prow = mrow0 + (row < mv ? row : 0);
      if (g.row_index) prow = g.row_index[prow];
      aptr[p] = A + static_cast<int64_t>(prow) * g.lda + ch * 8;
      aoff[p] = (row < BM ? row : 0) * kBK + ((ch ^ ((row >> 1) & 7)) * 8);
    }

    // ---- weight rows of this wave (4 blocks of 16)
    const bf16_t* W = static_cast<const bf16_t*>(g.W) + static_cast<int64_t>(s) * g.w_stride;
    const bf16_t* bptr[4];
    int col[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      int c, brow;
      if (SWIGLU) {
        c = nt * 128 + wave * 32 + (nb & 1) * 16 + (lane & 15);
        const int cc = c < g.n_out ? c : 0;
        brow = (nb < 2) ? cc : g.up_off + cc;
      } else {
        c = nt * 256 + wave * 64 + nb * 16 + (lane & 15);
        brow = c < g.n_out ? c : 0;
      }
      col[nb] = c;
      bptr[nb] = W + static_cast<int64_t>(brow) * K + (lane >> 4) * 8;
    }

    f32x4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 bbuf[NSLOT][2][4];
    u32x4 areg[APASS];

    auto load_b = [&](int step, u32x4 (&dst)[2][4]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          dst[ks][nb] = *reinterpret_cast<const u32x4*>(bptr[nb] + step * kBK + ks * 32);
    };
    auto load_a = [&](int step) {
#pragma unroll
      for (int p = 0; p < APASS; ++p)
        if (aval[p]) areg[p] = *reinterpret_cast<const u32x4*>(aptr[p] + step * kBK);
    };
    auto store_a = [&](int buf) {
#pragma unroll
      for (int p = 0; p < APASS; ++p)
        if (aval[p]) *reinterpret_cast<u32x4*>(&As[buf][aoff[p]]) = areg[p];
    };
    auto compute = [&](int buf, const u32x4 (&b)[2][4]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (mb < nmb) {
            const int row = mb * 16 + (lane & 15);
            const int ch = ks * 4 + (lane >> 4);
            const u32x4 av =
                *reinterpret_cast<const u32x4*>(&As[buf][row * kBK + ((ch ^ ((row >> 1) & 7)) * 8)]);
            const bf16x8 af = as_bf16x8(av);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, as_bf16x8(b[ks][nb]),
                                                                    acc[mb][nb], 0, 0, 0);
          }
        }
      }
    };

    // ---- prologue
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (u < nk) load_b(u, bbuf[u]);
    load_a(0);
    store_a(0);
    __syncthreads();

    // ---- main loop, unrolled by NSLOT so the register ring is static
    for (int s0 = 0; s0 < nk; s0 += NSLOT) {
#pragma unroll
      for (int u = 0; u < NSLOT; ++u) {
        const int st = s0 + u;
        if (st < nk) {
          if (st + PF < nk) load_b(st + PF, bbuf[(u + PF) % NSLOT]);
          if (st + 1 < nk) load_a(st + 1);
          compute(st & 1, bbuf[u]);
          if (st + 1 < nk) store_a((st + 1) & 1);
          __syncthreads();
        }
      }
    }

    // ---- epilogue: D element i of a lane is row 4*(lane/16)+i, col lane%16
    bf16_t* Out = static_cast<bf16_t*>(g.Out);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mb * 16 + (lane >> 4) * 4 + i;
          if (r < mv) {
            bf16_t* orow = Out + static_cast<int64_t>(mrow0 + r) * g.ldo;
            if (SWIGLU) {
#pragma unroll
              for (int nb = 0; nb < 2; ++nb) {
                if (col[nb] < g.n_out) {
                  const float gv = acc[mb][nb][i];
                  const float uv = acc[mb][nb + 2][i];
                  const float h = gv / (1.0f + __expf(-gv)) * uv;
                  orow[col[nb]] = f32_to_bf16(h);
                }
              }
            } else {
#pragma unroll
              for (int nb = 0; nb < 4; ++nb)
                if (col[nb] < g.n_out) orow[col[nb]] = f32_to_bf16(acc[mb][nb][i]);
            }
          }
        }
      }
    }
  }
}

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
      cus[dev] = prop.multiProcessorCount;
    else
      cus[dev] = 256;
  }
  return cus[dev];
}

template <int MB, int PF>
static hipError_t launch_mb(const FfnLaunch& fl, int phase, int blocks_per_cu, hipStream_t st) {
  constexpr int BM = 16 * MB;
  long long ub = 0;
  for (int i = 0; i < fl.ngroups; ++i) {
    const FfnGroup& g = fl.g[i];
    const long long maxrows = g.seg_off ? g.rows : g.rows;  // rows = max rows bound
    ub += ((maxrows + BM - 1) / BM + g.nseg) * static_cast<long long>(fl.nt[i]);
  }
  if (ub <= 0) return hipSuccess;
  long long grid = static_cast<long long>(device_cus()) * blocks_per_cu;
  const long long ub8 = (ub + 7) / 8 * 8;
  if (grid > ub8) grid = ub8;
  grid = (grid + 7) / 8 * 8;
  if (phase == 0)
    ffn_bf16_kernel<MB, PF, true><<<static_cast<int>(grid), kThreads, 0, st>>>(fl);
  else
    ffn_bf16_kernel<MB, PF, false><<<static_cast<int>(grid), kThreads, 0, st>>>(fl);
  return hipGetLastError();
}

hipError_t launch_ffn_bf16(const FfnGroup* groups, int ngroups, int phase, int rows_hint,
                           hipStream_t st) {
  FfnLaunch fl{};
  fl.ngroups = ngroups;
  for (int i = 0; i < ngroups; ++i) {
    fl.g[i] = groups[i];
    const int cols = phase == 0 ? 128 : 256;
    fl.nt[i] = (groups[i].n_out + cols - 1) / cols;
  }
  if (rows_hint >= 128) return launch_mb<8, 1>(fl, phase, 1, st);
  if (rows_hint >= 32) return launch_mb<4, 2>(fl, phase, 2, st);
  return launch_mb<1, 4>(fl, phase, 2, st);
}

// ================================================================ fp32 path
// Plain fp32 arithmetic, one thread per output element (small fp32 layers).
template <bool SWIGLU>
__global__ __launch_bounds__(256) void ffn_f32_kernel(FfnGroup g, int max_rows) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int r = static_cast<int>(idx / g.n_out);
  const int c = static_cast<int>(idx - static_cast<int64_t>(r) * g.n_out);
  if (r >= max_rows) return;
  const int total = g.seg_off ? g.seg_off[g.nseg] : g.rows;
  if (r >= total) return;
  int s = 0;
  if (g.seg_off) {
    int i0 = 0, i1 = g.nseg;
    while (i1 - i0 > 1) {
      const int mid = (i0 + i1) >> 1;
      if (g.seg_off[mid] <= r) i0 = mid;
      else i1 = mid;
    }
    s = i0;
  }
  const int arow = g.row_index ? g.row_index[r] : r;
  const float* a = static_cast<const float*>(g.A) + static_cast<int64_t>(arow) * g.lda;
  const float* W = static_cast<const float*>(g.W) + static_cast<int64_t>(s) * g.w_stride;
  float* out = static_cast<float*>(g.Out) + static_cast<int64_t>(r) * g.ldo;
  if (SWIGLU) {
    const float* wg = W + static_cast<int64_t>(c) * g.K;
    const float* wu = W + static_cast<int64_t>(g.up_off + c) * g.K;
    float gv = 0.f, uv = 0.f;
    for (int kk = 0; kk < g.K; ++kk) {
      gv = fmaf(wg[kk], a[kk], gv);
      uv = fmaf(wu[kk], a[kk], uv);
    }
    out[c] = gv / (1.0f + expf(-gv)) * uv;
  } else {
    const float* w = W + static_cast<int64_t>(c) * g.K;
    float acc = 0.f;
    for (int kk = 0; kk < g.K; ++kk) acc = fmaf(w[kk], a[kk], acc);
    out[c] = acc;
  }
}

hipError_t launch_ffn_f32(const FfnGroup& g, int phase, int max_rows, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(max_rows) * g.n_out;
  if (n <= 0) return hipSuccess;
  const int blocks = static_cast<int>((n + 255) / 256);
  if (phase == 0)
    ffn_f32_kernel<true><<<blocks, 256, 0, st>>>(g, max_rows);
  else
    ffn_f32_kernel<false><<<blocks, 256, 0, st>>>(g, max_rows);
  return hipGetLastError();
}

}  // namespace moe
