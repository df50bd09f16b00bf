// grouped_ffn.hip -- grouped SwiGLU expert GEMMs over variable-size row
// segments (the routed experts) plus extra groups (the shared expert), in one
// persistent launch per phase.
//
// Sources: "DeepSeek MoE：从v1到v3的演进" §DeepSeek-v1 (fine-grained routed
// experts; isolated shared experts every token passes through);
// "从零构建DeepSeekMoE…" §2.2 (layer output = shared experts + routed
// experts).  The expert form is SwiGLU: h = silu(Wg a) * (Wu a), y = Wd h.
//
// bf16 weights are tiled (see kTileElems): every wave-wide weight load is one
// contiguous KiB that already holds each lane's MFMA fragment, which streams
// from HBM measurably faster than 16 rows x 64 bytes of a row-major matrix.
//
// bf16 path (gfx950 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// Segments of 128 rows and more run the 8-wave large-tile kernels
// (ffn_pp_kernel, ffn_big_kernel: both operands loaded straight into LDS,
// described where they are defined); smaller segments (decode) run
// ffn_bf16_kernel:
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
//  * persistent grid, XCD-aware (workgroup id mod 8 is its XCD): tiles that
//    share an expert's weights (consecutive m-tiles of one n-tile) and its
//    activations (consecutive n-tiles) are handed to the same XCD at the same
//    time, so they meet in that XCD's L2.  The large-segment kernels deal the
//    tile list out in rounds (each XCD a run of consecutive tiles per round),
//    which keeps the XCDs equally loaded; the small-segment kernel gives each
//    XCD a contiguous eighth of the list.
#include <type_traits>

#include "moe_internal.h"
#include "lds_dma.h"

namespace moe {

// Tile configuration of the small-segment kernel's three tile families
// (rows per tile = 16 * MB, weight fragments prefetched PF steps ahead) and
// its occupancy (workgroups per CU).
constexpr int kBigMB = 8, kBigPF = 1;    // >= 128 rows when the large-tile kernels cannot run
constexpr int kMidMB = 4, kMidPF = 2;    // 32 .. 127 rows per segment
constexpr int kSmallPF = 4;              // < 32 rows per segment (decode), 16-row tiles
constexpr int kSmallBlocksPerCU = 2;
constexpr int kMinBlocks = 2;            // launch bound of ffn_bf16_kernel

constexpr int kBK = 64;        // k per pipeline step (8 chunks of 16 bytes)
// Tiled weights: blocks of 16 rows x 32 k (1 KiB, kTileElems elements); the
// blocks of one 16-row group are consecutive in k, and inside a block lane
// l's MFMA fragment (row l % 16, k 8 * (l / 16) .. + 7) is the l-th 16 bytes.
constexpr int kTileElems = 512;
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

// Group `grp` of a launch as a value chosen field by field: no address into
// the kernel arguments is formed, so they are not copied to private memory
// (whose loads would count among the loads in flight).
__device__ __forceinline__ FfnGroup pick_group(const FfnLaunch& a, int grp) {
  const bool o = grp != 0;
  const FfnGroup& g0 = a.g[0];
  const FfnGroup& g1 = a.g[1];
  FfnGroup g;
  g.A = o ? g1.A : g0.A;
  g.lda = o ? g1.lda : g0.lda;
  g.row_index = o ? g1.row_index : g0.row_index;
  g.seg_off = o ? g1.seg_off : g0.seg_off;
  g.nseg = o ? g1.nseg : g0.nseg;
  g.rows = o ? g1.rows : g0.rows;
  g.W = o ? g1.W : g0.W;
  g.w_stride = o ? g1.w_stride : g0.w_stride;
  g.Out = o ? g1.Out : g0.Out;
  g.ldo = o ? g1.ldo : g0.ldo;
  g.K = o ? g1.K : g0.K;
  g.n_out = o ? g1.n_out : g0.n_out;
  g.up_off = o ? g1.up_off : g0.up_off;
  g.a_bytes = o ? g1.a_bytes : g0.a_bytes;
  g.w_bytes = o ? g1.w_bytes : g0.w_bytes;
  g.o_bytes = o ? g1.o_bytes : g0.o_bytes;
  return g;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Threads beyond the first 256 of a larger workgroup pass the same barriers
// as build_tile_starts without work.
__device__ __forceinline__ void build_tile_starts_idle() {
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    __syncthreads();
    __syncthreads();
  }
  __syncthreads();
}

// Exclusive prefix of `cnt` tiles per flat segment into tstart[0..n].
template <int BM>
__device__ __forceinline__ void build_tile_starts(const FfnLaunch& a, int nsegT, int* tstart,
                                                  int* tmp) {
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
      const FfnGroup g = pick_group(a, grp);
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

// Rows/columns a tile works on, decoded once per tile.
struct TileCtx {
  FfnGroup g;  // a copy: uniform values, no pointer into the kernel arguments
  int s;       // segment
  int nt;      // n-tile
  int mrow0;   // first problem row of the tile
  int mv;      // valid rows in the tile (1..BM)
};

// One tile with NMB live M-blocks of 16 rows (NMB*16 >= mv), all loops
// static.  MFMA operands are (weights, activations), so the accumulator of
// a lane holds 4 consecutive output columns of one row: D'[4*(lane/16)+i]
// [lane%16] = out[row lane%16][col 4*(lane/16)+i].
template <int NMB, int PF, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const TileCtx& c, bf16_t* __restrict__ As) {
  constexpr int ROWS = 16 * NMB;
  constexpr int APASS = (ROWS * 8 + kThreads - 1) / kThreads;
  constexpr int NSLOT = PF + 1;
  constexpr int BUF = ROWS * kBK;  // elements per LDS buffer
  const FfnGroup& g = c.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int K = g.K;
  const int nk = K / kBK;

  // activation loader: thread -> (row, 16-byte chunk); rows past the valid
  // ones reload the last valid row (never read back into a stored output)
  const bf16_t* A = static_cast<const bf16_t*>(g.A);
  const bf16_t* aptr[APASS];
  int aoff[APASS];
  bool aact[APASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) {
    const int row = (tid >> 3) + 32 * p;
    const int ch = tid & 7;
    aact[p] = row < ROWS;
    int prow = c.mrow0 + min(row, c.mv - 1);
    if (g.row_index) prow = g.row_index[prow];
    aptr[p] = A + static_cast<int64_t>(prow) * g.lda + ch * 8;
    const int r = aact[p] ? row : 0;
    aoff[p] = r * kBK + ((ch ^ ((r >> 1) & 7)) * 8);
  }

  // weight blocks of this wave: 4 tiled blocks of 16 rows; lane l's fragment
  // of k-block kb is the 16 bytes at block + kb * 1 KiB + l * 16
  const bf16_t* W = static_cast<const bf16_t*>(g.W) + static_cast<int64_t>(c.s) * g.w_stride;
  const bf16_t* bptr[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    int brow;  // first weight row of the block (blocks past n_out read block 0)
    if (SWIGLU) {
      const int col = c.nt * 128 + wave * 32 + (nb & 1) * 16;
      const int cc = col < g.n_out ? col : 0;
      brow = (nb < 2) ? cc : g.up_off + cc;
    } else {
      const int col = c.nt * 256 + wave * 64 + nb * 16;
      brow = col < g.n_out ? col : 0;
    }
    bptr[nb] = W + static_cast<int64_t>(brow) * K + lane * 8;
  }

  f32x4 acc[NMB][4];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 bbuf[NSLOT][2][4];
  u32x4 areg[APASS];

  // each weight byte is read once, by this wave only: the loads carry the
  // non-temporal hint (measured on the V3 decode layer: gate/up 2.30 ->
  // 2.10 ms, 6.6 TB/s; down 1.14 -> 1.09 ms)
  auto load_b = [&](int step, u32x4 (&dst)[2][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        dst[ks][nb] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(bptr[nb] + (step * 2 + ks) * kTileElems));
  };
  auto load_a = [&](int step) {
#pragma unroll
    for (int p = 0; p < APASS; ++p)
      if (aact[p]) areg[p] = *reinterpret_cast<const u32x4*>(aptr[p] + step * kBK);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < APASS; ++p)
      if (aact[p]) *reinterpret_cast<u32x4*>(As + buf * BUF + aoff[p]) = areg[p];
  };
  auto compute = [&](int buf, const u32x4 (&b)[2][4]) {
    const bf16_t* Ab = As + buf * BUF;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int row = mb * 16 + (lane & 15);
        const int ch = ks * 4 + (lane >> 4);
        const bf16x8 af = as_bf16x8(
            *reinterpret_cast<const u32x4*>(Ab + row * kBK + ((ch ^ ((row >> 1) & 7)) * 8)));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b[ks][nb]), af,
                                                                acc[mb][nb], 0, 0, 0);
      }
    }
  };

  // prologue
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < nk) load_b(u, bbuf[u]);
  load_a(0);
  store_a(0);
  __syncthreads();

  // main loop, unrolled by NSLOT so the register ring is indexed statically
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

  // epilogue: 4 consecutive columns of one row per lane -> one 8-byte store
  bf16_t* Out = static_cast<bf16_t*>(g.Out);
  const int rl = lane & 15;
  const int cq = (lane >> 4) * 4;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * 16 + rl;
    if (r < c.mv) {
      bf16_t* orow = Out + static_cast<int64_t>(c.mrow0 + r) * g.ldo;
      if (SWIGLU) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = c.nt * 128 + wave * 32 + nb * 16 + cq;
          if (col < g.n_out) {
            uint32_t w[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float g0 = acc[mb][nb][2 * h], g1 = acc[mb][nb][2 * h + 1];
              const float u0 = acc[mb][nb + 2][2 * h], u1 = acc[mb][nb + 2][2 * h + 1];
              const float h0 = g0 / (1.0f + __expf(-g0)) * u0;
              const float h1 = g1 / (1.0f + __expf(-g1)) * u1;
              w[h] = pack_bf16x2(h0, h1);
            }
            *reinterpret_cast<u32x2*>(orow + col) = u32x2{w[0], w[1]};
          }
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = c.nt * 256 + wave * 64 + nb * 16 + cq;
          if (col < g.n_out) {
            const uint32_t w0 = pack_bf16x2(acc[mb][nb][0], acc[mb][nb][1]);
            const uint32_t w1 = pack_bf16x2(acc[mb][nb][2], acc[mb][nb][3]);
            *reinterpret_cast<u32x2*>(orow + col) = u32x2{w0, w1};
          }
        }
      }
    }
  }
}

template <int NMB, int PF, bool SWIGLU>
__device__ __forceinline__ void run_tile(const TileCtx& c, int nmb, bf16_t* As) {
  if constexpr (NMB == 1) {
    gemm_tile<1, PF, SWIGLU>(c, As);
  } else {
    if (nmb > NMB / 2) gemm_tile<NMB, PF, SWIGLU>(c, As);
    else run_tile<NMB / 2, PF, SWIGLU>(c, nmb, As);
  }
}

template <int MB, int PF, bool SWIGLU>
__global__ __launch_bounds__(kThreads, kMinBlocks) void ffn_bf16_kernel(FfnLaunch a) {
  constexpr int BM = 16 * MB;
  __shared__ __attribute__((aligned(16))) bf16_t As[2 * BM * kBK];
  __shared__ int tstart[kMaxSegs + 1];
  __shared__ int tmp[kThreads];

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
    int i0 = 0, i1 = nsegT;
    while (i1 - i0 > 1) {
      const int mid = (i0 + i1) >> 1;
      if (tstart[mid] <= L) i0 = mid;
      else i1 = mid;
    }
    const int grp = (a.ngroups > 1 && i0 >= a.g[0].nseg) ? 1 : 0;
    TileCtx c;
    c.g = grp ? a.g[1] : a.g[0];
    c.s = grp ? i0 - a.g[0].nseg : i0;
    const int r0 = seg_begin(c.g, c.s);
    const int rows = seg_end(c.g, c.s) - r0;
    const int mtc = (rows + BM - 1) / BM;
    const int local = L - tstart[i0];
    c.nt = local / mtc;
    const int mt = local - c.nt * mtc;
    c.mrow0 = r0 + mt * BM;
    c.mv = min(BM, rows - mt * BM);
    const int nmb = (c.mv + 15) >> 4;
    // the smallest compiled tile height (MB, MB/2, ..., 1 blocks) covering
    // the valid rows
    run_tile<MB, PF, SWIGLU>(c, nmb, As);
    __syncthreads();
  }
}

// =====================================================================
// Large-segment kernel (prefill-sized segments, >= ~128 rows per expert).
//
// One workgroup per CU computes a 256-row x 256-weight-row tile with 8 waves
// (2 per SIMD) in a 2 x 4 layout: wave (wm, wn) = (wave & 1, wave >> 1).
// Both operands stream global -> LDS with gfx950's direct buffer loads
// (buffer_load_dwordx4 ... lds, see lds_dma.h), so no registers stage them;
// each wave then reads 16-byte MFMA fragments from LDS.  A wave owns the
// M-blocks of one parity (blocks 2j + wm), so a tile with fewer rows
// shortens every wave's work equally.  Row splits of a segment are balanced
// (ceil(rows / tiles) rows each), so the tiles that share an expert's
// weights cost the same and stream them through L2 together.
// =====================================================================
constexpr int kBigRows = 256;   // max rows per tile
constexpr int kBigBufElems = 256 * kBK;

constexpr int kBigThreads = 512;  // 8 waves, 2 per SIMD

// Wave (wm, wn) = (wave & 1, wave >> 1): M-blocks 2j + wm (j < NMBW), four
// 16-row weight blocks; gate/up phase: gate blocks 2wn, 2wn+1 and the up
// blocks 8 + 2wn, 8 + 2wn + 1 (same h columns), plain phase: 4wn .. 4wn+3.
template <bool SWIGLU>
__device__ __forceinline__ int big_wblock(int wn, int nb) {
  if (SWIGLU) return (nb < 2 ? 0 : 8) + wn * 2 + (nb & 1);
  return wn * 4 + nb;
}

// Fragment reads of the large-tile kernels: the four weight fragments and
// the first kReadAhead activation fragments first, then per M-block two
// MFMAs, the read of the fragment kReadAhead blocks ahead, two MFMAs, so the
// LDS latency of a fragment is covered by the MFMAs of earlier blocks.
constexpr int kReadAhead = 2;
template <int NMBW>
__device__ __forceinline__ void fragment_issue_order() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4 + (kReadAhead < NMBW ? kReadAhead : NMBW), 0);
#pragma unroll
  for (int j = 0; j < NMBW; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    if (j + kReadAhead < NMBW) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

template <int NMBW, bool SWIGLU>
__device__ __forceinline__ void big_compute(const bf16_t* __restrict__ Ab,
                                            const bf16_t* __restrict__ Bb, f32x4 (&acc)[8][4],
                                            int wm, int wn) {
  const int lane = threadIdx.x & 63;
  // every fragment row is 16*block + lane%16, so the swizzle term
  // ((row >> 1) & 7) is (lane%16) >> 1 for all blocks: one base address per
  // operand, block offsets are immediates
  const int swz = (lane & 15) >> 1;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ch = (ks * 4 + (lane >> 4)) ^ swz;
    const bf16_t* abase = Ab + (wm * 16 + (lane & 15)) * kBK + ch * 8;
    // weight LDS slots: row block q, k-block ks at slot 2q + ks, fragment order
    const bf16_t* bbase = Bb + ks * kTileElems + lane * 8;
    bf16x8 bf[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bf[nb] = as_bf16x8(
          *reinterpret_cast<const u32x4*>(bbase + big_wblock<SWIGLU>(wn, nb) * 2 * kTileElems));
    bf16x8 af[NMBW];
#pragma unroll
    for (int j = 0; j < kReadAhead && j < NMBW; ++j)
      af[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + j * 32 * kBK));
#pragma unroll
    for (int j = 0; j < NMBW; ++j) {
      if (j + kReadAhead < NMBW)
        af[j + kReadAhead] =
            as_bf16x8(*reinterpret_cast<const u32x4*>(abase + (j + kReadAhead) * 32 * kBK));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[nb], af[j], acc[j][nb], 0, 0, 0);
    }
    fragment_issue_order<NMBW>();
  }
}

// v (in a vector register) as a value the compiler cannot see through, so
// that a constant used once is materialised where it is used instead of
// being held in a register across the kernel's loops
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// An LDS buffer's address as a value the compiler cannot trace back to the
// buffer.  The ping-pong kernel orders its direct global->LDS loads and the
// LDS reads of the same buffers with its own counted waits and barriers; on
// addresses it can trace, the compiler adds waits of its own before the
// reads, counted for the most cautious path through the kernel's loops,
// which hold back loads and stores the reads do not depend on.
template <typename T>
__device__ __forceinline__ T* lds_opaque(T* p) {
  __attribute__((address_space(3))) T* q = (__attribute__((address_space(3))) T*)p;
  asm volatile("" : "+s"(q));
  return (T*)q;
}

// SwiGLU of a gate/up accumulator pair, rounded to bf16 and packed: two h
// columns per 32-bit word (lower column in the low half).  silu(g) =
// g * 1/(1 + e^-g) with the hardware reciprocal (1 ulp), far below the bf16
// rounding of h; e^-g = inf gives 1/inf = 0, so silu -> -0 as g -> -inf.
__device__ __forceinline__ uint32_t swiglu_pack(float g0, float g1, float u0, float u1) {
  const float h0 = g0 * __builtin_amdgcn_rcpf(1.0f + __expf(-g0)) * u0;
  const float h1 = g1 * __builtin_amdgcn_rcpf(1.0f + __expf(-g1)) * u1;
  return pack_bf16x2(h0, h1);
}

// Stores a tile epilogue issues per wave, whatever the tile's height: the
// count the next tile's first wait is built from (gate/up: one per M-block
// of the tallest tile, down: two).
template <bool SWIGLU>
constexpr int kPPStores = SWIGLU ? 8 : 16;

// Lane swaps between two registers (gfx950): swap32 exchanges a's lanes
// 32-63 with b's lanes 0-31, swap16 a's odd 16-lane rows with b's even ones.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// Cache-policy bits of the ping-pong epilogues' h and y stores: device
// scope (sc1).  Measured against the default on V3 prefill, alternating in
// one process: the gate/up launch 1-1.5 % faster, the down launch 0.1-0.8 %
// faster in four of five runs (0.3 % slower in one).
constexpr int kStoreDeviceScope = 16;

// Gate/up tile epilogue straight from registers.  Per M-block a lane holds,
// for row r = lane % 16, h of columns 16 nb + 4 q .. + 3 (q = lane / 16) of
// the wave's two 16-column blocks nb, one 8-byte word each.  A swap of lane
// bit 5 with nb, then of lane bit 4 with nb, leaves lane (r, q) with the
// words of columns 8 q .. 8 q + 7, stored as one 16-byte piece: each store
// instruction writes 64 contiguous bytes (the wave's 32 columns) of each of
// 16 rows.  Every store is issued (a lane whose row lies past mv or whose
// columns lie past n_out gets an offset past the buffer's bound, which the
// hardware drops), and the count is padded with dropped stores, so a wave
// issues exactly kPPStores<true> store instructions.  The buffer bound (o_bytes)
// is at most 0xFFFFFF00, so a dropped offset never wraps.
template <int NJ>
__device__ __forceinline__ int gate_up_epilogue(const FfnGroup& g, const f32x4 (&acc)[NJ][4],
                                                int wm, int wn, int nt, int mrow0, int mv) {
  const int lane = static_cast<int>(opaque_u32(threadIdx.x)) & 63;  // derived here
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(g.Out, g.o_bytes);
  const int rl = lane & 15;
  const int col = nt * 128 + wn * 32 + (lane >> 4) * 8;
  const uint32_t ldo2 = static_cast<uint32_t>(g.ldo) * 2u;
  u32x4 last;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = (2 * j + wm) * 16 + rl;
    uint32_t w[2][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      w[nb][0] = swiglu_pack(acc[j][nb][0], acc[j][nb][1], acc[j][nb + 2][0], acc[j][nb + 2][1]);
      w[nb][1] = swiglu_pack(acc[j][nb][2], acc[j][nb][3], acc[j][nb + 2][2], acc[j][nb + 2][3]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      swap32(w[0][h], w[1][h]);
      swap16(w[0][h], w[1][h]);
    }
    const uint32_t off = (r < mv && col < g.n_out)
                             ? static_cast<uint32_t>(mrow0 + r) * ldo2 + static_cast<uint32_t>(col) * 2u
                             : 0xFFFFFFF0u;
    last = u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
    __builtin_amdgcn_raw_buffer_store_b128(last, ro, off, 0, kStoreDeviceScope);
  }
  if constexpr (NJ < kPPStores<true>) {
    const uint32_t drop = opaque_u32(0xFFFFFFF0u);
#pragma unroll
    for (int j = NJ; j < kPPStores<true>; ++j) __builtin_amdgcn_raw_buffer_store_b128(last, ro, drop, 0, 0);
  }
  return kPPStores<true>;
}

// Down tile epilogue of one wave, staged through the wave's own 2 KiB LDS
// slot so that the outputs leave as whole 128-byte row pieces: per M-block
// the wave writes its 16 rows x 64 columns, rounded to bf16, into the slot
// and reads them back as 8 rows x 128 bytes per instruction.  16-byte chunk
// c of staged row r sits at position c ^ (r % 8).  LDS instructions of one
// wave are processed in order, so a block's writes never overtake the
// previous block's reads of the slot, and no barrier is involved: group 0
// runs it while group 1 issues its last MFMAs, group 1 while group 0 issues
// the next tile's first ones.  Rows past mv and columns past n_out get an
// offset past the buffer's bound (dropped), and a short tile pads with
// dropped stores, so a wave issues exactly kPPStores<false> store instructions.
template <int NJ>
__device__ __forceinline__ int wave_staged_epilogue(const FfnGroup& g, const f32x4 (&acc)[NJ][4],
                                                    int wm, int wn, int nt, int mrow0, int mv,
                                                    bf16_t* slot) {
  const int lane = static_cast<int>(opaque_u32(threadIdx.x)) & 63;  // derived here
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(g.Out, g.o_bytes);
  const uint32_t ldo2 = static_cast<uint32_t>(g.ldo) * 2u;
  char* S = reinterpret_cast<char*>(slot);
  const int r = lane & 15;   // accumulator row of this lane
  const int q = lane >> 4;   // 4-column group inside a 16-column block
  const int rr = lane >> 3;  // rows rr and rr + 8 are read back
  const int cc = lane & 7;   // 16-byte chunk read back
  u32x4 last;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int c = 2 * nb + (q >> 1);
      *reinterpret_cast<u32x2*>(S + r * 128 + ((c ^ (r & 7)) << 4) + (q & 1) * 8) =
          u32x2{pack_bf16x2(acc[j][nb][0], acc[j][nb][1]), pack_bf16x2(acc[j][nb][2], acc[j][nb][3])};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = rr + 8 * i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(S + row * 128 + ((cc ^ (row & 7)) << 4));
      const int trow = (2 * j + wm) * 16 + row;
      const int col = nt * 256 + wn * 64 + cc * 8;
      const uint32_t o = (trow < mv && col < g.n_out)
                             ? static_cast<uint32_t>(mrow0 + trow) * ldo2 + static_cast<uint32_t>(col) * 2u
                             : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, o, 0, kStoreDeviceScope);
      last = v;
    }
  }
  if constexpr (2 * NJ < kPPStores<false>) {
    const uint32_t drop = opaque_u32(0xFFFFFFF0u);
#pragma unroll
    for (int j = 2 * NJ; j < kPPStores<false>; ++j) __builtin_amdgcn_raw_buffer_store_b128(last, ro, drop, 0, 0);
  }
  return kPPStores<false>;
}

// In the 2-stage kernel tiles run back to back: the first stage of the next
// tile is loaded during the last step of the current one, before the
// current tile's stores, so the next tile's first wait skips those stores
// (vmcnt retires in issue order) and no tile starts with an empty pipeline.
// Tile order inside one segment of mtc row tiles x ntc column tiles: row
// tiles are taken in groups of up to kGroupM, and inside a group the order is
// column-major (all row tiles of the group for column tile 0, then column 1,
// ...).  A run of 32 consecutive tiles (one XCD's share of a round) then covers
// a block of several row tiles by several column tiles, whose activation rows
// and weight rows are each fetched once into that XCD's L2.  Segments of at
// most kGroupM row tiles (every routed expert at the usual sizes) keep the
// plain column-major order; the 8192-row shared segment of a prefill batch no
// longer streams all of x once per column tile.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_nm(int local, int mtc, int ntc, int& nt, int& mt) {
  const int g = local / (kGroupM * ntc);
  const int m0 = g * kGroupM;
  const int gm = min(kGroupM, mtc - m0);
  const int w = local - g * kGroupM * ntc;
  nt = w / gm;
  mt = m0 + (w - nt * gm);
}

struct BigTile {
  int grp, s, nt, mrow0, mv, nmbw, nk;
};

// Where a tile's operands come from (plain values; buffer descriptors are
// built from them at issue time).
struct BigLoads {
  const void* a_base;
  const void* w_base;
  uint32_t a_bytes, w_bytes;
  uint32_t aoff[4];   // per lane: activation row byte offset + chunk
  uint32_t bsoff[4];  // uniform: first weight row of each row-block pair, in bytes
  int rows_needed;
};

__device__ __forceinline__ BigTile big_decode(const FfnLaunch& a, const int* tstart, int nsegT,
                                              int L) {
  int i0 = 0, i1 = nsegT;
  while (i1 - i0 > 1) {
    const int mid = (i0 + i1) >> 1;
    if (tstart[mid] <= L) i0 = mid;
    else i1 = mid;
  }
  BigTile t;
  t.grp = (a.ngroups > 1 && i0 >= a.g[0].nseg) ? 1 : 0;
  const FfnGroup g = t.grp ? a.g[1] : a.g[0];
  t.s = t.grp ? i0 - a.g[0].nseg : i0;
  const int r0 = seg_begin(g, t.s);
  const int rows = seg_end(g, t.s) - r0;
  const int mtc = (rows + kBigRows - 1) / kBigRows;
  const int rpt = ((rows + mtc - 1) / mtc + 15) & ~15;  // balanced rows per tile
  const int local = L - tstart[i0];
  int mt;
  tile_nm(local, mtc, t.grp ? a.nt[1] : a.nt[0], t.nt, mt);
  t.mrow0 = r0 + mt * rpt;
  t.mv = min(rpt, rows - mt * rpt);
  t.nmbw = (((t.mv + 15) >> 4) + 1) >> 1;  // blocks per wave (interleaved)
  t.nk = g.K / kBK;
  return t;
}

// DMA geometry: 4 activation row groups per thread, group q = p*8 + wave
// covers tile rows [8q, 8q+8); this lane brings row 8q + lane/8, physical
// chunk lane%8, i.e. logical chunk (lane%8) ^ ((row >> 1) & 7), where
// (row >> 1) & 7 = 4*(wave & 1) + lane/16 for every p.  Weights, tiled: a
// step (64 k) of the tile is 16 row blocks x 2 k-blocks of 1 KiB;
// instruction j = p*8 + wave copies block (j / 2, k-block j % 2) into LDS
// slot j as is (fragment order).
template <bool SWIGLU>
__device__ __forceinline__ BigLoads big_loads(const FfnGroup& g, const BigTile& t, int wave,
                                              int lane) {
  BigLoads L;
  L.a_base = g.A;
  L.a_bytes = g.a_bytes;
  L.w_base = static_cast<const bf16_t*>(g.W) + static_cast<int64_t>(t.s) * g.w_stride;
  L.w_bytes = g.w_bytes;
  const int logical = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = (p * 8 + wave) * 8 + (lane >> 3);
    int prow = t.mrow0 + min(row, t.mv - 1);
    if (g.row_index) prow = g.row_index[prow];
    L.aoff[p] = static_cast<uint32_t>(prow) * static_cast<uint32_t>(g.lda) * 2u + logical * 16;
  }
  const uint32_t krow_bytes = static_cast<uint32_t>(g.K) * 2u;
  const int col0 = SWIGLU ? t.nt * 128 : t.nt * 256;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int q = 4 * p + (wave >> 1);  // row block of the tile; gate/up: 8.. are the up half
    // columns past n_out (never stored) read block 0, so the offset, which
    // the buffer's range check does not cover, stays inside the expert
    const int c = col0 + 16 * ((SWIGLU && q >= 8) ? q - 8 : q);
    const int wr = ((SWIGLU && q >= 8) ? g.up_off : 0) + (c < g.n_out ? c : 0);
    L.bsoff[p] = wave_uniform(static_cast<uint32_t>(wr) * krow_bytes);
  }
  L.rows_needed = 2 * t.nmbw * 16;  // tile rows any wave reads
  return L;
}

__device__ __forceinline__ void big_issue(const BigLoads& L, int step, bf16_t* Ab, bf16_t* Bb,
                                          int wave, int lane) {
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(wave_uniform(L.a_base), L.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(wave_uniform(L.w_base), L.w_bytes);
  const uint32_t kb = static_cast<uint32_t>(step) * (kBK * 2);
  const uint32_t kw = static_cast<uint32_t>(step) * 2048u;
  const uint32_t boff = static_cast<uint32_t>(wave & 1) * 1024u + lane * 16u;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int q = p * 8 + wave;
    if (q * 8 < L.rows_needed) dma16(ra, L.aoff[p], kb, Ab + q * 8 * kBK);
    dma16(rb, boff, L.bsoff[p] + kw, Bb + q * kTileElems);
  }
}

// s_waitcnt vmcnt(n) for the store counts a 2-stage tile epilogue issues
__device__ __forceinline__ void wait_vmcnt_upto32(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 24: wait_vmcnt<24>(); break;
    case 28: wait_vmcnt<28>(); break;
    case 32: wait_vmcnt<32>(); break;
    default: wait_vmcnt<0>(); break;  // waiting for more is always correct
  }
}

// Stores of a finished tile: one 8-byte buffer store per (M-block, column
// block) and lane, issued unconditionally (a lane outside the tile gets an
// offset past the buffer bound, which the hardware drops), so the count is
// fixed: NMBW * (SWIGLU ? 2 : 4).
template <int NMBW, bool SWIGLU>
__device__ __forceinline__ int big_store(const FfnGroup& g, const f32x4 (&acc)[8][4], int wm,
                                         int wn, int nt, int mrow0, int mv) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(wave_uniform(static_cast<const void*>(g.Out)), g.o_bytes);
  const int rl = lane & 15;
  const int cq = (lane >> 4) * 4;
  const uint32_t ldo2 = static_cast<uint32_t>(g.ldo) * 2u;
#pragma unroll
  for (int j = 0; j < NMBW; ++j) {
    const int r = (2 * j + wm) * 16 + rl;
    const bool rv = r < mv;
    const uint32_t rowoff = static_cast<uint32_t>(mrow0 + r) * ldo2;
    if (SWIGLU) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = nt * 128 + wn * 32 + nb * 16 + cq;
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g0 = acc[j][nb][2 * h], g1 = acc[j][nb][2 * h + 1];
          const float u0 = acc[j][nb + 2][2 * h], u1 = acc[j][nb + 2][2 * h + 1];
          const float h0 = g0 / (1.0f + __expf(-g0)) * u0;
          const float h1 = g1 / (1.0f + __expf(-g1)) * u1;
          w[h] = pack_bf16x2(h0, h1);
        }
        const uint32_t off = (rv && col < g.n_out) ? rowoff + static_cast<uint32_t>(col) * 2u : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, ro, off, 0, 0);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = nt * 256 + wn * 64 + nb * 16 + cq;
        const uint32_t w0 = pack_bf16x2(acc[j][nb][0], acc[j][nb][1]);
        const uint32_t w1 = pack_bf16x2(acc[j][nb][2], acc[j][nb][3]);
        const uint32_t off = (rv && col < g.n_out) ? rowoff + static_cast<uint32_t>(col) * 2u : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, ro, off, 0, 0);
      }
    }
  }
  return NMBW * (SWIGLU ? 2 : 4);
}

// Persistent loop of the 2-stage kernel.  Every tile runs the 8-M-block
// compute (a short tile's extra MFMAs read rows that are never stored),
// while loads and stores cover only the tile's rows; one instantiation keeps
// the whole loop, both tiles' load addresses included, in registers.
template <bool SWIGLU>
__global__ __launch_bounds__(kBigThreads, 1) void ffn_big_kernel(FfnLaunch a) {
  __shared__ __attribute__((aligned(16))) bf16_t As0[kBigBufElems];
  __shared__ __attribute__((aligned(16))) bf16_t As1[kBigBufElems];
  __shared__ __attribute__((aligned(16))) bf16_t Bs0[kBigBufElems];
  __shared__ __attribute__((aligned(16))) bf16_t Bs1[kBigBufElems];
  __shared__ int tstart[kMaxSegs + 1];
  __shared__ int tmp[kThreads];

  const int nsegT = a.g[0].nseg + (a.ngroups > 1 ? a.g[1].nseg : 0);
  if (threadIdx.x < kThreads) build_tile_starts<kBigRows>(a, nsegT, tstart, tmp);
  else build_tile_starts_idle();
  const int total = tstart[nsegT];
  const int nxcd = 8;
  const int per = gridDim.x / nxcd;
  const int xcd = blockIdx.x % nxcd;
  const int slot = blockIdx.x / nxcd;
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int wm = wave & 1;
  const int wn = wave >> 1;
  // rounds of gridDim.x consecutive tiles; inside a round XCD x takes the
  // x-th run of `per` tiles (two experts' n-tiles: shared activation rows in
  // one L2), and every XCD gets work in every round
  int L = xcd * per + slot;
  if (L >= total) return;  // whole workgroup
  BigTile t = big_decode(a, tstart, nsegT, L);
  BigLoads cur = big_loads<SWIGLU>(t.grp ? a.g[1] : a.g[0], t, wave, lane);
  big_issue(cur, 0, As0, Bs0, wave, lane);
  int par = 0;        // buffer of the tile's first step
  int pending = 0;    // store instructions issued after the current step's loads
  for (;;) {
    const int Ln = L + static_cast<int>(gridDim.x);
    const bool has_next = Ln < total;
    BigTile tn = t;
    BigLoads nxt = cur;
    if (has_next) {
      tn = big_decode(a, tstart, nsegT, Ln);
      nxt = big_loads<SWIGLU>(tn.grp ? a.g[1] : a.g[0], tn, wave, lane);
    }
    f32x4 acc[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < t.nk; ++st) {
      const int b = (par + st) & 1;
      // this wave's loads of step st have landed (the previous tile's
      // stores, issued after them, may still be in flight at st == 0);
      // after the barrier every wave's share is in LDS and the other buffer
      // is no longer read
      if (st == 0) wait_vmcnt_upto32(pending);
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      bf16_t* Ac = b ? As1 : As0;
      bf16_t* Bc = b ? Bs1 : Bs0;
      if (st + 1 < t.nk) big_issue(cur, st + 1, b ? As0 : As1, b ? Bs0 : Bs1, wave, lane);
      else if (has_next) big_issue(nxt, 0, b ? As0 : As1, b ? Bs0 : Bs1, wave, lane);
      big_compute<8, SWIGLU>(Ac, Bc, acc, wm, wn);
    }
    pending = big_store<8, SWIGLU>(t.grp ? a.g[1] : a.g[0], acc, wm, wn, t.nt, t.mrow0, t.mv);
    if (!has_next) break;
    par = (par + t.nk) & 1;
    L = Ln;
    t = tn;
    cur = nxt;
  }
}

// ---------------------------------------------------------------------
// Ping-pong kernel (large segments, K % 128 = 0: both phases of the
// V3-shaped prefill layers, the gate/up phase of v1/v2).  Tiles of up to
// 256 activation rows x 256 weight rows, k-steps of 32, four weight stages
// and two activation buffers filled by direct global->LDS loads.
// The dispatcher places waves w and w + 4 of a workgroup on the same SIMD.
// Group 0 (waves 0-3) and group 1 (waves 4-7) run half a k-step apart: in
// every phase (closed by a workgroup barrier) one group reads a whole
// k-step's fragments from LDS into registers, and issues its part of a
// later stage's loads, while the other group issues that k-step's MFMAs
// back to back.  Each SIMD's matrix core is then fed by one wave at a time
// with no LDS waits between its MFMAs.
// Tiles run back to back in one stream of k-steps: the last three k-steps
// of a tile load the first stages of the workgroup's next tile into the
// buffers they have finished with, so a tile starts on stages already in
// LDS, and the groups keep their half-step offset across the tile boundary:
// group 0 stores its outputs while group 1 runs the last MFMAs, group 1
// while group 0 runs the next tile's first ones (down tiles, 256 output
// columns, through a per-wave LDS slot, so they leave as whole rows).
// An activation buffer holds two k-steps as 128-byte rows, so one wave's
// activation load covers 8 whole 128-byte lines.  (Loading each k-step as
// 64-byte rows, half of 16 lines per load, measured 6 % slower on both
// phases of the V3-shaped prefill layer.)
// ---------------------------------------------------------------------
constexpr int kBK4 = 32;
constexpr int kStages = 4;
constexpr int kBuf4Elems = 256 * kBK4;  // 16 KiB weight stage (256 weight rows)
// Activation rows per tile.  Taller tiles would keep an expert slightly over
// 256 rows in one tile and load its weights once, but 9 or 10 M-blocks per
// wave spill registers with this layout's address registers; with 64-byte
// rows, 320-row down tiles had been 4 % faster than 256 and 320-row gate/up
// tiles 5 % slower.
constexpr int kPPRows = 256;

// A tile of the ping-pong kernel (wave-uniform values).
struct PPTile {
  int grp, s, nt, mrow0, mv, nmbw, nk;
};

// Tile L of the flat tile list: its segment is the last one whose first
// tile is <= L, found by the whole wave in two rounds of LDS reads (lane l
// compares entry 16 l, then entries 16 h .. 16 h + 15 after the last lane h
// that passed; the tile starts do not decrease, so the lanes that pass form
// a prefix), rows from the segment table; all in LDS, so no memory
// instruction enters the count of loads in flight.
__device__ __forceinline__ PPTile pp_decode(const FfnLaunch& a, const int* tstart,
                                            const int* sbeg, const int* srows, int nsegT, int L) {
  static_assert(kMaxSegs <= 64 * 16, "two rounds of 64 lanes cover the segments");
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int i1 = lane * 16;
  const uint64_t m1 = __ballot(i1 < nsegT && tstart[i1] <= L);  // lane 0 always (tstart[0] = 0)
  const int h = 63 - __clzll(static_cast<long long>(m1));
  const int i2 = h * 16 + (lane & 15);
  const uint64_t m2 = __ballot(lane < 16 && i2 < nsegT && tstart[i2] <= L);
  const int i0 = wave_uniform(h * 16 + 63 - __clzll(static_cast<long long>(m2)));
  const int b0 = sbeg[i0], n0 = srows[i0], f0 = tstart[i0];  // three reads in flight together
  PPTile t;
  t.grp = (a.ngroups > 1 && i0 >= a.g[0].nseg) ? 1 : 0;
  t.s = t.grp ? i0 - a.g[0].nseg : i0;
  const int r0 = wave_uniform(b0);
  const int rows = wave_uniform(n0);
  const int mtc = (rows + kPPRows - 1) / kPPRows;
  const int rpt = ((rows + mtc - 1) / mtc + 15) & ~15;  // balanced rows per tile
  const int local = L - wave_uniform(f0);
  int mt;
  tile_nm(local, mtc, t.grp ? a.nt[1] : a.nt[0], t.nt, mt);
  t.mrow0 = r0 + mt * rpt;
  t.mv = min(rpt, rows - mt * rpt);
  t.nmbw = (((t.mv + 15) >> 4) + 1) >> 1;  // M-blocks per wave
  t.nk = (t.grp ? a.g[1].K : a.g[0].K) / kBK4;
  return t;
}

// Where a tile's operands come from.  Activation loads: 8 rows x 128 bytes
// per wave instruction; row group q = p*8 + wave covers tile rows [8q, 8q+8);
// lane -> row 8q + lane/8, physical chunk lane%8, logical chunk
// (lane%8) ^ ((row >> 1) & 7), and (row >> 1) & 7 = 4*(wave & 1) + lane/16
// for every p.  Rows past the tile's valid ones read from past the buffer's
// end, which returns zeros without a memory request (their results are
// never stored; a buffer within 256 MiB of 4 GiB repeats the last valid row
// instead, so that no offset wraps); groups past the tile's height are not
// loaded.  Weights, tiled: the wave copies the KiB of k-block `step` of row
// blocks `wave` and 8 + `wave` (gate/up: the gate and the up block of the
// same columns) into LDS slots `wave` and 8 + `wave`, in fragment order; a
// block whose columns lie past n_out (never stored) reads block 0 instead,
// so every address stays inside the expert's weights.
struct PPLoads {
  const void* a_base;
  const void* w_base;
  uint32_t a_bytes, w_bytes;
  uint32_t aoff[4];      // per lane: activation row byte offset + chunk of row group p*8 + wave
  uint32_t wrow0, wrow1; // uniform: byte offsets of the wave's two weight row blocks
  int g8;                // row groups of 8 the tile loads
};

// The row_index entries of this lane's four row groups, as exactly four
// buffer loads (without a row_index the buffer is empty: they return 0
// without touching memory), so that the count of loads in flight is known.
__device__ __forceinline__ void pp_rows_issue(const FfnGroup& g, const PPTile& t, int wave,
                                              int lane, uint32_t (&raw)[4]) {
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(g.row_index, g.row_index ? 0x7FFFFFF0u : 0u);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = (p * 8 + wave) * 8 + (lane >> 3);
    const int prow = t.mrow0 + min(row, t.mv - 1);
    raw[p] = __builtin_amdgcn_raw_buffer_load_b32(rr, static_cast<uint32_t>(prow) * 4u, 0, 0);
  }
}

// the weight half of a tile's load state
// The four row_index entries of every lane of the wave, brought into the
// wave's 256-byte slot of LDS by one direct load (lane l fetches entry l % 32:
// row group (l % 32) / 8, row l % 8 of the group, at slot[l]; lanes 32..63
// repeat lanes 0..31), so no register holds them while the tile's last
// steps run.
__device__ __forceinline__ void pp_rows_issue_lds(const FfnGroup& g, const PPTile& t, int wave,
                                                  int lane, int32_t* slot) {
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(g.row_index, g.row_index ? 0x7FFFFFF0u : 0u);
  lane = static_cast<int>(opaque_u32(threadIdx.x)) & 63;
  const int l = lane & 31;
  const int row = ((l >> 3) * 8 + wave) * 8 + (l & 7);
  const int prow = t.mrow0 + min(row, t.mv - 1);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)slot, 4,
                                           static_cast<uint32_t>(prow) * 4u, 0, 0, 0);
}
// this lane's four entries from the slot (the load has completed)
__device__ __forceinline__ void pp_rows_read_lds(const int32_t* slot, int lane,
                                                 uint32_t (&raw)[4]) {
  lane = static_cast<int>(opaque_u32(threadIdx.x)) & 63;
#pragma unroll
  for (int p = 0; p < 4; ++p) raw[p] = static_cast<uint32_t>(slot[p * 8 + (lane >> 3)]);
}

template <bool SWIGLU>
__device__ __forceinline__ void pp_wloads(const FfnGroup& g, const PPTile& t, int wave,
                                          PPLoads& L) {
  L.w_base = static_cast<const bf16_t*>(g.W) + static_cast<int64_t>(t.s) * g.w_stride;
  L.w_bytes = g.w_bytes;
  const uint32_t krow_bytes = static_cast<uint32_t>(g.K) * 2u;
  const int col0 = (SWIGLU ? t.nt * 128 : t.nt * 256) + wave * 16;
  const int c0 = col0 < g.n_out ? col0 : 0;
  const int c1 = SWIGLU ? g.up_off + c0 : (col0 + 128 < g.n_out ? col0 + 128 : 0);
  L.wrow0 = wave_uniform(static_cast<uint32_t>(c0) * krow_bytes);
  L.wrow1 = wave_uniform(static_cast<uint32_t>(c1) * krow_bytes);
}
// the activation half, from the row_index values pp_rows_issue loaded
__device__ __forceinline__ void pp_aloads(const FfnGroup& g, const PPTile& t, int wave, int lane,
                                          const uint32_t (&raw)[4], PPLoads& L) {
  lane = static_cast<int>(opaque_u32(threadIdx.x)) & 63;  // derived here, not held across the tile
  L.a_base = g.A;
  L.a_bytes = g.a_bytes;
  const int logical = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const bool zero_pad = g.a_bytes <= 0xF0000000u;
  const bool gather = g.row_index != nullptr;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = (p * 8 + wave) * 8 + (lane >> 3);
    const int prow = gather ? static_cast<int>(raw[p]) : t.mrow0 + min(row, t.mv - 1);
    L.aoff[p] = (row < t.mv || !zero_pad)
                    ? static_cast<uint32_t>(prow) * static_cast<uint32_t>(g.lda) * 2u + logical * 16
                    : g.a_bytes;
  }
  L.g8 = 4 * t.nmbw;
}

// activations of k-steps step, step + 1 (step even) into buffer Xb: NA
// loads per wave, row groups p*8 + wave for p < NA; a group past the tile's
// height reads zeros (its offset lies past the buffer's bound) into rows no
// M-block of the tile reads, so every wave issues the same count and the
// waits below are compile-time constants
template <int NA>
__device__ __forceinline__ void pp_issue_a(const PPLoads& L, int step, bf16_t* Xb, int wave) {
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(L.a_base, L.a_bytes);
  const uint32_t kb = static_cast<uint32_t>(step) * (kBK4 * 2);
#pragma unroll
  for (int p = 0; p < NA; ++p)
    dma16(ra, L.aoff[p], kb, Xb + (p * 8 + wave) * 8 * (2 * kBK4));
}
// weights of k-step `step` into stage Bb
__device__ __forceinline__ void pp_issue_w(const PPLoads& L, int step, bf16_t* Bb, int wave,
                                           uint32_t lane16) {
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(L.w_base, L.w_bytes);
  const uint32_t kw = static_cast<uint32_t>(step) * 1024u;
  dma16(rb, lane16, L.wrow0 + kw, Bb + wave * kTileElems);
  dma16(rb, lane16, L.wrow1 + kw, Bb + (8 + wave) * kTileElems);
}

// One tile, its epilogue and the first stages of the workgroup's next tile
// (Ln < total; without one, the same loads over empty buffers); on return t
// and cur describe the next tile.
//
// Load order of a wave.  Step k of a tile with nk >= 8 steps issues I(k):
//   k + 3 < nk: A(k+2, k+3) if k is even (NA loads), at k = nk - 4 the
//               next tile's row_index load R (1), W(k+3) (2);
//   otherwise:  k = nk-3: W'(0); k = nk-2: A'(0,1) (4 loads), W'(1);
//               k = nk-1: W'(2)  (the next tile's first stages);
// and between a tile's last step and the next tile's first the epilogue's
// kPPStores stores (S).  The first tile of a workgroup starts with W(0),
// A(0,1), W(1), W(2), the same order, and waits for all but W(2).  Stage j
// (W(j) and the activation pair holding j) is read by group 0 in phase 2j
// and by group 1 in phase 2j + 1; before the barrier that ends phase 2j - 1
// every wave waits for its own loads of stage j: after step j - 1 it lets
// only the loads issued after the last one stage j needs stay in flight
// (loads complete in issue order):
//   even k: |I(k-1)| + |I(k)|         (k = 0: W'(2) + S + |I(0)|)
//   odd k:  |I(k-1)| - (A count) + |I(k)|     (the pair is first in I(k-1))
// which is 4 + NA (even) and 4 (odd) in the middle of a tile, 4 + NA + S at
// k = 0, 4 + NA + 1 at nk-4, 5 at nk-3, 8 at nk-2 and 4 at nk-1; R has
// landed at the start of step nk-2 once at most W(nk-1) and W'(0) (4) are in
// flight.  A load into a buffer is issued only after the barrier by which
// both groups have read that buffer's last stage (W(k+3) goes where W(k-1)
// was, A(k+2, k+3) where A(k-2, k-1) was).
template <int NMBW, bool SWIGLU>
__device__ __forceinline__ void pp_tile(const FfnLaunch& a, const int* tstart, const int* sbeg,
                                        const int* srows, int nsegT, int Ln, int total,
                                        PPTile& t, PPLoads& cur, bf16_t* X0, bf16_t* X1,
                                        bf16_t* B0, bf16_t* B1, bf16_t* B2, bf16_t* B3,
                                        int32_t* rslot, bf16_t* stage) {
  static_assert(NMBW >= 1 && NMBW <= 8, "tiles hold at most 256 rows");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
  const int nk = wave_uniform(t.nk);  // multiple of 4, at least 8
  const bool has_next = Ln < total;
  constexpr int NA = (4 * NMBW + 7) / 8;  // activation loads per wave and pair of steps

  // a whole k-step's fragments: M-blocks 2j + wm (j < NMBW), weight blocks
  // of columns 32wn .. 32wn + 31 (gate and up); row 16*block + lane%16 has
  // swizzle term (lane%16) >> 1
  const int swz = (lane & 15) >> 1;
  const int arow = (wm * 16 + (lane & 15)) * (2 * kBK4);
  bf16x8 af[NMBW], bf[4];
  auto read = [&](const bf16_t* Xb, int half, const bf16_t* Bb) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bf[nb] = as_bf16x8(
          *reinterpret_cast<const u32x4*>(Bb + lane * 8 + big_wblock<SWIGLU>(wn, nb) * kTileElems));
    const bf16_t* abase = Xb + arow + (((half * 4 + (lane >> 4)) ^ swz) * 8);
#pragma unroll
    for (int j = 0; j < NMBW; ++j)
      af[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + j * 32 * (2 * kBK4)));
  };
  // fragment reads LO .. HI - 1 of a k-step (weight blocks 0-3, then
  // activation blocks), for interleaving with the direct-load issue
  auto read_part = [&](const bf16_t* Xb, int half, const bf16_t* Bb, auto lo_c, auto hi_c)
                       __attribute__((always_inline)) {
    constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
    const bf16_t* abase = Xb + arow + (((half * 4 + (lane >> 4)) ^ swz) * 8);
#pragma unroll
    for (int i = 0; i < 4 + NMBW; ++i) {
      if (i >= LO && i < HI) {
        if (i < 4)
          bf[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
              Bb + lane * 8 + big_wblock<SWIGLU>(wn, i) * kTileElems));
        else
          af[i - 4] = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + (i - 4) * 32 * (2 * kBK4)));
      }
    }
  };
  f32x4 acc[NMBW][4];
#pragma unroll
  for (int j = 0; j < NMBW; ++j)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // with an odd number of 16-row blocks the last block of the odd-parity
  // waves lies past the tile's rows: they skip its MFMAs (nothing of it is
  // stored)
  const bool skip_last = wm == 1 && ((((t.mv + 15) >> 4) & 1) != 0);
  auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NMBW - 1; ++j)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[nb], af[j], acc[j][nb], 0, 0, 0);
    if (!skip_last) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[NMBW - 1][nb] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[nb], af[NMBW - 1], acc[NMBW - 1][nb], 0, 0, 0);
    }
  };

// vmcnt(4 + NA + C)
#define PP_WAIT_NA(C) wait_vmcnt<4 + NA + (C)>();
// read phase of k-step (I), the waits of stage k + 1, the MFMA phase.  The
// wait after the second barrier repeats the one each group made (no loads
// are issued in between, so it returns at once); being unconditional, it
// tells the compiler that stage k + 1 has landed, which keeps it from adding
// waits of its own before the next LDS reads.
#define PP_PHASES(I, XR, BR, WAIT)        \
  read(XR, (I) & 1, BR);                  \
  wait_lgkmcnt0();                        \
  if (grp) { WAIT; }                      \
  __builtin_amdgcn_sched_barrier(0);      \
  __builtin_amdgcn_s_barrier();           \
  __builtin_amdgcn_sched_barrier(0);      \
  compute();                              \
  if (!grp) { WAIT; }                     \
  __builtin_amdgcn_sched_barrier(0);      \
  __builtin_amdgcn_s_barrier();           \
  __builtin_amdgcn_sched_barrier(0);      \
  { WAIT; }
#define PP_PHASES_NOREAD(WAIT)            \
  wait_lgkmcnt0();                        \
  if (grp) { WAIT; }                      \
  __builtin_amdgcn_sched_barrier(0);      \
  __builtin_amdgcn_s_barrier();           \
  __builtin_amdgcn_sched_barrier(0);      \
  compute();                              \
  if (!grp) { WAIT; }                     \
  __builtin_amdgcn_sched_barrier(0);      \
  __builtin_amdgcn_s_barrier();           \
  __builtin_amdgcn_sched_barrier(0);      \
  { WAIT; }
  using IC0 = std::integral_constant<int, 0>;
  constexpr int RA = 4 + NMBW;  // fragment reads per step
  // even step: each activation load followed by a share of the reads, then
  // the weight loads; odd step: weight load, half the reads, weight load, rest
#define PP_STEP_MID(I, XR, BR, XI, BI)                                              \
  {                                                                                 \
    const int k = st + (I);                                                         \
    if constexpr (((I) & 1) == 0) {                                                 \
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(cur.a_base, cur.a_bytes);         \
      const uint32_t kb = static_cast<uint32_t>(k + 2) * (kBK4 * 2);                \
      constexpr int P = (RA + NA - 1) / NA;                                         \
      dma16(ra, cur.aoff[0], kb, XI + (0 * 8 + wave) * 8 * (2 * kBK4));             \
      read_part(XR, (I) & 1, BR, IC0{}, std::integral_constant<int, (P < RA ? P : RA)>{}); \
      if constexpr (NA > 1) {                                                       \
        dma16(ra, cur.aoff[1], kb, XI + (1 * 8 + wave) * 8 * (2 * kBK4));           \
        read_part(XR, (I) & 1, BR, std::integral_constant<int, (P < RA ? P : RA)>{},  \
                  std::integral_constant<int, (2 * P < RA ? 2 * P : RA)>{});        \
      }                                                                             \
      if constexpr (NA > 2) {                                                       \
        dma16(ra, cur.aoff[2], kb, XI + (2 * 8 + wave) * 8 * (2 * kBK4));           \
        read_part(XR, (I) & 1, BR, std::integral_constant<int, (2 * P < RA ? 2 * P : RA)>{}, \
                  std::integral_constant<int, (3 * P < RA ? 3 * P : RA)>{});        \
      }                                                                             \
      if constexpr (NA > 3) {                                                       \
        dma16(ra, cur.aoff[3], kb, XI + (3 * 8 + wave) * 8 * (2 * kBK4));           \
      }                                                                             \
      read_part(XR, (I) & 1, BR, std::integral_constant<int, ((NA > 3 ? 3 : NA) * P < RA ? (NA > 3 ? 3 : NA) * P : RA)>{}, \
                std::integral_constant<int, RA>{});                                 \
      pp_issue_w(cur, k + 3, BI, wave, lane16);                                     \
      PP_PHASES_NOREAD(PP_WAIT_NA(0))                                               \
    } else {                                                                        \
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(cur.w_base, cur.w_bytes);         \
      const uint32_t kw = static_cast<uint32_t>(k + 3) * 1024u;                     \
      dma16(rb, lane16, cur.wrow0 + kw, BI + wave * kTileElems);                    \
      read_part(XR, (I) & 1, BR, IC0{}, std::integral_constant<int, RA / 2>{});     \
      dma16(rb, lane16, cur.wrow1 + kw, BI + (8 + wave) * kTileElems);              \
      read_part(XR, (I) & 1, BR, std::integral_constant<int, RA / 2>{}, std::integral_constant<int, RA>{}); \
      PP_PHASES_NOREAD(wait_vmcnt<4>())                                             \
    }                                                                               \
  }

  {  // step 0: the previous tile's stores may stay in flight
    pp_issue_a<NA>(cur, 2, X1, wave);
    pp_issue_w(cur, 3, B3, wave, lane16);
    PP_PHASES(0, X0, B0, PP_WAIT_NA(kPPStores<SWIGLU>))
  }
  int st = 0;
  PP_STEP_MID(1, X0, B1, X1, B0)
  PP_STEP_MID(2, X1, B2, X0, B1)
  PP_STEP_MID(3, X1, B3, X0, B2)
  for (st = 4; st < nk - 4; st += kStages) {
    PP_STEP_MID(0, X0, B0, X1, B3)
    PP_STEP_MID(1, X0, B1, X1, B0)
    PP_STEP_MID(2, X1, B2, X0, B1)
    PP_STEP_MID(3, X1, B3, X0, B2)
  }
  // The last four steps (st = nk - 4) load the next tile's first stages.
  // Without a next tile they issue the same loads over empty buffers (zeros
  // into buffers nothing reads any more), so the code is one straight line
  // whose loads in flight the compiler counts exactly.
  const PPTile tc = t;
  FfnGroup gn = pick_group(a, tc.grp);
  {  // k = nk - 4
    pp_issue_a<NA>(cur, st + 2, X1, wave);
    if (has_next) {
      t = pp_decode(a, tstart, sbeg, srows, nsegT, Ln);
      gn = pick_group(a, t.grp);
    } else {
      gn.row_index = nullptr;
      gn.a_bytes = 0u;
      gn.w_bytes = 0u;
    }
    pp_rows_issue_lds(gn, t, wave, lane, rslot);
    pp_issue_w(cur, st + 3, B3, wave, lane16);
    PP_PHASES(0, X0, B0, PP_WAIT_NA(1))
  }
  {  // k = nk - 3: the next tile's weights
    pp_wloads<SWIGLU>(gn, t, wave, cur);
    pp_issue_w(cur, 0, B0, wave, lane16);
    PP_PHASES(1, X0, B1, wait_vmcnt<5>())
  }
  {  // k = nk - 2: and its activations
    // the row_index load has landed once only W(nk-1) and W'(0) may be in
    // flight after it
    wait_vmcnt<4>();
    uint32_t raw[4];
    pp_rows_read_lds(rslot, lane, raw);
    pp_aloads(gn, t, wave, lane, raw, cur);
    pp_issue_a<4>(cur, 0, X0, wave);
    pp_issue_w(cur, 1, B1, wave, lane16);
    PP_PHASES(2, X1, B2, wait_vmcnt<8>())
  }
  {  // k = nk - 1
    pp_issue_w(cur, 2, B2, wave, lane16);
    PP_PHASES(3, X1, B3, wait_vmcnt<4>())
  }
#undef PP_STEP_MID
#undef PP_PHASES
#undef PP_PHASES_NOREAD
#undef PP_WAIT_NA

  const FfnGroup g = pick_group(a, tc.grp);
  // each group right after its last MFMA phase: group 0's stores overlap
  // group 1's last MFMAs, group 1's the next tile's first MFMAs of group 0
  // (the groups stage down tiles in the same four slots, one phase apart:
  // group 0's slot reads complete before the barrier that ends that phase).
  // With no next tile, group 0's extra barrier pairs with group 1's last one.
  if constexpr (SWIGLU) gate_up_epilogue<NMBW>(g, acc, wm, wn, tc.nt, tc.mrow0, tc.mv);
  else wave_staged_epilogue<NMBW>(g, acc, wm, wn, tc.nt, tc.mrow0, tc.mv, stage);
  if (!has_next && !grp) __builtin_amdgcn_s_barrier();
}

// Persistent ping-pong kernel over the tiles of both groups: rounds of
// gridDim.x tiles, inside a round XCD x takes the x-th run of gridDim.x / 8
// tiles (tiles sharing activation rows or weights in one L2), tile_nm order
// inside a segment.  The tiles of a workgroup form one stream of k-steps.
template <bool SWIGLU>
__global__ __launch_bounds__(kBigThreads, 1) void ffn_pp_kernel(FfnLaunch a) {
  constexpr int ROWS = kPPRows;
  constexpr int XE = ROWS * 2 * kBK4;  // activation buffer: two k-steps of 256 rows
  __shared__ __attribute__((aligned(16))) bf16_t X0s[XE];
  __shared__ __attribute__((aligned(16))) bf16_t X1s[XE];
  __shared__ __attribute__((aligned(16))) bf16_t B0s[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) bf16_t B1s[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) bf16_t B2s[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) bf16_t B3s[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) int32_t rslots[8 * 64];  // a 256-byte row_index slot per wave
  __shared__ __attribute__((aligned(16))) bf16_t stages[SWIGLU ? 8 : 4 * 1024];  // down: 2 KiB per wave of a group
  __shared__ int tstart[kMaxSegs + 1];
  __shared__ int sbeg[kMaxSegs];
  __shared__ int srows[kMaxSegs];
  __shared__ int tmp[kThreads];

  const int nsegT = a.g[0].nseg + (a.ngroups > 1 ? a.g[1].nseg : 0);
  for (int i = threadIdx.x; i < nsegT; i += kBigThreads) {
    const int gi = (a.ngroups > 1 && i >= a.g[0].nseg) ? 1 : 0;
    const FfnGroup gg = pick_group(a, gi);
    const int s = gi ? i - a.g[0].nseg : i;
    const int b = seg_begin(gg, s);
    sbeg[i] = b;
    srows[i] = seg_end(gg, s) - b;
  }
  if (threadIdx.x < kThreads) build_tile_starts<ROWS>(a, nsegT, tstart, tmp);
  else build_tile_starts_idle();
  const int total = tstart[nsegT];
  const int nxcd = 8;
  const int per = gridDim.x / nxcd;
  const int xcd = blockIdx.x % nxcd;
  const int slot = blockIdx.x / nxcd;
  int L = xcd * per + slot;
  if (L >= total) return;  // whole workgroup
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(static_cast<int>(threadIdx.x >> 6));
  const int grp = wave >> 2;
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
  int32_t* rslot = lds_opaque(rslots) + wave * 64;
  bf16_t* stage = lds_opaque(stages) + (SWIGLU ? 0 : (wave & 3) * 1024);
  bf16_t* X0 = lds_opaque(X0s);
  bf16_t* X1 = lds_opaque(X1s);
  bf16_t* B0 = lds_opaque(B0s);
  bf16_t* B1 = lds_opaque(B1s);
  bf16_t* B2 = lds_opaque(B2s);
  bf16_t* B3 = lds_opaque(B3s);

  PPTile t = pp_decode(a, tstart, sbeg, srows, nsegT, L);
  PPLoads cur;
  {
    const FfnGroup g = pick_group(a, t.grp);
    uint32_t raw[4];
    pp_rows_issue(g, t, wave, lane, raw);
    pp_wloads<SWIGLU>(g, t, wave, cur);
    pp_aloads(g, t, wave, lane, raw, cur);
  }
  // the first tile's first stages, in the order a previous tile issues them;
  // all but W(2) are waited for, so the first step's wait (which counts a
  // previous tile's stores) is met
  pp_issue_w(cur, 0, B0, wave, lane16);
  pp_issue_a<4>(cur, 0, X0, wave);
  pp_issue_w(cur, 1, B1, wave, lane16);
  pp_issue_w(cur, 2, B2, wave, lane16);
  wait_vmcnt<2>();
  __builtin_amdgcn_s_barrier();
  if (grp) __builtin_amdgcn_s_barrier();  // group 1 starts one phase later
  __builtin_amdgcn_sched_barrier(0);
  for (;;) {
    const int Ln = L + static_cast<int>(gridDim.x);
    switch (t.nmbw) {
#define PP_CASE(N)                                                                       \
  case N:                                                                                \
    pp_tile<N, SWIGLU>(a, tstart, sbeg, srows, nsegT, Ln, total, t, cur, X0, X1, B0, B1, \
                       B2, B3, rslot, stage);                                            \
    break;
      PP_CASE(8) PP_CASE(7) PP_CASE(6) PP_CASE(5) PP_CASE(4) PP_CASE(3) PP_CASE(2)
      default: PP_CASE(1)
#undef PP_CASE
    }
    if (Ln >= total) break;
    L = Ln;
  }
}

// Wave placement of a large-tile workgroup: wave w of workgroup g reads the
// number of the SIMD it runs on (bits 5:4 of the HW_ID hardware register)
// and the workgroup's first wave writes all eight to simd[8g .. 8g + 7].
// The ping-pong schedule's speed relies on waves w and w + 4 sharing a SIMD
// (its correctness does not: barriers order every access).  Same launch
// shape as ffn_pp_kernel, and like it enough LDS (its stage buffers) that
// one workgroup holds a CU.
constexpr int kPPLdsInts = (2 * kPPRows * 2 * kBK4 + kStages * kBuf4Elems) / 2;
__global__ __launch_bounds__(kBigThreads, 1) void wave_simd_kernel(int32_t* __restrict__ simd) {
  __shared__ int32_t ids[kPPLdsInts];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t hw_id = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);  // HW_REG_HW_ID
  constexpr int kStride = kPPLdsInts / 8;
  if (lane == 0) ids[wave * kStride] = static_cast<int32_t>((hw_id >> 4) & 3);
  __syncthreads();
  if (wave == 0 && lane < 8) simd[blockIdx.x * 8 + lane] = ids[lane * kStride];
}

hipError_t launch_wave_simd_probe(int32_t* simd, int n_workgroups, hipStream_t st) {
  if (n_workgroups <= 0) return hipSuccess;
  wave_simd_kernel<<<n_workgroups, kBigThreads, 0, st>>>(simd);
  return hipGetLastError();
}

static hipError_t launch_big(const FfnLaunch& fl, int phase, hipStream_t st);

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
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

static hipError_t launch_big(const FfnLaunch& fl, int phase, hipStream_t st) {
  long long ub = 0;
  for (int i = 0; i < fl.ngroups; ++i)
    ub += ((static_cast<long long>(fl.g[i].rows) + kBigRows - 1) / kBigRows + fl.g[i].nseg) *
          static_cast<long long>(fl.nt[i]);
  if (ub <= 0) return hipSuccess;
  long long grid = device_cus();
  const long long ub8 = (ub + 7) / 8 * 8;
  if (grid > ub8) grid = ub8;
  grid = (grid + 7) / 8 * 8;
  bool k128 = true;  // the ping-pong kernel: 4 k-steps of 32 per block, at least 2 blocks
  bool klong = true;
  for (int i = 0; i < fl.ngroups; ++i) {
    k128 = k128 && fl.g[i].K % 128 == 0 && fl.g[i].K >= 256;
    klong = klong && fl.g[i].K >= 1024;
  }
  // Measured (V3 prefill: gate/up K = 7168, down K = 2048; v1 and v2:
  // gate/up K = 2048, down K = 1408): every one of these phases runs faster
  // on the ping-pong kernel (v1 down 0.264 -> 0.238 ms, v2 down 0.331 ->
  // 0.306 ms).  A down phase with short K keeps the persistent 2-stage
  // kernel, which overlaps a tile's first loads with the previous tile.
  if (k128 && (phase == 0 || klong)) {
    if (phase == 0)
      ffn_pp_kernel<true><<<static_cast<int>(grid), kBigThreads, 0, st>>>(fl);
    else
      ffn_pp_kernel<false><<<static_cast<int>(grid), kBigThreads, 0, st>>>(fl);
    return hipGetLastError();
  }
  if (phase == 0)
    ffn_big_kernel<true><<<static_cast<int>(grid), kBigThreads, 0, st>>>(fl);
  else
    ffn_big_kernel<false><<<static_cast<int>(grid), kBigThreads, 0, st>>>(fl);
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
  bool big_ok = true;  // buffer addressing needs 32-bit byte offsets
  for (int i = 0; i < ngroups; ++i)
    big_ok = big_ok && groups[i].a_bytes != 0 && groups[i].w_bytes != 0 && groups[i].o_bytes != 0;
  if (rows_hint >= 128 && big_ok) return launch_big(fl, phase, st);
  if (rows_hint >= 128) return launch_mb<kBigMB, kBigPF>(fl, phase, kMinBlocks, st);
  if (rows_hint >= 32) return launch_mb<kMidMB, kMidPF>(fl, phase, 2, st);
  return launch_mb<1, kSmallPF>(fl, phase, kSmallBlocksPerCU, st);
}

// ================================================================ weight packing
// Row-major [n_mat][R][K] -> tiled: 16-row x 32-k blocks of 1 KiB, the blocks
// of a 16-row group consecutive in k, inside a block lane l's fragment (row
// l % 16, k-chunk l / 16 of 8 elements) at the l-th 16 bytes.  One 16-byte
// chunk per thread and iteration.
__global__ __launch_bounds__(256) void pack_tiled_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n_chunks,
                                                         int R, int K) {
  const int64_t kc = K / 8;       // 16-byte chunks per row
  const int64_t kbn = K / 32;     // k-blocks per 16-row group
  const int64_t per_mat = static_cast<int64_t>(R) * kc;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n_chunks;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t mat = idx / per_mat;
    const int64_t rem = idx - mat * per_mat;
    const int64_t blk = rem / 64;
    const int l = static_cast<int>(rem - blk * 64);
    const int64_t rb = blk / kbn;
    const int64_t kb = blk - rb * kbn;
    const int64_t row = rb * 16 + (l & 15);
    dst[idx] = src[mat * per_mat + row * kc + kb * 4 + (l >> 4)];
  }
}

hipError_t launch_pack_tiled(const void* src, void* dst, int64_t n_mat, int R, int K,
                             hipStream_t st) {
  const int64_t n_chunks = n_mat * R * static_cast<int64_t>(K) / 8;
  if (n_chunks <= 0) return hipSuccess;
  int64_t blocks = (n_chunks + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  pack_tiled_kernel<<<static_cast<int>(blocks), 256, 0, st>>>(static_cast<const u32x4*>(src),
                                                               static_cast<u32x4*>(dst), n_chunks,
                                                               R, K);
  return hipGetLastError();
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
