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
#include "moe_internal.h"
#include "lds_dma.h"

namespace moe {

// Tile configuration of the three tile families (rows per tile = 16 * MB,
// weight fragments prefetched PF steps ahead); overridable at build time.
#ifndef MOE_FFN_BIG_MB
#define MOE_FFN_BIG_MB 8
#endif
#ifndef MOE_FFN_BIG_PF
#define MOE_FFN_BIG_PF 1
#endif
#ifndef MOE_FFN_MID_MB
#define MOE_FFN_MID_MB 4
#endif
#ifndef MOE_FFN_MID_PF
#define MOE_FFN_MID_PF 2
#endif
#ifndef MOE_FFN_SMALL_PF
#define MOE_FFN_SMALL_PF 4
#endif

#ifndef MOE_FFN_SMALL_BPC
#define MOE_FFN_SMALL_BPC 2  // workgroups per CU of the small-segment launch
#endif
#ifndef MOE_FFN_MINBLK
#define MOE_FFN_MINBLK 2
#endif

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
__global__ __launch_bounds__(kThreads, MOE_FFN_MINBLK) void ffn_bf16_kernel(FfnLaunch a) {
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
// One workgroup per CU computes a 256-row x 256-weight-row tile with 4 waves
// in a 2x2 layout.  Both operands stream global -> LDS with gfx950's direct
// loads (global_load_lds_dwordx4), double buffered, so no registers stage
// them; each wave then reads 16-byte MFMA fragments from LDS.  A wave owns
// the 8 M-blocks of one parity (blocks 2j + wm), so a tile with fewer rows
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

// SwiGLU of a gate/up accumulator pair, rounded to bf16 and packed: two h
// columns per 32-bit word (lower column in the low half)
__device__ __forceinline__ uint32_t swiglu_pack(float g0, float g1, float u0, float u1) {
  const float h0 = g0 / (1.0f + __expf(-g0)) * u0;
  const float h1 = g1 / (1.0f + __expf(-g1)) * u1;
  return pack_bf16x2(h0, h1);
}

// Gate/up tile epilogue straight from registers: per M-block and lane, h of
// 4 consecutive columns of one row (8 bytes) for each of the wave's two
// 16-column blocks; rows past mv and columns past n_out are not stored.
template <int NJ>
__device__ __forceinline__ void gate_up_epilogue(const FfnGroup& g, const f32x4 (&acc)[NJ][4],
                                                 int nmbw, int wm, int wn, int nt, int mrow0,
                                                 int mv) {
  const int lane = threadIdx.x & 63;
  bf16_t* Out = static_cast<bf16_t*>(g.Out);
  const int rl = lane & 15;
  const int cq = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j < nmbw) {
      const int r = (2 * j + wm) * 16 + rl;
      if (r < mv) {
        bf16_t* orow = Out + static_cast<int64_t>(mrow0 + r) * g.ldo;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = nt * 128 + wn * 32 + nb * 16 + cq;
          if (col < g.n_out)
            *reinterpret_cast<u32x2*>(orow + col) =
                u32x2{swiglu_pack(acc[j][nb][0], acc[j][nb][1], acc[j][nb + 2][0], acc[j][nb + 2][1]),
                      swiglu_pack(acc[j][nb][2], acc[j][nb][3], acc[j][nb + 2][2], acc[j][nb + 2][3])};
        }
      }
    }
  }
}

// Down tile epilogue through LDS, so the outputs leave as whole rows.  Pass
// p covers M-block p of both wave rows (tile rows 32p .. 32p + 31): every
// wave writes its accumulators for those rows, rounded to bf16, into a
// staging buffer; after a barrier each wave reads whole 1 KiB pieces of the
// buffer and stores them, so a store instruction writes two whole 512-byte
// rows (8 complete 128-byte lines) instead of 32-byte pieces of 16 rows, a
// quarter of the write requests.  The 16-byte chunk c of staged row r sits
// at position c ^ (r % 32), so the 8-byte writes of 16 rows and the row
// reads touch distinct LDS banks.  The two staging buffers (16 KiB each,
// free when this is called) alternate, so one barrier per pass orders the
// writes before the reads, and the reads of pass p before the writes of
// pass p + 2 (each wave's reads complete before its stores issue, which
// precede its arrival at the next barrier).  Rows past mv and columns past
// n_out are not stored (n_out is a multiple of 8).
template <int NJ>
__device__ __forceinline__ void staged_epilogue(const FfnGroup& g, const f32x4 (&acc)[NJ][4],
                                                int nmbw, int wm, int wn, int nt, int mrow0,
                                                int mv, bf16_t* S0, bf16_t* S1) {
  constexpr int COLS = 256;                 // output columns of a tile
  constexpr int RB = COLS * 2;              // bytes of a staged row
  constexpr int CPR = RB / 16;              // 16-byte chunks per staged row
  constexpr int NI = 32 * RB / 1024;        // 1 KiB pieces per pass
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(static_cast<int>(threadIdx.x >> 6));
  const int rloc = wm * 16 + (lane & 15);   // staged row of this lane's accumulators
  const int q = lane >> 4;                  // 4-column group inside a 16-column block
  bf16_t* Out = static_cast<bf16_t*>(g.Out);
#pragma unroll
  for (int p = 0; p < NJ; ++p) {
    if (p < nmbw) {  // tile-uniform
      char* S = reinterpret_cast<char*>(p & 1 ? S1 : S0);
      char* srow = S + rloc * RB;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = wn * 64 + nb * 16 + q * 4;
        const uint32_t w0 = pack_bf16x2(acc[p][nb][0], acc[p][nb][1]);
        const uint32_t w1 = pack_bf16x2(acc[p][nb][2], acc[p][nb][3]);
        *reinterpret_cast<u32x2*>(srow + (((col >> 3) ^ (rloc % CPR)) << 4) + ((col >> 2) & 1) * 8) =
            u32x2{w0, w1};
      }
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int i0 = 0; i0 < NI; i0 += 8) {
        const int off = (i0 + wave) * 1024 + lane * 16;
        const int r = off / RB;
        const int c = (off % RB) >> 4;
        const u32x4 v = *reinterpret_cast<const u32x4*>(S + r * RB + ((c ^ (r % CPR)) << 4));
        const int row = 32 * p + r;
        const int col = nt * COLS + c * 8;
        if (row < mv && col < g.n_out)
          *reinterpret_cast<u32x4*>(Out + static_cast<int64_t>(mrow0 + row) * g.ldo + col) = v;
      }
    }
  }
}

// Tiles run back to back: the first stage of the next tile is loaded during
// the last step of the current one, before the current tile's stores, so the
// next tile's first wait skips those stores (vmcnt retires in issue order)
// and no tile starts with an empty pipeline.
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
    const int wr = (SWIGLU && q >= 8) ? g.up_off + col0 + 16 * (q - 8) : col0 + 16 * q;
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
// with no LDS waits between its MFMAs.  Gate/up tiles store h straight from
// registers, group 0 while group 1 runs the last MFMAs; down tiles (256
// output columns) go through the staged epilogue.
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

// wait until at most N vector-memory instructions of this wave are
// outstanding; N < 0: no wait
template <int N>
__device__ __forceinline__ void pp_wait_n() {
  if constexpr (N >= 0) wait_vmcnt<N>();
}

// One tile of the ping-pong kernel; the activations of k-steps 2i and
// 2i + 1 arrive together as 128-byte rows in buffer X0 (i even) or X1
// (i odd).
template <int NMBW, bool SWIGLU>
__device__ __noinline__ void pp_tile(const FfnGroup& g, int s, int nt, int mrow0, int mv,
                                     bf16_t* X0, bf16_t* X1, bf16_t* B0, bf16_t* B1, bf16_t* B2,
                                     bf16_t* B3) {
  static_assert(NMBW >= 1 && NMBW <= 8, "tiles hold at most 256 rows");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int K = wave_uniform(g.K);
  const int nk = K / kBK4;  // multiple of 4

  // Activation loads: 8 rows x 128 bytes per wave instruction; row group
  // q = p*8 + wave covers tile rows [8q, 8q+8); lane -> row 8q + lane/8,
  // physical chunk lane%8, logical chunk (lane%8) ^ ((row >> 1) & 7), and
  // (row >> 1) & 7 = 4*(wave & 1) + lane/16 for every p.  Rows past the
  // tile's valid ones read from past the buffer's end, which returns zeros
  // without a memory request (their results are never stored; a buffer
  // within 256 MiB of 4 GiB repeats the last valid row instead, so that no
  // offset wraps); groups past the tile's height are not loaded.
  const int logical = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(
      static_cast<const bf16_t*>(g.W) + static_cast<int64_t>(s) * g.w_stride, g.w_bytes);
  constexpr int G8 = 4 * NMBW;  // row groups of 8 the tile loads
  constexpr int NAG = (G8 + 7) / 8;
  const bool zero_pad = g.a_bytes <= 0xF0000000u;
  uint32_t aoff[NAG];
#pragma unroll
  for (int p = 0; p < NAG; ++p) {
    const int row = (p * 8 + wave) * 8 + (lane >> 3);
    if (row < mv || !zero_pad) {
      int prow = mrow0 + min(row, mv - 1);
      if (g.row_index) prow = g.row_index[prow];
      aoff[p] = static_cast<uint32_t>(prow) * static_cast<uint32_t>(g.lda) * 2u + logical * 16;
    } else {
      aoff[p] = g.a_bytes;
    }
  }
  // Weights, tiled: the wave copies the KiB of k-block `step` of row blocks
  // `wave` and 8 + `wave` (gate/up: the gate and the up block of the same
  // columns) into LDS slots `wave` and 8 + `wave`, in fragment order.
  const uint32_t krow_bytes = static_cast<uint32_t>(K) * 2u;
  const uint32_t boff =
      static_cast<uint32_t>((SWIGLU ? nt * 128 : nt * 256) + wave * 16) * krow_bytes + lane * 16u;
  const uint32_t bsoff1 = static_cast<uint32_t>(SWIGLU ? g.up_off : 128) * krow_bytes;

  // k-steps step, step + 1 (step even)
  auto issue_a = [&](int step, bf16_t* Xb) {
    const uint32_t kb = static_cast<uint32_t>(step) * (kBK4 * 2);
#pragma unroll
    for (int p = 0; p < NAG; ++p)
      if (p * 8 + wave < G8) dma16(ra, aoff[p], kb, Xb + (p * 8 + wave) * 8 * (2 * kBK4));
  };
  auto issue_w = [&](int step, bf16_t* Bb) {
    const uint32_t kw = static_cast<uint32_t>(step) * 1024u;
    dma16(rb, boff, kw, Bb + wave * kTileElems);
    dma16(rb, boff, bsoff1 + kw, Bb + (8 + wave) * kTileElems);
  };
  // activation loads of this wave per pair of k-steps: NA0, one more with
  // `extra`
  constexpr int NA0 = G8 / 8;
  const bool extra = wave < (G8 % 8);

  // a whole k-step's fragments: M-blocks 2j + wm (j < NMBW), weight blocks
  // of columns 32wn .. 32wn + 31 (gate and up); row 16*block + lane%16 has
  // swizzle term (lane%16) >> 1
  const int swz = (lane & 15) >> 1;
  const int arow = (wm * 16 + (lane & 15)) * (2 * kBK4);
  bf16x8 af[NMBW], bf[4];
  auto read = [&](const bf16_t* Xb, int half, const bf16_t* Bb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bf[nb] = as_bf16x8(
          *reinterpret_cast<const u32x4*>(Bb + lane * 8 + big_wblock<SWIGLU>(wn, nb) * kTileElems));
    const bf16_t* abase = Xb + arow + (((half * 4 + (lane >> 4)) ^ swz) * 8);
#pragma unroll
    for (int j = 0; j < NMBW; ++j)
      af[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + j * 32 * (2 * kBK4)));
  };

  f32x4 acc[NMBW][4];
#pragma unroll
  for (int j = 0; j < NMBW; ++j)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&]() {
#pragma unroll
    for (int j = 0; j < NMBW; ++j)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[nb], af[j], acc[j][nb], 0, 0, 0);
  };

  // prologue: A(0,1) W0 W1 A(2,3) W2 W3; k-step 0 needs A(0,1) and W0
  issue_a(0, X0);
  issue_w(0, B0);
  issue_w(1, B1);
  issue_a(2, X1);
  issue_w(2, B2);
  issue_w(3, B3);
  if (extra) wait_vmcnt<6 + NA0 + 1>();
  else wait_vmcnt<6 + NA0>();
  __builtin_amdgcn_s_barrier();
  if (grp) __builtin_amdgcn_s_barrier();  // group 1 starts one phase later
  __builtin_amdgcn_sched_barrier(0);
  // k-step k reads stage k in phase 2k (group 0) or 2k + 1 (group 1) and
  // computes it in the phase after.  At the start of its read phase a wave
  // issues W(k + 3) into the weight buffer of k - 1 and, for even k, first
  // A(k + 2, k + 3) into the activation buffer of k - 2 and k - 1; both
  // groups read k - 1 by phase 2k - 1.  Before the barrier that closes phase
  // 2k + 1 every wave waits for its own loads of stage k + 1.  Even k:
  // W(k + 1), then W(k + 2), A(k + 2, k + 3) and W(k + 3) may stay
  // outstanding.  Odd k: A(k + 1, k + 2) (after W(k + 1)), then W(k + 2) and
  // W(k + 3) may.  In the last four k-steps nothing is issued after k = nk - 4,
  // so fewer stay outstanding.  The LDS reads of a read phase are complete
  // (lgkmcnt 0) before its barrier.
#define PP_WAIT(I)                                                     \
  if (last) {                                                          \
    if constexpr ((I) == 0) {                                          \
      if (extra) pp_wait_n<4 + NA0 + 1>();                             \
      else pp_wait_n<4 + NA0>();                                       \
    } else if constexpr ((I) == 1) {                                   \
      pp_wait_n<2>();                                                  \
    } else if constexpr ((I) == 2) {                                   \
      pp_wait_n<0>();                                                  \
    }                                                                  \
  } else if constexpr (((I) & 1) == 0) {                               \
    if (extra) pp_wait_n<4 + NA0 + 1>();                               \
    else pp_wait_n<4 + NA0>();                                         \
  } else {                                                             \
    pp_wait_n<4>();                                                    \
  }
#define PP_STEP(I, XR, BR, XI, BI)              \
  {                                             \
    const int k = st + (I);                     \
    if (k >= 1 && k + 3 < nk) {                 \
      if (((I) & 1) == 0) issue_a(k + 2, XI);   \
      issue_w(k + 3, BI);                       \
    }                                           \
    read(XR, (I) & 1, BR);                      \
    wait_lgkmcnt0();                            \
    if (grp) { PP_WAIT(I) }                     \
    __builtin_amdgcn_sched_barrier(0);          \
    __builtin_amdgcn_s_barrier();               \
    __builtin_amdgcn_sched_barrier(0);          \
    compute();                                  \
    if (!grp) { PP_WAIT(I) }                    \
    __builtin_amdgcn_sched_barrier(0);          \
    __builtin_amdgcn_s_barrier();               \
    __builtin_amdgcn_sched_barrier(0);          \
  }
  for (int st = 0; st < nk; st += kStages) {
    const bool last = st + kStages >= nk;  // the last four k-steps
    PP_STEP(0, X0, B0, X1, B3)
    PP_STEP(1, X0, B1, X1, B0)
    PP_STEP(2, X1, B2, X0, B1)
    PP_STEP(3, X1, B3, X0, B2)
  }
#undef PP_STEP
#undef PP_WAIT
  // Group 0's extra barrier pairs with group 1's last one, so both groups
  // pass the same number of barriers per tile.
  if constexpr (SWIGLU) {
    // group 0 stores h while group 1 runs the last MFMAs; no LDS is read
    // after the extra barrier, so the next tile's loads need no other one
    gate_up_epilogue<NMBW>(g, acc, NMBW, wm, wn, nt, mrow0, mv);
    if (!grp) __builtin_amdgcn_s_barrier();
  } else {
    // staging in B1/B2: every read phase ended with lgkmcnt(0) before its
    // barrier (group 1's last one closes phase 2nk - 1) and every load was
    // waited for, so both buffers are free
    if (!grp) __builtin_amdgcn_s_barrier();
    staged_epilogue<NMBW>(g, acc, NMBW, wm, wn, nt, mrow0, mv, B1, B2);
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();  // staging reads done before the next tile's loads
  }
}

// pp_tile for the instantiated height covering nmbw M-blocks per wave
template <int N, bool SWIGLU>
__device__ __forceinline__ void pp_dispatch(int nmbw, const FfnGroup& g, int s, int nt, int mrow0,
                                            int mv, bf16_t* X0, bf16_t* X1, bf16_t* B0,
                                            bf16_t* B1, bf16_t* B2, bf16_t* B3) {
  if constexpr (N > 1) {
    if (nmbw >= N) {
      pp_tile<N, SWIGLU>(g, s, nt, mrow0, mv, X0, X1, B0, B1, B2, B3);
      return;
    }
    pp_dispatch<N - 1, SWIGLU>(nmbw, g, s, nt, mrow0, mv, X0, X1, B0, B1, B2, B3);
  } else {
    pp_tile<1, SWIGLU>(g, s, nt, mrow0, mv, X0, X1, B0, B1, B2, B3);
  }
}

// Persistent ping-pong kernel over the tiles of both groups: rounds of
// gridDim.x tiles, inside a round XCD x takes the x-th run of gridDim.x / 8
// tiles (tiles sharing activation rows or weights in one L2), tile_nm order
// inside a segment.
template <bool SWIGLU>
__global__ __launch_bounds__(kBigThreads, 1) void ffn_pp_kernel(FfnLaunch a) {
  constexpr int ROWS = kPPRows;
  __shared__ __attribute__((aligned(16))) bf16_t X0[ROWS * 2 * kBK4];
  __shared__ __attribute__((aligned(16))) bf16_t X1[ROWS * 2 * kBK4];
  __shared__ __attribute__((aligned(16))) bf16_t B0[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) bf16_t B1[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) bf16_t B2[kBuf4Elems];
  __shared__ __attribute__((aligned(16))) bf16_t B3[kBuf4Elems];
  __shared__ int tstart[kMaxSegs + 1];
  __shared__ int tmp[kThreads];

  const int nsegT = a.g[0].nseg + (a.ngroups > 1 ? a.g[1].nseg : 0);
  if (threadIdx.x < kThreads) build_tile_starts<ROWS>(a, nsegT, tstart, tmp);
  else build_tile_starts_idle();
  const int total = tstart[nsegT];
  const int nxcd = 8;
  const int per = gridDim.x / nxcd;
  const int xcd = blockIdx.x % nxcd;
  const int slot = blockIdx.x / nxcd;
  for (int L = xcd * per + slot; L < total; L += gridDim.x) {
    int i0 = 0, i1 = nsegT;
    while (i1 - i0 > 1) {
      const int mid = (i0 + i1) >> 1;
      if (tstart[mid] <= L) i0 = mid;
      else i1 = mid;
    }
    const int grp = (a.ngroups > 1 && i0 >= a.g[0].nseg) ? 1 : 0;
    const FfnGroup g = grp ? a.g[1] : a.g[0];
    const int s = grp ? i0 - a.g[0].nseg : i0;
    const int r0 = seg_begin(g, s);
    const int rows = seg_end(g, s) - r0;
    const int mtc = (rows + ROWS - 1) / ROWS;
    const int rpt = ((rows + mtc - 1) / mtc + 15) & ~15;
    const int local = L - tstart[i0];
    int nt, mt;
    tile_nm(local, mtc, grp ? a.nt[1] : a.nt[0], nt, mt);
    const int mrow0 = r0 + mt * rpt;
    const int mv = min(rpt, rows - mt * rpt);
    const int nmbw = (((mv + 15) >> 4) + 1) >> 1;
    pp_dispatch<ROWS / 32, SWIGLU>(nmbw, g, s, nt, mrow0, mv, X0, X1, B0, B1, B2, B3);
  }
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
  bool k128 = true;  // the ping-pong kernel consumes 4 k-steps of 32 per iteration
  bool klong = true;
  for (int i = 0; i < fl.ngroups; ++i) {
    k128 = k128 && fl.g[i].K % 128 == 0;
    klong = klong && fl.g[i].K >= 1024;
  }
#ifndef MOE_FFN_NO_PP
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
#endif
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
#ifndef MOE_FFN_NO_BIG
  bool big_ok = true;  // buffer addressing needs 32-bit byte offsets
  for (int i = 0; i < ngroups; ++i)
    big_ok = big_ok && groups[i].a_bytes != 0 && groups[i].w_bytes != 0 && groups[i].o_bytes != 0;
  if (rows_hint >= 128 && big_ok) return launch_big(fl, phase, st);
#endif
  if (rows_hint >= 128) return launch_mb<MOE_FFN_BIG_MB, MOE_FFN_BIG_PF>(fl, phase, MOE_FFN_MINBLK, st);
  if (rows_hint >= 32) return launch_mb<MOE_FFN_MID_MB, MOE_FFN_MID_PF>(fl, phase, 2, st);
  return launch_mb<1, MOE_FFN_SMALL_PF>(fl, phase, MOE_FFN_SMALL_BPC, st);
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
