// route.hip -- router GEMM (bf16 MFMA over exact bf16 pieces of the fp32
// weight, or fp32 MFMA) and per-token scoring, group-limited
// top-k and gates (one wavefront per token).
//
// Sources: "DeepSeek MoE：从v1到v3的演进" §DeepSeek-v3 (sigmoid score, bias
// used for selection only, gate from the unbiased score) and §ST-MoE (z-loss
// log-sum-exp); "DeepSeek-V3的Group-Limited Expert Routing与负载均衡优化实践"
// §1 and §3 (score the groups, keep the best ones, mask the rest, choose the
// top-k experts); "DeepSeek-V3技术解密…" §四.2 (router kept in fp32).
#include "moe_internal.h"
#include "lds_dma.h"

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

// ============================================================ router GEMM, bf16 MFMA
// An fp32 weight w is written as three bf16 pieces with w = hi + mid + lo
// exactly: hi is w with its low 16 bits cleared, mid the same of r = w - hi,
// lo = r - mid.  Both differences are exact in fp32 (Sterbenz: the operands
// share a sign and lie within a factor of two), r keeps at most the 16
// significand bits below hi's 8, and what mid leaves fits lo's 8 bits, so
// the pieces hold all 24 bits of w (for |w| >= 2^-103 or w = 0; smaller
// magnitudes would need subnormal pieces).  A bf16 x bf16 product is exact in
// fp32, so accumulating x*hi + x*mid + x*lo in fp32 gives the fp32-accumulated
// dot product of x with the full fp32 weight -- only the order of the fp32
// additions differs from a plain fp32 GEMM -- at the bf16 MFMA rate.
//
// Piece layout (tiled, as the grouped GEMM's weights): piece p is an
// [npad][H] bf16 matrix at p*npad*H; block (i, j) of 16 rows x 32 columns is
// the 512 elements at (i*(H/32) + j)*512, chunk l (8 elements) of a block is
// row 16i + l%16, columns 32j + 8(l/16) .. +7: a wave's MFMA operand for 16
// experts x 32 k is one contiguous KiB.

__device__ __forceinline__ uint32_t bf16_hi_bits(float v) { return __float_as_uint(v) >> 16; }

// One thread per 8-element chunk: block (i, j) = (id/64) split over
// npad/16 x H/32 blocks, chunk l = id % 64.
template <typename WT>
__global__ __launch_bounds__(256) void router_pieces_kernel(const WT* __restrict__ wg,
                                                            bf16_t* __restrict__ pieces, int N,
                                                            int npad, int H) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int kb = H / 32;
  const int64_t nchunks = static_cast<int64_t>(npad) * (H / 8);
  if (id >= nchunks) return;
  const int64_t blk = id >> 6;
  const int l = static_cast<int>(id & 63);
  const int i = static_cast<int>(blk / kb), j = static_cast<int>(blk % kb);
  const int r = 16 * i + (l & 15);
  const int c0 = 32 * j + 8 * (l >> 4);
  float w[8];
  if (r < N) {
    const WT* src = wg + static_cast<int64_t>(r) * H + c0;
    if constexpr (sizeof(WT) == 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[2 * e] = __uint_as_float(q[e] << 16);
        w[2 * e + 1] = __uint_as_float(q[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = 0.0f;
  }
  const int64_t off = blk * 512 + l * 8;
  const int64_t pstride = static_cast<int64_t>(npad) * H;
  uint32_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t h2[2], m2[2], l2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float v = w[2 * e + u];
      h2[u] = bf16_hi_bits(v);
      const float rr = v - __uint_as_float(h2[u] << 16);
      m2[u] = bf16_hi_bits(rr);
      l2[u] = bf16_hi_bits(rr - __uint_as_float(m2[u] << 16));
    }
    hi[e] = h2[0] | (h2[1] << 16);
    mid[e] = m2[0] | (m2[1] << 16);
    lo[e] = l2[0] | (l2[1] << 16);
  }
  *reinterpret_cast<u32x4*>(pieces + off) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  if constexpr (sizeof(WT) == 4) {
    *reinterpret_cast<u32x4*>(pieces + pstride + off) = u32x4{mid[0], mid[1], mid[2], mid[3]};
    *reinterpret_cast<u32x4*>(pieces + 2 * pstride + off) = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }
}

// GEMM: a workgroup of 8 waves owns 256 tokens x 256 experts of one K split;
// wave (wm, wn) = (wave & 1, wave >> 1) owns token blocks 2j + wm (j < 8) and
// expert blocks 4wn .. 4wn+3 (16 x 16 each).  k-steps of 32 in two LDS
// stages, both operands loaded global -> LDS directly:
//   tokens: 256 rows x 64 B per step, 16-byte chunks XOR-swizzled by row
//           pairs (physical chunk = logical ^ ((row >> 1) & 3));
//   pieces: np x 16 expert blocks of 1 KiB per step, already in fragment
//           order.
// Ping-pong schedule: waves 0-3 (expert blocks 0-7, group 0) and waves 4-7
// (blocks 8-15, group 1; the dispatcher puts waves w and w + 4 on one SIMD)
// run half a k-step apart.  In every phase (closed by a workgroup barrier)
// one group reads a k-step's fragments from LDS while the other issues that
// k-step's 32 np MFMAs back to back, so each matrix core is fed by one wave
// at a time with no LDS waits between its MFMAs.  Group 0 issues all of the
// next stage's loads at the start of its read phase, into the stage both
// groups finished reading by the barrier before, and waits for them after
// its MFMA phase, before the barrier after which it reads them (group 1
// reads them one phase later); group 1 issues no loads.
// MFMA operands are (weights, tokens), so a lane's accumulator holds four
// consecutive experts of one token: 16-byte partial stores, group 0's while
// group 1 issues its last MFMAs.
constexpr int kRtRows = 256;
constexpr int kRtThreads = 512;
constexpr int kRtAElems = kRtRows * 32;  // one stage of token rows
constexpr int kRtBElems = 16 * 512;      // one stage of one piece (256 experts)

template <int NP>
__global__ __launch_bounds__(kRtThreads, 1) void router_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ pieces, float* __restrict__ part,
    int T, int H, int N, int npad, int ksteps) {
  // one array per stage: the compiler then sees that the direct loads into
  // one stage do not alias the fragment reads of the other, and does not
  // wait for them before reading
  __shared__ __attribute__((aligned(16))) bf16_t A0[kRtAElems];
  __shared__ __attribute__((aligned(16))) bf16_t A1[kRtAElems];
  __shared__ __attribute__((aligned(16))) bf16_t B0[NP * kRtBElems];
  __shared__ __attribute__((aligned(16))) bf16_t B1[NP * kRtBElems];
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(static_cast<int>(threadIdx.x >> 6));
  const int grp = wave >> 2;
  const int gw = wave & 3;  // wave within its group
  const int wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * kRtRows;
  const int eb = blockIdx.y * 16;  // first expert block of the tile
  const int nkb = H / 32;
  const int k0 = blockIdx.z * ksteps;
  const int k1 = min(nkb, k0 + ksteps);
  const int nblk = npad / 16;

  // group 0's loads: token row groups q*4 + gw (16 rows, 1 KiB; lane ->
  // row 16 g + lane/4, chunk lane%4), piece blocks b = q*4 + gw (piece b/16,
  // expert block b%16)
  const int rows = min(kRtRows, T - t0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(
      x + static_cast<int64_t>(t0) * H, static_cast<uint32_t>(rows) * static_cast<uint32_t>(H) * 2u);
  const int logical = (lane & 3) ^ ((lane >> 3) & 3);
  uint32_t aoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (q * 4 + gw) * 16 + (lane >> 2);
    aoff[q] = static_cast<uint32_t>(row) * static_cast<uint32_t>(H) * 2u + logical * 16u;
  }
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(pieces, static_cast<uint32_t>(NP) * static_cast<uint32_t>(npad) *
                            static_cast<uint32_t>(H) * 2u);
  const uint32_t pbytes = static_cast<uint32_t>(npad) * static_cast<uint32_t>(H) * 2u;

  auto issue = [&](int kb, bf16_t* Ab, bf16_t* Bb) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dma16(rx, aoff[q], static_cast<uint32_t>(kb) * 64u, Ab + (q * 4 + gw) * 512);
#pragma unroll
    for (int q = 0; q < 4 * NP; ++q) {
      const int b = q * 4 + gw;
      const int blk = eb + (b & 15);
      if (blk < nblk)  // wave-uniform
        dma16(rw, lane * 16u,
              static_cast<uint32_t>(b >> 4) * pbytes +
                  (static_cast<uint32_t>(blk) * nkb + kb) * 1024u,
              Bb + b * 512);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool active = eb + 4 * wn < nblk;  // wave-uniform: some expert of this wave exists

  // fragment addresses: token row 16*blk + lane%16, logical chunk lane/16
  const int ch = (lane >> 4) ^ (((lane & 15) >> 1) & 3);
  const int aread = (wm * 16 + (lane & 15)) * 32 + ch * 8;
  const int bread = (4 * wn) * 512 + lane * 8;
  bf16x8 af[8], bf[NP][4];
  auto read = [&](const bf16_t* Ab, const bf16_t* Bb) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bf[p][nb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Bb + p * kRtBElems + bread + nb * 512));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      af[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Ab + aread + j * 32 * 32));
  };
  auto mfma = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int p = NP - 1; p >= 0; --p)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[p][nb], af[j], acc[j][nb], 0, 0, 0);
  };
  // step kb reads (Ac, Bc); group 0 first issues step kb + 1 into (An, Bn)
  auto step = [&](int kb, const bf16_t* Ac, const bf16_t* Bc, bf16_t* An, bf16_t* Bn) {
    if (grp == 0 && kb + 1 < k1) issue(kb + 1, An, Bn);
    if (active) read(Ac, Bc);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (active) mfma();
    if (grp == 0) wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  if (grp == 0) {
    issue(k0, A0, B0);
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  if (grp) __builtin_amdgcn_s_barrier();  // group 1 starts one phase later
  for (int kb = k0; kb < k1; kb += 2) {
    step(kb, A0, B0, A1, B1);
    if (kb + 1 < k1) step(kb + 1, A1, B1, A0, B0);
  }
  // D layout: lane holds experts 4*(lane/16) .. +3 of token lane%16
  if (active) {
    float* out = part + static_cast<int64_t>(blockIdx.z) * T * N;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + (2 * j + wm) * 16 + (lane & 15);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int e = (eb + 4 * wn + nb) * 16 + 4 * (lane >> 4);
        if (t < T && e < N) *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(t) * N + e) = acc[j][nb];
      }
    }
  }
  // group 0's extra barrier pairs with group 1's last one
  if (grp == 0) __builtin_amdgcn_s_barrier();
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

RouterPlan router_plan(int T, int H, int N, int x_dtype, int wg_dtype) {
  RouterPlan rp{};
  rp.np = wg_dtype == MOE_F32 ? 3 : 1;
  rp.npad = (N + 15) / 16 * 16;
  rp.bf16 = (x_dtype == MOE_BF16 && H % 32 == 0 && T > 0) ? 1 : 0;
  if (rp.bf16) {
    const int nkb = H / 32;
    const int tiles = ((T + kRtRows - 1) / kRtRows) * ((N + 255) / 256);
    int s = (256 + tiles - 1) / tiles;            // about one workgroup per CU
    const int smax = nkb / 4 > 1 ? nkb / 4 : 1;   // at least 4 k-steps per split
    s = s < 1 ? 1 : (s > smax ? smax : s);
    const int ks = (nkb + s - 1) / s;
    rp.splits = (nkb + ks - 1) / ks;              // no empty split
    rp.kchunk = ks * 32;
  } else {
    const int tiles = ((T + 31) / 32) * ((N + 255) / 256);
    int s = tiles > 0 ? (1024 + tiles - 1) / tiles : 1;
    const int smax = H / 64 < 32 ? H / 64 : 32;
    s = s > smax ? smax : s;
    rp.splits = s < 1 ? 1 : s;
    rp.kchunk = ((H + rp.splits - 1) / rp.splits + 15) / 16 * 16;
  }
  rp.part_bytes = rp.splits > 1 ? static_cast<size_t>(rp.splits) * T * N * 4 : 0;
  rp.piece_off = align256(rp.part_bytes);
  rp.ws_bytes = rp.piece_off + (rp.bf16 ? static_cast<size_t>(rp.np) * rp.npad * H * 2 : 0);
  return rp;
}

hipError_t launch_router_gemm(const RouterPlan& rp, const void* x, int x_dtype, const void* wg,
                              int wg_dtype, float* logits, void* ws, int T, int H, int N,
                              const float** part_out, hipStream_t st) {
  float* part = rp.splits > 1 ? static_cast<float*>(ws) : logits;
  *part_out = part;
  if (T == 0) return hipSuccess;
  if (rp.bf16) {
    bf16_t* pieces = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + rp.piece_off);
    const int64_t nchunks = static_cast<int64_t>(rp.npad) * (H / 8);
    const unsigned pgrid = static_cast<unsigned>((nchunks + 255) / 256);
    if (wg_dtype == MOE_F32)
      router_pieces_kernel<float><<<pgrid, 256, 0, st>>>(static_cast<const float*>(wg), pieces,
                                                        N, rp.npad, H);
    else
      router_pieces_kernel<bf16_t><<<pgrid, 256, 0, st>>>(static_cast<const bf16_t*>(wg), pieces,
                                                         N, rp.npad, H);
    dim3 grid((T + kRtRows - 1) / kRtRows, (N + 255) / 256, rp.splits);
    const int ks = rp.kchunk / 32;
    if (rp.np == 3)
      router_bf16_kernel<3><<<grid, kRtThreads, 0, st>>>(static_cast<const bf16_t*>(x), pieces,
                                                         part, T, H, N, rp.npad, ks);
    else
      router_bf16_kernel<1><<<grid, kRtThreads, 0, st>>>(static_cast<const bf16_t*>(x), pieces,
                                                         part, T, H, N, rp.npad, ks);
    return hipGetLastError();
  }
  const int kchunk = rp.kchunk;
  dim3 grid((T + 31) / 32, (N + 255) / 256, rp.splits);
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

  // logits: the K-split partials added in split order (0 + p0) + p1 + ...;
  // the partials of up to 8 splits are loaded before any is added, so their
  // memory latencies overlap
  float l[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.part + static_cast<int64_t>(t) * N + e0);
    const int64_t sstride = static_cast<int64_t>(p.T) * N / 4;  // f32x4 per split
    for (int s0 = 0; s0 < p.splits; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < p.splits) v[u] = src[(s0 + u) * sstride];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < p.splits) {
          l[0] += v[u].x;
          l[1] += v[u].y;
          l[2] += v[u].z;
          l[3] += v[u].w;
        }
    }
    *reinterpret_cast<f32x4*>(p.logits + static_cast<int64_t>(t) * N + e0) =
        f32x4{l[0], l[1], l[2], l[3]};
  }

  // softmax numerators E_e = e^(l_e - m) and their sum S, both defined
  // exactly (exp32_cw, terms under e^-64 of the largest are 0; S is the
  // pairwise sum over the 256 expert slots, empty slots 0), so the softmax
  // score E_e / S is reproducible bit for bit; S also gives the
  // log-sum-exp of the z-loss.
  float m = valid ? fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])) : -INFINITY;
  m = wave_max_f32(m);
  float ex[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
#pragma unroll
    for (int r = 0; r < 4; ++r) ex[r] = softmax_numerator(l[r], m);
  }
  const float se = wave_sum_pairwise_f32((ex[0] + ex[1]) + (ex[2] + ex[3]));
  const float lse = m + __logf(se);

  // scores and selection keys
  float s[4];
  uint32_t ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (p.score_fn == MOE_SCORE_SIGMOID) {
      s[r] = sigmoid_score(l[r]);
    } else {
      s[r] = ex[r] / se;
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
    // fused dispatch count: one integer add per selection into the token's
    // dispatch block (the sum does not depend on the order of the adds)
    if (p.block_counts)
      atomicAdd(&p.block_counts[static_cast<int64_t>(t / kDispatchTokPerBlock) * p.N + my_idx], 1);
  }
  if (lane == 0 && p.token_lse) p.token_lse[t] = lse;
}

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  route_kernel<<<(p.T + 3) / 4, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe
