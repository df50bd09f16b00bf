// moe_capi.hip -- the C ABI of libmoe.so: host-side validation, workspace
// layout and the launch sequence of one DeepSeekMoE layer forward.
#include <limits.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

// Fixed device scratch of moe_layer_forward_noalloc (for callers that cannot
// allocate).  Every GPU the library runs on holds its own copy of this array
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address (one per GPU) comes from
// hipGetSymbolAddress, and only that address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

size_t a256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }
size_t esize(int dt) { return dt == MOE_BF16 ? 2 : 4; }

moe_status check_cfg(const moe_cfg* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->H <= 0 || c->N <= 0 || c->k < 0) return MOE_ERR_INVALID_ARG;
  if (c->n_groups <= 0 || c->N % c->n_groups != 0) return MOE_ERR_INVALID_ARG;
  const int gs = c->N / c->n_groups;
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_ERR_INVALID_ARG;
  if (c->k > c->topk_groups * gs) return MOE_ERR_INVALID_ARG;
  if (c->n_groups > 1 && (c->group_topn < 1 || c->group_topn > 2 || c->group_topn > gs))
    return MOE_ERR_INVALID_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID)
    return MOE_ERR_INVALID_ARG;
  if (c->norm_topk != 0 && c->norm_topk != 1) return MOE_ERR_INVALID_ARG;
  if (c->capacity < 0 || c->I <= 0 || c->n_shared < 0 || c->I_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->n_shared > 0 && c->I_shared <= 0) return MOE_ERR_INVALID_ARG;
  for (int dt : {c->act_dtype, c->w_dtype, c->router_dtype})
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(c->T) * (c->k > 0 ? c->k : 1) > INT_MAX / 2)
    return MOE_ERR_INVALID_ARG;
  // valid, but outside what the kernels implement
  if (c->N > 256 || c->N % 4 != 0 || c->k > 64 || c->n_groups > 64) return MOE_ERR_UNSUPPORTED;
  if (c->n_groups > 1 && gs % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->H % 64 != 0 || c->I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && (static_cast<long long>(c->n_shared) * c->I_shared) % 64 != 0)
    return MOE_ERR_UNSUPPORTED;
  if (c->w_layout != MOE_LAYOUT_ROWS && c->w_layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (c->group_capacity < -1) return MOE_ERR_INVALID_ARG;
  if (c->group_capacity != 0 && c->capacity > 0) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != c->w_dtype) return MOE_ERR_UNSUPPORTED;
  // bf16 expert weights are read tiled, fp32 ones row-major
  if (c->w_layout != (c->w_dtype == MOE_BF16 ? MOE_LAYOUT_TILED : MOE_LAYOUT_ROWS))
    return MOE_ERR_UNSUPPORTED;
  // dropping keys hold the token index in 24 bits
  if ((c->capacity > 0 || c->group_capacity != 0) && c->T >= (1 << 24)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The dropping policy a configuration stands for.
DropPolicy drop_policy(const moe_cfg* c) {
  DropPolicy d{};
  d.capacity = c->capacity;
  d.n_groups = c->n_groups;
  if (c->group_capacity > 0) {
    d.group_cap = c->group_capacity;
  } else if (c->group_capacity == -1) {  // average group load, rounded up
    const long long tk = static_cast<long long>(c->T) * c->k;
    d.group_cap = static_cast<int>((tk + c->n_groups - 1) / c->n_groups);
  }
  if (d.group_cap <= 0) d.group_cap = 0;  // no assignments: nothing to drop
  return d;
}

struct LayerLayout {
  size_t router, logits, idx, gate, score, lse, counts, offsets, ndrop, disp, row_token, inv_row;
  size_t h_r, h_s, y_r, y_s, stats, f, P, scalars, total;
  RouterPlan rp;
};

LayerLayout layout(const moe_cfg* c) {
  LayerLayout L{};
  const size_t T = c->T, N = c->N, k = c->k, H = c->H, es = esize(c->act_dtype);
  const size_t TK = T * k;
  const size_t Ish = static_cast<size_t>(c->n_shared) * c->I_shared;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += a256(bytes > 0 ? bytes : 1);
    return at;
  };
  L.rp = router_plan(c->T, c->H, c->N, c->act_dtype, c->router_dtype);
  L.router = take(L.rp.ws_bytes);
  L.logits = take(T * N * 4);
  L.idx = take(TK * 4);
  L.gate = take(TK * 4);
  L.score = take(TK * 4);
  L.lse = take(T * 4);
  L.counts = take(N * 4);
  L.offsets = take((N + 1) * 4);
  L.ndrop = take(2 * 4);
  L.disp = take(dispatch_ws_bytes(c->T, c->N, c->k, drop_policy(c)));
  L.row_token = take(TK * 4);
  L.inv_row = take(TK * 4);
  L.h_r = take(TK * c->I * es);
  L.h_s = take(T * Ish * es);
  L.y_r = take(TK * H * es);
  L.y_s = take(Ish > 0 ? T * H * es : 0);
  L.stats = take(stats_ws_bytes(c->T, c->N));
  L.f = take(N * 4);
  L.P = take(N * 4);
  L.scalars = take(3 * 4);
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Byte bound of an operand for buffer addressing, or 0 when it does not fit
// a 32-bit byte offset.  At most 0xFFFFFF00: the kernels drop a store or
// load by giving it the offset 0xFFFFFFF0, which then lies past every bound.
uint32_t bound32(long long rows, long long cols, size_t es) {
  const unsigned long long b = static_cast<unsigned long long>(rows) * cols * es;
  return b <= 0xFFFFFF00ull ? static_cast<uint32_t>(b) : 0u;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Arguments of a layer forward other than the workspace.
moe_status check_layer_args(const moe_cfg* cfg, const moe_weights* w, const void* x,
                            const void* out) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!x || !out || !w->w_router)) return MOE_ERR_INVALID_ARG;
  if (cfg->k > 0 && (!w->w13 || !w->w2)) return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared > 0 && (!w->ws13 || !w->ws2)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

#define MOE_TRY(expr)                                   \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return MOE_ERR_HIP;           \
  } while (0)

hipError_t record(const moe_aux* aux, int i, hipStream_t st) {
  if (aux && aux->stage_events && aux->stage_events[i])
    return hipEventRecord(static_cast<hipEvent_t>(aux->stage_events[i]), st);
  return hipSuccess;
}

// Gate/up (phase 0) and down (phase 1) over the routed segments and the
// shared expert.  h_r/h_s: intermediates; y_r/y_s: outputs.
moe_status run_ffn(const moe_cfg* c, const void* x, const int32_t* row_token,
                   const int32_t* offsets, const moe_weights* w, void* h_r, void* h_s,
                   void* y_r, void* y_s, hipStream_t st, const moe_aux* aux) {
  const int TK = c->T * c->k;
  const int Ish = c->n_shared * c->I_shared;
  const bool routed = TK > 0;
  const bool shared = c->n_shared > 0 && c->T > 0;
  const size_t es = esize(c->act_dtype);
  FfnGroup g0[2], g1[2];
  int n = 0;
  if (routed) {
    FfnGroup a{};
    a.A = x; a.lda = c->H; a.row_index = row_token; a.seg_off = offsets; a.nseg = c->N;
    a.rows = TK; a.W = w->w13; a.w_stride = 2LL * c->I * c->H; a.Out = h_r; a.ldo = c->I;
    a.K = c->H; a.n_out = c->I; a.up_off = c->I;
    a.a_bytes = bound32(c->T, c->H, es); a.w_bytes = bound32(2LL * c->I, c->H, es);
    a.o_bytes = bound32(TK, c->I, es);
    FfnGroup b{};
    b.A = h_r; b.lda = c->I; b.row_index = nullptr; b.seg_off = offsets; b.nseg = c->N;
    b.rows = TK; b.W = w->w2; b.w_stride = static_cast<int64_t>(c->H) * c->I; b.Out = y_r;
    b.ldo = c->H; b.K = c->I; b.n_out = c->H; b.up_off = 0;
    b.a_bytes = bound32(TK, c->I, es); b.w_bytes = bound32(c->H, c->I, es);
    b.o_bytes = bound32(TK, c->H, es);
    g0[n] = a;
    g1[n] = b;
    ++n;
  }
  if (shared) {
    FfnGroup a{};
    a.A = x; a.lda = c->H; a.row_index = nullptr; a.seg_off = nullptr; a.nseg = 1;
    a.rows = c->T; a.W = w->ws13; a.w_stride = 0; a.Out = h_s; a.ldo = Ish;
    a.K = c->H; a.n_out = Ish; a.up_off = Ish;
    a.a_bytes = bound32(c->T, c->H, es); a.w_bytes = bound32(2LL * Ish, c->H, es);
    a.o_bytes = bound32(c->T, Ish, es);
    FfnGroup b{};
    b.A = h_s; b.lda = Ish; b.row_index = nullptr; b.seg_off = nullptr; b.nseg = 1;
    b.rows = c->T; b.W = w->ws2; b.w_stride = 0; b.Out = y_s; b.ldo = c->H;
    b.K = Ish; b.n_out = c->H; b.up_off = 0;
    b.a_bytes = bound32(c->T, Ish, es); b.w_bytes = bound32(c->H, Ish, es);
    b.o_bytes = bound32(c->T, c->H, es);
    g0[n] = a;
    g1[n] = b;
    ++n;
  }
  MOE_TRY(record(aux, MOE_STAGE_FFN_GATE_UP, st));
  if (c->act_dtype == MOE_BF16) {
    const int hint = routed ? TK / c->N : c->T;
    if (n) MOE_TRY(launch_ffn_bf16(g0, n, 0, hint, st));
    MOE_TRY(record(aux, MOE_STAGE_FFN_DOWN, st));
    if (n) MOE_TRY(launch_ffn_bf16(g1, n, 1, hint, st));
  } else {
    for (int i = 0; i < n; ++i) MOE_TRY(launch_ffn_f32(g0[i], 0, g0[i].rows, st));
    MOE_TRY(record(aux, MOE_STAGE_FFN_DOWN, st));
    for (int i = 0; i < n; ++i) MOE_TRY(launch_ffn_f32(g1[i], 1, g1[i].rows, st));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument or configuration";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: configuration outside the implemented kernels";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch or runtime call failed";
    case MOE_ERR_TOO_LARGE:
      return "MOE_ERR_TOO_LARGE: the call needs more than the library's fixed scratch "
             "(MOE_NOALLOC_SCRATCH_BYTES) holds";
  }
  return "unknown moe_status";
}

moe_status moe_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  *bytes = layout(cfg).total;
  return MOE_OK;
}

moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router, float* logits,
                     const float* bias, int32_t* topk_idx, float* topk_gate, float* topk_score,
                     float* token_lse, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && (!logits || (cfg->k > 0 && (!topk_idx || !topk_gate || !topk_score))))
    return MOE_ERR_INVALID_ARG;
  if (x && !w_router) return MOE_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float* part = logits;
  int splits = 1;
  if (x) {
    const RouterPlan rp = router_plan(cfg->T, cfg->H, cfg->N, cfg->act_dtype, cfg->router_dtype);
    if (rp.ws_bytes > 0 && (!ws || ws_bytes < rp.ws_bytes)) return MOE_ERR_WORKSPACE;
    splits = rp.splits;
    MOE_TRY(launch_router_gemm(rp, x, cfg->act_dtype, w_router, cfg->router_dtype, logits, ws,
                               cfg->T, cfg->H, cfg->N, &part, st));
  }
  RouteParams p{};
  p.part = part; p.splits = splits; p.logits = logits; p.bias = bias; p.topk_idx = topk_idx;
  p.topk_gate = topk_gate; p.topk_score = topk_score; p.token_lse = token_lse; p.T = cfg->T;
  p.N = cfg->N; p.k = cfg->k; p.n_groups = cfg->n_groups; p.topk_groups = cfg->topk_groups;
  p.group_topn = cfg->group_topn; p.score_fn = cfg->score_fn; p.norm_topk = cfg->norm_topk;
  p.route_scale = cfg->route_scale;
  return hip_status(launch_route(p, st));
}

moe_status moe_permute(const moe_cfg* cfg, const int32_t* topk_idx, const float* topk_score,
                       const void* x, int32_t* counts, int32_t* offsets, int32_t* row_token,
                       int32_t* inv_row, void* x_perm, int32_t* n_dropped, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  const long long TK = static_cast<long long>(cfg->T) * cfg->k;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (TK > 0 && (!topk_idx || !topk_score || !row_token || !inv_row)) return MOE_ERR_INVALID_ARG;
  if (x_perm && !x) return MOE_ERR_INVALID_ARG;
  const DropPolicy dp = drop_policy(cfg);
  const size_t need = dispatch_ws_bytes(cfg->T, cfg->N, cfg->k, dp);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  DispatchWs w = dispatch_ws_carve(ws, cfg->T, cfg->N, cfg->k, dp);
  MOE_TRY(launch_dispatch(topk_idx, topk_score, cfg->T, cfg->N, cfg->k, dp, counts, offsets,
                          row_token, inv_row, n_dropped, w, st));
  if (x_perm && TK > 0)
    MOE_TRY(launch_permute(x, static_cast<int>(esize(cfg->act_dtype)), cfg->H, row_token, offsets,
                           cfg->N, static_cast<int>(TK), x_perm, st));
  return MOE_OK;
}

moe_status moe_grouped_ffn_workspace_size(const moe_cfg* cfg, int32_t max_rows, int32_t inter,
                                          size_t* bytes) {
  if (!bytes || max_rows < 0 || inter <= 0) return MOE_ERR_INVALID_ARG;
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  *bytes = a256(static_cast<size_t>(max_rows) * inter * esize(cfg->act_dtype));
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_cfg* cfg, int32_t n_segments, const int32_t* seg_offsets,
                           int32_t max_rows, int32_t inter, const void* a,
                           const int32_t* row_index, const void* w13, const void* w2, void* y,
                           void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (n_segments <= 0 || max_rows < 0 || inter <= 0) return MOE_ERR_INVALID_ARG;
  if (!seg_offsets && n_segments != 1) return MOE_ERR_INVALID_ARG;
  if (n_segments > 1000) return MOE_ERR_UNSUPPORTED;
  if (inter % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  if (!a || !w13 || !w2 || !y) return MOE_ERR_INVALID_ARG;
  size_t need = 0;
  moe_grouped_ffn_workspace_size(cfg, max_rows, inter, &need);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  FfnGroup g0{};
  g0.A = a; g0.lda = cfg->H; g0.row_index = row_index; g0.seg_off = seg_offsets;
  g0.nseg = n_segments; g0.rows = max_rows; g0.W = w13; g0.w_stride = 2LL * inter * cfg->H;
  g0.Out = ws; g0.ldo = inter; g0.K = cfg->H; g0.n_out = inter; g0.up_off = inter;
  // the gathered rows of `a` may lie anywhere below the largest row index;
  // without that bound the buffer-addressed kernel is not used
  g0.a_bytes = row_index ? 0u : bound32(max_rows, cfg->H, esize(cfg->act_dtype));
  g0.w_bytes = bound32(2LL * inter, cfg->H, esize(cfg->act_dtype));
  g0.o_bytes = bound32(max_rows, inter, esize(cfg->act_dtype));
  FfnGroup g1{};
  g1.A = ws; g1.lda = inter; g1.row_index = nullptr; g1.seg_off = seg_offsets;
  g1.nseg = n_segments; g1.rows = max_rows; g1.W = w2; g1.w_stride = static_cast<int64_t>(cfg->H) * inter;
  g1.Out = y; g1.ldo = cfg->H; g1.K = inter; g1.n_out = cfg->H; g1.up_off = 0;
  g1.a_bytes = bound32(max_rows, inter, esize(cfg->act_dtype));
  g1.w_bytes = bound32(cfg->H, inter, esize(cfg->act_dtype));
  g1.o_bytes = bound32(max_rows, cfg->H, esize(cfg->act_dtype));
  if (cfg->act_dtype == MOE_BF16) {
    const int hint = max_rows / n_segments;
    MOE_TRY(launch_ffn_bf16(&g0, 1, 0, hint, st));
    MOE_TRY(launch_ffn_bf16(&g1, 1, 1, hint, st));
  } else {
    MOE_TRY(launch_ffn_f32(g0, 0, max_rows, st));
    MOE_TRY(launch_ffn_f32(g1, 1, max_rows, st));
  }
  return MOE_OK;
}

moe_status moe_combine(const moe_cfg* cfg, const void* y_perm, const int32_t* inv_row,
                       const float* topk_gate, const void* y_shared, void* out, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (cfg->T > 0 && !out) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && cfg->k > 0 && (!y_perm || !inv_row || !topk_gate)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_perm, inv_row, topk_gate, y_shared, out, cfg->T, cfg->H,
                                   cfg->k, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

moe_status moe_load_stats(const moe_cfg* cfg, const int32_t* counts, const float* token_lse,
                          const float* logits, float* f, float* P, float* scalars, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (!counts || (cfg->T > 0 && (!token_lse || !logits))) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < stats_ws_bytes(cfg->T, cfg->N)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_stats(counts, token_lse, logits, cfg->T, cfg->N, cfg->k, cfg->score_fn,
                                 f, P, scalars, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_pack_weights(int64_t n_mat, int32_t rows, int32_t cols, int32_t dtype,
                            const void* src, void* dst, void* stream) {
  if (n_mat < 0 || rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (rows % 16 != 0 || cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (n_mat == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_INVALID_ARG;
  const uint64_t bytes = static_cast<uint64_t>(n_mat) * rows * cols * 2;
  const uint64_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlapping
  return hip_status(launch_pack_tiled(src, dst, n_mat, rows, cols, static_cast<hipStream_t>(stream)));
}

moe_status moe_seq_load_stats_workspace_size(const moe_cfg* cfg, int32_t n_seq, size_t* bytes) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (!bytes || n_seq < 0) return MOE_ERR_INVALID_ARG;
  *bytes = seq_stats_ws_bytes(cfg->T, cfg->N, n_seq);
  return MOE_OK;
}

moe_status moe_seq_load_stats(const moe_cfg* cfg, int32_t n_seq, const int32_t* cu_seqlens,
                              const int32_t* topk_idx, const float* token_lse,
                              const float* logits, float* f_seq, float* P_seq, float* L_seq,
                              float* L_mean, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (n_seq < 0) return MOE_ERR_INVALID_ARG;
  if (n_seq > 0) {
    if (!cu_seqlens || !f_seq || !P_seq || !L_seq) return MOE_ERR_INVALID_ARG;
    if (cfg->T > 0 && (!logits || (cfg->k > 0 && !topk_idx))) return MOE_ERR_INVALID_ARG;
    if (cfg->T > 0 && cfg->score_fn == MOE_SCORE_SOFTMAX && !token_lse) return MOE_ERR_INVALID_ARG;
  }
  if (!ws || ws_bytes < seq_stats_ws_bytes(cfg->T, cfg->N, n_seq)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_seq_stats(cu_seqlens, n_seq, topk_idx, token_lse, logits, cfg->T,
                                     cfg->N, cfg->k, cfg->score_fn, f_seq, P_seq, L_seq, L_mean,
                                     ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_group_load_stats(const moe_cfg* cfg, const float* f, const float* P,
                                float* F_group, float* P_group, float* L_dev, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (!f || !P) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_group_stats(f, P, cfg->N, cfg->n_groups, F_group, P_group, L_dev,
                                       static_cast<hipStream_t>(stream)));
}

moe_status moe_bias_update(const moe_cfg* cfg, const int32_t* counts, float* bias, float u,
                           void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (!counts || !bias) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(counts, bias, cfg->N, u, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_cfg* cfg, const moe_weights* w, const void* x,
                             const float* bias, void* out, const moe_aux* aux, void* ws,
                             size_t ws_bytes, void* stream) {
  moe_status s = check_layer_args(cfg, w, x, out);
  if (s != MOE_OK) return s;
  const LayerLayout L = layout(cfg);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int T = cfg->T, N = cfg->N, k = cfg->k;

  auto pick = [&](auto* user, size_t off) {
    using P = std::remove_pointer_t<decltype(user)>;
    return user ? user : at<P>(ws, off);
  };
  float* logits = pick(aux ? aux->logits : static_cast<float*>(nullptr), L.logits);
  int32_t* idx = pick(aux ? aux->topk_idx : static_cast<int32_t*>(nullptr), L.idx);
  float* gate = pick(aux ? aux->topk_gate : static_cast<float*>(nullptr), L.gate);
  float* score = pick(aux ? aux->topk_score : static_cast<float*>(nullptr), L.score);
  float* lse = pick(aux ? aux->token_lse : static_cast<float*>(nullptr), L.lse);
  int32_t* counts = pick(aux ? aux->counts : static_cast<int32_t*>(nullptr), L.counts);
  int32_t* offsets = pick(aux ? aux->offsets : static_cast<int32_t*>(nullptr), L.offsets);
  int32_t* row_token = pick(aux ? aux->row_token : static_cast<int32_t*>(nullptr), L.row_token);
  int32_t* inv_row = pick(aux ? aux->inv_row : static_cast<int32_t*>(nullptr), L.inv_row);
  int32_t* ndrop = pick(aux ? aux->n_dropped : static_cast<int32_t*>(nullptr), L.ndrop);
  float* f = pick(aux ? aux->f : static_cast<float*>(nullptr), L.f);
  float* P = pick(aux ? aux->P : static_cast<float*>(nullptr), L.P);
  float* scalars = pick(aux ? aux->scalars : static_cast<float*>(nullptr), L.scalars);

  // 1. router GEMM
  MOE_TRY(record(aux, MOE_STAGE_ROUTER_GEMM, st));
  const float* part = logits;
  MOE_TRY(launch_router_gemm(L.rp, x, cfg->act_dtype, w->w_router, cfg->router_dtype, logits,
                             at<char>(ws, L.router), T, cfg->H, N, &part, st));
  // 2. scores, group limit, top-k, gates; the route kernel also adds up the
  // per-block expert counts of dispatch (route -> dispatch fusion)
  MOE_TRY(record(aux, MOE_STAGE_ROUTE, st));
  const DropPolicy dp = drop_policy(cfg);
  DispatchWs dw = dispatch_ws_carve(at<char>(ws, L.disp), T, N, k, dp);
  MOE_TRY(launch_zero_block_counts(dw, T, N, st));
  RouteParams p{};
  p.part = part; p.splits = L.rp.splits; p.logits = logits; p.bias = bias; p.topk_idx = idx;
  p.topk_gate = gate; p.topk_score = score; p.token_lse = lse; p.T = T; p.N = N; p.k = k;
  p.n_groups = cfg->n_groups; p.topk_groups = cfg->topk_groups; p.group_topn = cfg->group_topn;
  p.score_fn = cfg->score_fn; p.norm_topk = cfg->norm_topk; p.route_scale = cfg->route_scale;
  p.block_counts = dw.block_counts;
  MOE_TRY(launch_route(p, st));
  // 3. dispatch (the row gather itself is fused into the gate/up loads)
  MOE_TRY(record(aux, MOE_STAGE_DISPATCH, st));
  MOE_TRY(launch_dispatch(idx, score, T, N, k, dp, counts, offsets, row_token, inv_row, ndrop, dw,
                          st, /*counts_ready=*/true));
  // 4. experts
  void* y_r = at<char>(ws, L.y_r);
  void* y_s = cfg->n_shared > 0 ? at<char>(ws, L.y_s) : nullptr;
  s = run_ffn(cfg, x, row_token, offsets, w, at<char>(ws, L.h_r), at<char>(ws, L.h_s), y_r, y_s,
              st, aux);
  if (s != MOE_OK) return s;
  // 5. combine
  MOE_TRY(record(aux, MOE_STAGE_COMBINE, st));
  MOE_TRY(launch_combine(y_r, inv_row, gate, y_s, out, T, cfg->H, k, cfg->act_dtype, st));
  // 6. load statistics
  MOE_TRY(record(aux, MOE_STAGE_STATS, st));
  MOE_TRY(launch_stats(counts, lse, logits, T, N, k, cfg->score_fn, f, P, scalars,
                       at<char>(ws, L.stats), st));
  MOE_TRY(record(aux, MOE_N_STAGES, st));
  return MOE_OK;
}

}  // extern "C"

namespace {

// Device address of `scratch` on each GPU, looked up once per device with
// that device current (the first no-alloc call on it).
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 256;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_cfg* cfg, const moe_weights* weights,
                                     const void* x, const float* bias, void* out,
                                     const moe_aux* aux, void* stream) {
  moe_status s = check_layer_args(cfg, weights, x, out);
  if (s != MOE_OK) return s;
  if (layout(cfg).total > kNoAllocScratchBytes) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != MOE_OK) return s;
  // the same launch sequence as moe_layer_forward, on the fixed scratch; it
  // clears every buffer it accumulates into with a kernel, so what a
  // previous call left in the scratch does not matter
  return moe_layer_forward(cfg, weights, x, bias, out, aux, ws, kNoAllocScratchBytes, stream);
}

moe_status moe_probe_wave_simd(int32_t n_workgroups, int32_t* simd, void* stream) {
  if (n_workgroups < 0 || (n_workgroups > 0 && !simd)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_wave_simd_probe(simd, n_workgroups, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
