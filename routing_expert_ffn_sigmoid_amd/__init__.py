"""Python binding of libmoe.so, the MI355X (gfx950) DeepSeekMoE layer forward.

Argument marshalling only: every function below has the name of the C entry
point it calls (include/moe.h), takes torch tensors resident on the GPU (or
None for optional pointers), checks their dtype, shape, device and
contiguity, and passes ``data_ptr()`` plus the current HIP stream.  Every
step of the computation runs in the HIP kernels of libmoe.so; there is no
fallback.  Calls raise ``MoeError`` on a non-OK status and ``RuntimeError``
if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

from . import workloads
from .workloads import BF16, F32, SIGMOID, SOFTMAX, Workload

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

(MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
 MOE_ERR_TOO_LARGE) = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
MOE_F32, MOE_BF16 = 0, 1
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = 0, 1
STAGES = ["router_gemm", "route", "dispatch", "ffn_gate_up", "ffn_down", "combine", "stats"]
N_STAGES = len(STAGES)

EXPORTS = ["moe_workspace_size", "moe_route", "moe_permute", "moe_grouped_ffn",
           "moe_grouped_ffn_workspace_size", "moe_combine", "moe_load_stats",
           "moe_seq_load_stats", "moe_seq_load_stats_workspace_size", "moe_group_load_stats",
           "moe_pack_weights",
           "moe_bias_update", "moe_layer_forward", "moe_status_string", "moe_probe_wave_simd",
           "moe_layer_forward_noalloc"]

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


class MoeCfg(ctypes.Structure):
    _fields_ = [("T", _i32), ("H", _i32), ("N", _i32), ("k", _i32),
                ("n_groups", _i32), ("topk_groups", _i32), ("group_topn", _i32),
                ("score_fn", _i32), ("norm_topk", _i32), ("route_scale", ctypes.c_float),
                ("capacity", _i32), ("I", _i32), ("n_shared", _i32), ("I_shared", _i32),
                ("act_dtype", _i32), ("w_dtype", _i32), ("router_dtype", _i32),
                ("group_capacity", _i32), ("w_layout", _i32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_router", _vp), ("w13", _vp), ("w2", _vp), ("ws13", _vp), ("ws2", _vp)]


class MoeAux(ctypes.Structure):
    _fields_ = [("logits", _vp), ("topk_idx", _vp), ("topk_gate", _vp), ("topk_score", _vp),
                ("token_lse", _vp), ("counts", _vp), ("offsets", _vp), ("row_token", _vp),
                ("inv_row", _vp), ("n_dropped", _vp), ("f", _vp), ("P", _vp),
                ("scalars", _vp), ("stage_events", ctypes.POINTER(_vp))]


_LIB = None


def lib():
    """Load libmoe.so (built in-tree by __graft_entry__.build())."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        cfgp = ctypes.POINTER(MoeCfg)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [st]
        L.moe_workspace_size.restype = st
        L.moe_workspace_size.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route.restype = st
        L.moe_route.argtypes = [cfgp] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]
        L.moe_permute.restype = st
        L.moe_permute.argtypes = [cfgp] + [_vp] * 9 + [_vp, ctypes.c_size_t, _vp]
        L.moe_grouped_ffn.restype = st
        L.moe_grouped_ffn.argtypes = [cfgp, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                      _vp, ctypes.c_size_t, _vp]
        L.moe_grouped_ffn_workspace_size.restype = st
        L.moe_grouped_ffn_workspace_size.argtypes = [cfgp, _i32, _i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
        L.moe_combine.restype = st
        L.moe_combine.argtypes = [cfgp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_load_stats.restype = st
        L.moe_load_stats.argtypes = [cfgp] + [_vp] * 6 + [_vp, ctypes.c_size_t, _vp]
        L.moe_seq_load_stats.restype = st
        L.moe_seq_load_stats.argtypes = [cfgp, _i32] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]
        L.moe_seq_load_stats_workspace_size.restype = st
        L.moe_seq_load_stats_workspace_size.argtypes = [cfgp, _i32, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_group_load_stats.restype = st
        L.moe_group_load_stats.argtypes = [cfgp] + [_vp] * 5 + [_vp]
        L.moe_pack_weights.restype = st
        L.moe_pack_weights.argtypes = [ctypes.c_int64, _i32, _i32, _i32, _vp, _vp, _vp]
        L.moe_bias_update.restype = st
        L.moe_bias_update.argtypes = [cfgp, _vp, _vp, ctypes.c_float, _vp]
        L.moe_layer_forward.restype = st
        L.moe_layer_forward.argtypes = [cfgp, ctypes.POINTER(MoeWeights), _vp, _vp, _vp,
                                        ctypes.POINTER(MoeAux), _vp, ctypes.c_size_t, _vp]
        L.moe_layer_forward_noalloc.restype = st
        L.moe_layer_forward_noalloc.argtypes = [cfgp, ctypes.POINTER(MoeWeights), _vp, _vp, _vp,
                                                ctypes.POINTER(MoeAux), _vp]
        L.moe_probe_wave_simd.restype = st
        L.moe_probe_wave_simd.argtypes = [_i32, _vp, _vp]
        _LIB = L
    return _LIB


def status_string(code: int) -> str:
    try:
        return lib().moe_status_string(code).decode()
    except RuntimeError:
        return f"status {code}"


def _check(code: int, where: str):
    if code != MOE_OK:
        raise MoeError(code, where)


# ------------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor", shape=None):
    """data_ptr of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _tdtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_cfg(wl: Workload | None = None, **kw) -> MoeCfg:
    """MoeCfg from a workload preset, with keyword overrides."""
    fields = {}
    if wl is not None:
        for name, _ in MoeCfg._fields_:
            fields[name] = getattr(wl, name)
    fields.update(kw)
    return MoeCfg(**fields)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, name="ws"), ws.numel() * ws.element_size()


def moe_workspace_size(cfg: MoeCfg) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def alloc_workspace(cfg: MoeCfg, device="cuda"):
    torch = _torch()
    return torch.empty(moe_workspace_size(cfg), dtype=torch.uint8, device=device)


def moe_route(cfg: MoeCfg, x, w_router, logits, bias, topk_idx, topk_gate, topk_score,
              token_lse=None, ws=None, stream=None):
    torch = _torch()
    T, N, k, H = cfg.T, cfg.N, cfg.k, cfg.H
    wsp, wsb = _ws(ws)
    code = lib().moe_route(
        ctypes.byref(cfg), _ptr(x, _tdtype(cfg.act_dtype), "x", (T, H)),
        _ptr(w_router, _tdtype(cfg.router_dtype), "w_router", (N, H)),
        _ptr(logits, torch.float32, "logits", (T, N)),
        _ptr(bias, torch.float32, "bias", (N,)),
        _ptr(topk_idx, torch.int32, "topk_idx", (T, k)),
        _ptr(topk_gate, torch.float32, "topk_gate", (T, k)),
        _ptr(topk_score, torch.float32, "topk_score", (T, k)),
        _ptr(token_lse, torch.float32, "token_lse", (T,)), wsp, wsb, _stream(stream))
    _check(code, "moe_route")


def moe_permute(cfg: MoeCfg, topk_idx, topk_score, x, counts, offsets, row_token, inv_row,
                x_perm=None, n_dropped=None, ws=None, stream=None):
    torch = _torch()
    T, N, k, H = cfg.T, cfg.N, cfg.k, cfg.H
    wsp, wsb = _ws(ws)
    code = lib().moe_permute(
        ctypes.byref(cfg), _ptr(topk_idx, torch.int32, "topk_idx", (T, k)),
        _ptr(topk_score, torch.float32, "topk_score", (T, k)),
        _ptr(x, _tdtype(cfg.act_dtype), "x", (T, H)),
        _ptr(counts, torch.int32, "counts", (N,)),
        _ptr(offsets, torch.int32, "offsets", (N + 1,)),
        _ptr(row_token, torch.int32, "row_token", (T * k,)),
        _ptr(inv_row, torch.int32, "inv_row", (T, k)),
        _ptr(x_perm, _tdtype(cfg.act_dtype), "x_perm", (T * k, H)),
        _ptr(n_dropped, torch.int32, "n_dropped", (2,)), wsp, wsb, _stream(stream))
    _check(code, "moe_permute")


def moe_grouped_ffn_workspace_size(cfg: MoeCfg, max_rows: int, inter: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_grouped_ffn_workspace_size(ctypes.byref(cfg), max_rows, inter,
                                                ctypes.byref(n)),
           "moe_grouped_ffn_workspace_size")
    return n.value


def moe_grouped_ffn(cfg: MoeCfg, n_segments: int, seg_offsets, max_rows: int, inter: int, a,
                    row_index, w13, w2, y, ws, stream=None):
    torch = _torch()
    dt = _tdtype(cfg.act_dtype)
    wsp, wsb = _ws(ws)
    code = lib().moe_grouped_ffn(
        ctypes.byref(cfg), n_segments,
        _ptr(seg_offsets, torch.int32, "seg_offsets", (n_segments + 1,)), max_rows, inter,
        _ptr(a, dt, "a"), _ptr(row_index, torch.int32, "row_index"),
        _ptr(w13, _tdtype(cfg.w_dtype), "w13"), _ptr(w2, _tdtype(cfg.w_dtype), "w2"),
        _ptr(y, dt, "y"), wsp, wsb, _stream(stream))
    _check(code, "moe_grouped_ffn")


def moe_combine(cfg: MoeCfg, y_perm, inv_row, topk_gate, y_shared, out, stream=None):
    torch = _torch()
    dt = _tdtype(cfg.act_dtype)
    T, k, H = cfg.T, cfg.k, cfg.H
    code = lib().moe_combine(
        ctypes.byref(cfg), _ptr(y_perm, dt, "y_perm"), _ptr(inv_row, torch.int32, "inv_row", (T, k)),
        _ptr(topk_gate, torch.float32, "topk_gate", (T, k)),
        _ptr(y_shared, dt, "y_shared", (T, H)), _ptr(out, dt, "out", (T, H)), _stream(stream))
    _check(code, "moe_combine")


def moe_load_stats(cfg: MoeCfg, counts, token_lse, logits, f, P, scalars, ws, stream=None):
    torch = _torch()
    T, N = cfg.T, cfg.N
    wsp, wsb = _ws(ws)
    code = lib().moe_load_stats(
        ctypes.byref(cfg), _ptr(counts, torch.int32, "counts", (N,)),
        _ptr(token_lse, torch.float32, "token_lse", (T,)),
        _ptr(logits, torch.float32, "logits", (T, N)), _ptr(f, torch.float32, "f", (N,)),
        _ptr(P, torch.float32, "P", (N,)), _ptr(scalars, torch.float32, "scalars", (3,)),
        wsp, wsb, _stream(stream))
    _check(code, "moe_load_stats")


def pack_weights(w, stream=None):
    """Row-major bf16 expert weights [..., R, K] -> a new tensor of the same
    shape holding them in MOE_LAYOUT_TILED (moe_pack_weights)."""
    torch = _torch()
    if w.dtype != torch.bfloat16 or w.dim() < 2 or not w.is_contiguous():
        raise ValueError("pack_weights: contiguous bf16 tensor [..., R, K] expected")
    R, K = int(w.shape[-2]), int(w.shape[-1])
    n_mat = w.numel() // (R * K) if R * K else 0
    out = torch.empty_like(w)
    _check(lib().moe_pack_weights(n_mat, R, K, MOE_BF16, _vp(w.data_ptr()), _vp(out.data_ptr()),
                                  _stream(stream)), "moe_pack_weights")
    return out


def prepare_weights(cfg: MoeCfg, weights: dict, stream=None) -> dict:
    """The layer weights as the library reads them: the expert matrices
    (w13, w2, ws13, ws2) packed when cfg.w_layout is MOE_LAYOUT_TILED."""
    out = dict(weights)
    if cfg.w_layout == MOE_LAYOUT_TILED:
        for n in ("w13", "w2", "ws13", "ws2"):
            if out.get(n) is not None:
                out[n] = pack_weights(out[n], stream)
    return out


def moe_seq_load_stats_workspace_size(cfg: MoeCfg, n_seq: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_seq_load_stats_workspace_size(ctypes.byref(cfg), n_seq, ctypes.byref(n)),
           "moe_seq_load_stats_workspace_size")
    return n.value


def moe_seq_load_stats(cfg: MoeCfg, cu_seqlens, topk_idx, token_lse, logits, f_seq, P_seq,
                       L_seq, L_mean=None, ws=None, stream=None):
    torch = _torch()
    T, N, k = cfg.T, cfg.N, cfg.k
    S = cu_seqlens.numel() - 1
    wsp, wsb = _ws(ws)
    code = lib().moe_seq_load_stats(
        ctypes.byref(cfg), S, _ptr(cu_seqlens, torch.int32, "cu_seqlens", (S + 1,)),
        _ptr(topk_idx, torch.int32, "topk_idx", (T, k)),
        _ptr(token_lse, torch.float32, "token_lse", (T,)),
        _ptr(logits, torch.float32, "logits", (T, N)),
        _ptr(f_seq, torch.float32, "f_seq", (S, N)), _ptr(P_seq, torch.float32, "P_seq", (S, N)),
        _ptr(L_seq, torch.float32, "L_seq", (S,)), _ptr(L_mean, torch.float32, "L_mean", (1,)),
        wsp, wsb, _stream(stream))
    _check(code, "moe_seq_load_stats")


def moe_group_load_stats(cfg: MoeCfg, f, P, F_group=None, P_group=None, L_dev=None, stream=None):
    torch = _torch()
    N, G = cfg.N, cfg.n_groups
    code = lib().moe_group_load_stats(
        ctypes.byref(cfg), _ptr(f, torch.float32, "f", (N,)), _ptr(P, torch.float32, "P", (N,)),
        _ptr(F_group, torch.float32, "F_group", (G,)), _ptr(P_group, torch.float32, "P_group", (G,)),
        _ptr(L_dev, torch.float32, "L_dev", (1,)), _stream(stream))
    _check(code, "moe_group_load_stats")


def moe_bias_update(cfg: MoeCfg, counts, bias, u: float, stream=None):
    torch = _torch()
    code = lib().moe_bias_update(ctypes.byref(cfg), _ptr(counts, torch.int32, "counts", (cfg.N,)),
                                 _ptr(bias, torch.float32, "bias", (cfg.N,)), u, _stream(stream))
    _check(code, "moe_bias_update")


def moe_probe_wave_simd(n_workgroups: int, simd, stream=None):
    """simd: int32 tensor [n_workgroups, 8] on the GPU; receives the SIMD of
    each wave of large-tile-shaped workgroups."""
    torch = _torch()
    code = lib().moe_probe_wave_simd(n_workgroups, _ptr(simd, torch.int32, "simd",
                                                        (n_workgroups, 8)), _stream(stream))
    _check(code, "moe_probe_wave_simd")


AUX_FIELDS = {"logits": "f32", "topk_idx": "i32", "topk_gate": "f32", "topk_score": "f32",
              "token_lse": "f32", "counts": "i32", "offsets": "i32", "row_token": "i32",
              "inv_row": "i32", "n_dropped": "i32", "f": "f32", "P": "f32", "scalars": "f32"}


def aux_shapes(cfg: MoeCfg) -> dict:
    T, N, k = cfg.T, cfg.N, cfg.k
    return {"logits": (T, N), "topk_idx": (T, k), "topk_gate": (T, k), "topk_score": (T, k),
            "token_lse": (T,), "counts": (N,), "offsets": (N + 1,), "row_token": (T * k,),
            "inv_row": (T, k), "n_dropped": (2,), "f": (N,), "P": (N,), "scalars": (3,)}


def alloc_aux(cfg: MoeCfg, device="cuda") -> dict:
    torch = _torch()
    shapes = aux_shapes(cfg)
    return {n: torch.empty(shapes[n], dtype=torch.int32 if d == "i32" else torch.float32,
                           device=device) for n, d in AUX_FIELDS.items()}


def _layer_args(cfg: MoeCfg, weights: dict, x, bias, out, aux: dict | None, stage_events):
    torch = _torch()
    T, N, k, H, I = cfg.T, cfg.N, cfg.k, cfg.H, cfg.I
    wdt = _tdtype(cfg.w_dtype)
    ish = cfg.n_shared * cfg.I_shared
    w = MoeWeights(
        _ptr(weights["w_router"], _tdtype(cfg.router_dtype), "w_router", (N, H)),
        _ptr(weights["w13"], wdt, "w13", (N, 2 * I, H)),
        _ptr(weights["w2"], wdt, "w2", (N, H, I)),
        _ptr(weights.get("ws13"), wdt, "ws13", (2 * ish, H)),
        _ptr(weights.get("ws2"), wdt, "ws2", (H, ish)))
    shapes = aux_shapes(cfg)
    a = MoeAux()
    ev_arr = None
    if aux:
        for name, d in AUX_FIELDS.items():
            if aux.get(name) is not None:
                setattr(a, name, _ptr(aux[name], torch.int32 if d == "i32" else torch.float32,
                                      name, shapes[name]))
    if stage_events is not None:
        if len(stage_events) != N_STAGES + 1:
            raise ValueError(f"stage_events needs {N_STAGES + 1} events")
        ev_arr = (_vp * (N_STAGES + 1))(*stage_events)
        a.stage_events = ctypes.cast(ev_arr, ctypes.POINTER(_vp))
    xp = _ptr(x, _tdtype(cfg.act_dtype), "x", (T, H))
    bp = _ptr(bias, torch.float32, "bias", (N,))
    op = _ptr(out, _tdtype(cfg.act_dtype), "out", (T, H))
    return w, a, ev_arr, xp, bp, op


def moe_layer_forward(cfg: MoeCfg, weights: dict, x, bias, out, aux: dict | None, ws,
                      stage_events=None, stream=None):
    """weights: dict with w_router, w13, w2, ws13, ws2 (tensors or None).
    aux: dict of optional output tensors (see alloc_aux).  stage_events:
    optional list of N_STAGES+1 raw hipEvent_t handles (ints)."""
    w, a, ev_arr, xp, bp, op = _layer_args(cfg, weights, x, bias, out, aux, stage_events)
    wsp, wsb = _ws(ws)
    code = lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), xp, bp, op,
                                   ctypes.byref(a), wsp, wsb, _stream(stream))
    del ev_arr
    _check(code, "moe_layer_forward")


def moe_layer_forward_noalloc(cfg: MoeCfg, weights: dict, x, bias, out, aux: dict | None,
                              stage_events=None, stream=None):
    """moe_layer_forward on the library's fixed per-GPU scratch (no workspace
    argument, nothing allocated); MoeError(MOE_ERR_TOO_LARGE) beyond
    NOALLOC_SCRATCH_BYTES of workspace."""
    w, a, ev_arr, xp, bp, op = _layer_args(cfg, weights, x, bias, out, aux, stage_events)
    code = lib().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), xp, bp, op,
                                           ctypes.byref(a), _stream(stream))
    del ev_arr
    _check(code, "moe_layer_forward_noalloc")
