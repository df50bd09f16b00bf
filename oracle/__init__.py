"""CPU parity oracle for one DeepSeekMoE layer forward -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
one thread, see ``moe_oracle.c``) with numpy-level helpers.  It shares no code
with the HIP library and imports nothing from it.

Typed arrays: ``np.float32`` arrays are fp32; ``np.uint16`` arrays hold raw
bfloat16 bit patterns (widened exactly inside the C code).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

F32, BF16 = 0, 1
SOFTMAX, SIGMOID = 0, 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64


class RouteCfg(ctypes.Structure):
    _fields_ = [("T", _i), ("N", _i), ("k", _i), ("n_groups", _i),
                ("topk_groups", _i), ("group_topn", _i), ("score_fn", _i),
                ("norm_topk", _i), ("route_scale", ctypes.c_double)]


def build() -> str:
    """Compile liboracle.so with the oracle's own Makefile; return its path."""
    subprocess.check_call(["make", "-s", "-C", _HERE, "liboracle.so"])
    return os.path.join(_HERE, "liboracle.so")


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            path = build()
        L = ctypes.CDLL(path)
        L.orc_sigmoid32.restype = ctypes.c_float
        L.orc_sigmoid32.argtypes = [ctypes.c_float]
        L.orc_sigmoid32_array.argtypes = [_vp, _vp, _i64]
        L.orc_softmax32.restype = _i
        L.orc_softmax32.argtypes = [_i, _vp, _vp]
        L.orc_router_logits.argtypes = [_i, _i, _i, _vp, _i, _vp, _i, _vp]
        L.orc_route.restype = _i
        L.orc_route.argtypes = [ctypes.POINTER(RouteCfg), _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp]
        L.orc_dispatch_grouped.restype = _i
        L.orc_dispatch_grouped.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp]
        L.orc_seq_load_stats.restype = _i
        L.orc_seq_load_stats.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.orc_group_load_stats.restype = _i
        L.orc_group_load_stats.argtypes = [_i, _i, _vp, _vp, _vp, _vp, _vp]
        L.orc_dispatch.restype = _i
        L.orc_dispatch.argtypes = [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp]
        L.orc_swiglu_row.argtypes = [_i, _i, _vp, _i, _vp, _vp, _i, _vp]
        L.orc_token_output.argtypes = [_i, _i, _i, _i, _i, _vp, _i, _vp, _vp,
                                       _vp, _vp, _vp, _i, _vp]
        L.orc_combine.argtypes = [_i, _i, _i, _vp, _vp, _i, _vp, _vp, _vp]
        L.orc_load_stats.argtypes = [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]
        L.orc_bias_update.argtypes = [_i, _vp, _vp, ctypes.c_float, _vp]
        _LIB = L
    return _LIB


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(_vp)


def _typed(a: np.ndarray):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"typed oracle input must be float32 or uint16(bf16 bits), got {a.dtype}")


def sigmoid32(l: np.ndarray) -> np.ndarray:
    l = np.ascontiguousarray(l, dtype=np.float32)
    out = np.empty_like(l)
    lib().orc_sigmoid32_array(_ptr(l), _ptr(out), l.size)
    return out


def softmax32(logits: np.ndarray) -> np.ndarray:
    """The fp32 softmax score of each row of logits [T, N] (N <= 256)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    if logits.ndim == 1:
        logits = logits[None, :]
    T, N = logits.shape
    out = np.empty_like(logits)
    for t in range(T):
        if lib().orc_softmax32(N, _ptr(logits[t]), _ptr(out[t])) != 0:
            raise ValueError("oracle softmax32: N must be 1..256")
    return out


def router_logits(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """fp64 logits [T,N] from x [T,H] and Wg [N,H]."""
    x = np.ascontiguousarray(x)
    wg = np.ascontiguousarray(wg)
    T, H = x.shape
    N = wg.shape[0]
    assert wg.shape[1] == H
    out = np.empty((T, N), np.float64)
    lib().orc_router_logits(T, H, N, _ptr(x), _typed(x), _ptr(wg), _typed(wg), _ptr(out))
    return out


def route(logits: np.ndarray, bias: np.ndarray | None, k: int, n_groups: int = 1,
          topk_groups: int = 1, group_topn: int = 2, score_fn: int = SIGMOID,
          norm_topk: int = 1, route_scale: float = 1.0) -> dict:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, N = logits.shape
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
    cfg = RouteCfg(T, N, k, n_groups, topk_groups, group_topn, score_fn,
                   norm_topk, route_scale)
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float64)
    score = np.empty((T, k), np.float32)
    lse = np.empty((T,), np.float64)
    kept = np.empty((T, n_groups), np.uint8)
    rc = lib().orc_route(ctypes.byref(cfg), _ptr(logits), _ptr(bias), _ptr(idx),
                         _ptr(gate), _ptr(score), _ptr(lse), _ptr(kept))
    if rc != 0:
        raise ValueError("oracle route: invalid configuration")
    return dict(topk_idx=idx, topk_gate=gate, topk_score=score, lse=lse,
                kept_groups=kept.astype(bool))


def dispatch(topk_idx: np.ndarray, topk_score: np.ndarray, N: int,
             capacity: int = 0) -> dict:
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    topk_score = np.ascontiguousarray(topk_score, dtype=np.float32)
    T, k = topk_idx.shape
    counts = np.empty((N,), np.int32)
    offsets = np.empty((N + 1,), np.int32)
    row_token = np.full((max(T * k, 1),), -1, np.int32)
    inv_row = np.empty((T, k), np.int32)
    drops = np.zeros((2,), np.int64)
    rc = lib().orc_dispatch(T, N, k, capacity, _ptr(topk_idx), _ptr(topk_score),
                            _ptr(counts), _ptr(offsets), _ptr(row_token),
                            _ptr(inv_row), _ptr(drops))
    if rc != 0:
        raise ValueError("oracle dispatch: invalid input")
    M = int(offsets[N])
    return dict(counts=counts, offsets=offsets, row_token=row_token[:M].copy(),
                inv_row=inv_row, n_dropped=int(drops[0]),
                n_tok_all_dropped=int(drops[1]))


def dispatch_grouped(topk_idx: np.ndarray, topk_score: np.ndarray, N: int, G: int,
                     group_cap: int) -> dict:
    """Dispatch with device-level token dropping (group_cap > 0 per group)."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    topk_score = np.ascontiguousarray(topk_score, dtype=np.float32)
    T, k = topk_idx.shape
    counts = np.empty((N,), np.int32)
    offsets = np.empty((N + 1,), np.int32)
    row_token = np.full((max(T * k, 1),), -1, np.int32)
    inv_row = np.empty((T, k), np.int32)
    drops = np.zeros((2,), np.int64)
    rc = lib().orc_dispatch_grouped(T, N, k, G, group_cap, _ptr(topk_idx), _ptr(topk_score),
                                    _ptr(counts), _ptr(offsets), _ptr(row_token),
                                    _ptr(inv_row), _ptr(drops))
    if rc != 0:
        raise ValueError("oracle dispatch_grouped: invalid input")
    M = int(offsets[N])
    return dict(counts=counts, offsets=offsets, row_token=row_token[:M].copy(),
                inv_row=inv_row, n_dropped=int(drops[0]),
                n_tok_all_dropped=int(drops[1]))


def swiglu_row(x_row: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    x_row = np.ascontiguousarray(x_row)
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    H = x_row.shape[0]
    I = w13.shape[0] // 2
    assert w13.shape == (2 * I, H) and w2.shape == (H, I)
    assert _typed(w13) == _typed(w2)
    y = np.empty((H,), np.float64)
    lib().orc_swiglu_row(H, I, _ptr(x_row), _typed(x_row), _ptr(w13), _ptr(w2),
                         _typed(w13), _ptr(y))
    return y


def token_output(x_row: np.ndarray, w13_sel: list, w2_sel: list, gates: np.ndarray,
                 ws13: np.ndarray | None, ws2: np.ndarray | None, n_shared: int,
                 I_sh: int, I: int) -> np.ndarray:
    """Layer output (fp64) for one token.  w13_sel[j]/w2_sel[j] are the slot-j
    expert's weights, or None for a dropped slot."""
    x_row = np.ascontiguousarray(x_row)
    H = x_row.shape[0]
    k = len(w13_sel)
    keep = [np.ascontiguousarray(a) if a is not None else None for a in w13_sel + w2_sel]
    dts = {_typed(a) for a in keep if a is not None}
    if ws13 is not None:
        ws13 = np.ascontiguousarray(ws13)
        ws2 = np.ascontiguousarray(ws2)
        dts |= {_typed(ws13), _typed(ws2)}
    assert len(dts) <= 1, "all weights must share one dtype"
    wdt = dts.pop() if dts else F32
    arr13 = (_vp * max(k, 1))(*[(a.ctypes.data if a is not None else None) for a in keep[:k]])
    arr2 = (_vp * max(k, 1))(*[(a.ctypes.data if a is not None else None) for a in keep[k:]])
    g = np.ascontiguousarray(gates, dtype=np.float64)
    out = np.empty((H,), np.float64)
    lib().orc_token_output(H, k, I, n_shared, I_sh, _ptr(x_row), _typed(x_row),
                           arr13, arr2, _ptr(g), _ptr(ws13), _ptr(ws2), wdt, _ptr(out))
    return out


def combine(y: np.ndarray, y_sh: np.ndarray | None, inv_row: np.ndarray,
            gate: np.ndarray) -> np.ndarray:
    """fp64 [T,H] = y_sh + sum of gate-weighted rows of y (dropped = -1)."""
    y = np.ascontiguousarray(y)
    inv_row = np.ascontiguousarray(inv_row, dtype=np.int32)
    T, k = inv_row.shape
    H = y.shape[1]
    if y_sh is not None:
        y_sh = np.ascontiguousarray(y_sh)
        assert y_sh.dtype == y.dtype and y_sh.shape == (T, H)
    g = np.ascontiguousarray(gate, dtype=np.float64)
    out = np.empty((T, H), np.float64)
    lib().orc_combine(T, H, k, _ptr(y), _ptr(y_sh), _typed(y), _ptr(inv_row), _ptr(g), _ptr(out))
    return out


def load_stats(logits: np.ndarray, counts: np.ndarray, k: int, score_fn: int) -> dict:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    T, N = logits.shape
    f = np.empty((N,), np.float64)
    P = np.empty((N,), np.float64)
    sc = np.empty((3,), np.float64)
    lib().orc_load_stats(T, N, k, score_fn, _ptr(logits), _ptr(counts), _ptr(f),
                         _ptr(P), _ptr(sc))
    return dict(f=f, P=P, L_B=float(sc[0]), z=float(sc[1]), z_sq=float(sc[2]))


def bias_update(counts: np.ndarray, bias: np.ndarray, u: float) -> np.ndarray:
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty_like(bias)
    lib().orc_bias_update(counts.shape[0], _ptr(counts), _ptr(bias), u, _ptr(out))
    return out


def seq_load_stats(logits: np.ndarray, topk_idx: np.ndarray, cu_seqlens, k: int,
                   score_fn: int = SIGMOID) -> dict:
    """Per-sequence f, P, L_B and their mean over non-empty sequences."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, N = logits.shape
    S = cu.size - 1
    f = np.zeros((max(S, 1), N), np.float64)
    P = np.zeros((max(S, 1), N), np.float64)
    L = np.zeros((max(S, 1),), np.float64)
    Lm = np.zeros((1,), np.float64)
    rc = lib().orc_seq_load_stats(T, N, k, score_fn, S, _ptr(cu), _ptr(topk_idx), _ptr(logits),
                                  _ptr(f), _ptr(P), _ptr(L), _ptr(Lm))
    if rc != 0:
        raise ValueError("oracle seq_load_stats: invalid input")
    return dict(f=f[:S], P=P[:S], L=L[:S], L_mean=float(Lm[0]))


def group_load_stats(f: np.ndarray, P: np.ndarray, G: int) -> dict:
    """Device-level F_g, P_g and L_dev = G * sum F_g P_g."""
    f = np.ascontiguousarray(f, dtype=np.float64)
    P = np.ascontiguousarray(P, dtype=np.float64)
    N = f.size
    Fg = np.empty((G,), np.float64)
    Pg = np.empty((G,), np.float64)
    L = np.zeros((1,), np.float64)
    rc = lib().orc_group_load_stats(N, G, _ptr(f), _ptr(P), _ptr(Fg), _ptr(Pg), _ptr(L))
    if rc != 0:
        raise ValueError("oracle group_load_stats: invalid input")
    return dict(F=Fg, P=Pg, L_dev=float(L[0]))
