"""Shared helpers of the GPU parity tests: tensors <-> oracle arrays, the
normwise error measures and one-call drivers of the HIP library."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import synth, workloads

BF16_MAXREL, BF16_RELL2 = 2e-2, 5e-3   # bf16 paths vs fp32-or-better oracle
F32_MAXREL = 1e-5                      # fp32 paths
# Per-token bars: a single wrong row among thousands moves the block norms
# above very little, so every compared row must also pass on its own. bf16
# output rounding alone gives up to 2^-9 relative error per row and the bf16
# hidden activations about as much again; 1e-2 leaves a margin of ~3x over the
# worst row measured at full size (3.1e-3). fp32 paths round each output once in fp32 after fp32 sums
# of at most a few thousand terms.
BF16_ROW_RELL2, F32_ROW_RELL2 = 1e-2, 1e-4

gpu = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def typed(t: torch.Tensor) -> np.ndarray:
    """Tensor -> oracle typed array (fp32, or raw bf16 bits as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float32).numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    den_inf = np.max(np.abs(ref)) if ref.size else 0.0
    den_l2 = np.linalg.norm(ref)
    maxrel = float(np.max(np.abs(d)) / den_inf) if den_inf > 0 else float(np.max(np.abs(d), initial=0))
    rell2 = float(np.linalg.norm(d) / den_l2) if den_l2 > 0 else float(np.linalg.norm(d))
    return maxrel, rell2


def score_fn_const(wl) -> int:
    return oracle.SIGMOID if wl.score_fn == workloads.SIGMOID else oracle.SOFTMAX


def oracle_route(wl, logits_np, bias_np):
    return oracle.route(logits_np, bias_np, wl.k, wl.n_groups, wl.topk_groups, wl.group_topn,
                        score_fn_const(wl), wl.norm_topk, wl.route_scale)


def layer_forward(wl, inp, ws=None, aux=None, cfg=None):
    cfg = cfg or moe.make_cfg(wl)
    dt = torch.bfloat16 if wl.act_dtype == workloads.BF16 else torch.float32
    out = torch.empty((wl.T, wl.H), dtype=dt, device="cuda")
    if aux is None:
        aux = moe.alloc_aux(cfg)
    if ws is None:
        ws = moe.alloc_workspace(cfg)
    weights = moe.prepare_weights(cfg, {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2")})
    moe.moe_layer_forward(cfg, weights, inp["x"], inp["bias"], out, aux, ws)
    torch.cuda.synchronize()
    return out, aux


def check_routing(wl, aux, bias):
    """Bit-exact selection given the GPU's fp32 logits; gates/lse to 1e-5."""
    logits = aux["logits"].cpu().numpy()
    b = bias.cpu().numpy() if bias is not None else None
    r = oracle_route(wl, logits, b)
    got_idx = aux["topk_idx"].cpu().numpy()
    mism = np.argwhere(got_idx != r["topk_idx"])
    assert mism.size == 0, f"{len(mism)} expert-index mismatches, first at {mism[:3].tolist()}"
    # the scores (fp32 sigmoid or fp32 softmax, each defined step by step)
    # decide capacity and device-level drops: bit for bit
    np.testing.assert_array_equal(aux["topk_score"].cpu().numpy(), r["topk_score"])
    if wl.group_topn == 1 and wl.n_groups > 1:  # device-limited: fan-out <= kept devices
        gs = wl.N // wl.n_groups
        dev = got_idx // gs
        fan = np.array([len(set(row)) for row in dev])
        assert fan.max(initial=0) <= wl.topk_groups
    mr, _ = normwise(aux["topk_gate"].cpu().numpy(), r["topk_gate"])
    assert mr <= F32_MAXREL, f"gate max-rel {mr}"
    mr, _ = normwise(aux["token_lse"].cpu().numpy(), r["lse"])
    assert mr <= F32_MAXREL, f"lse max-rel {mr}"
    return r


def oracle_dispatch(wl, topk_idx, topk_score):
    gcap = workloads.group_capacity_for(wl)
    if gcap > 0:
        return oracle.dispatch_grouped(topk_idx, topk_score, wl.N, wl.n_groups, gcap)
    return oracle.dispatch(topk_idx, topk_score, wl.N, wl.capacity)


def check_dispatch(wl, aux, r):
    """Bit-exact dispatch against the oracle's dispatch of the oracle's own
    routing (indices and fp32 scores computed from the logits)."""
    d = oracle_dispatch(wl, r["topk_idx"], r["topk_score"])
    np.testing.assert_array_equal(aux["counts"].cpu().numpy(), d["counts"])
    np.testing.assert_array_equal(aux["offsets"].cpu().numpy(), d["offsets"])
    M = int(d["offsets"][-1])
    np.testing.assert_array_equal(aux["row_token"].cpu().numpy()[:M], d["row_token"])
    np.testing.assert_array_equal(aux["inv_row"].cpu().numpy(), d["inv_row"])
    nd = aux["n_dropped"].cpu().numpy()
    assert int(nd[0]) == d["n_dropped"] and int(nd[1]) == d["n_tok_all_dropped"]
    return d


def check_stats(wl, aux):
    st = oracle.load_stats(aux["logits"].cpu().numpy(), aux["counts"].cpu().numpy(), wl.k,
                           score_fn_const(wl))
    for name, ref in (("f", st["f"]), ("P", st["P"])):
        mr, _ = normwise(aux[name].cpu().numpy(), ref)
        assert mr <= F32_MAXREL, f"{name} max-rel {mr}"
    sc = aux["scalars"].cpu().numpy().astype(np.float64)
    for i, key in enumerate(("L_B", "z", "z_sq")):
        assert abs(sc[i] - st[key]) <= F32_MAXREL * max(1.0, abs(st[key])), (key, sc[i], st[key])
    return st


def oracle_workers() -> int:
    """Concurrent oracle calls: the host cores this process may use (a GPU
    box's share is 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_rows(wl, inp, r, d, tokens, workers=None):
    """Oracle layer output (fp64) for the given tokens.  Each token is one
    call of the single-threaded C oracle; independent calls run side by side
    on the host cores (ctypes releases the GIL for the C call)."""
    x = inp["x"]
    ws13 = typed(inp["ws13"]) if inp.get("ws13") is not None else None
    ws2 = typed(inp["ws2"]) if inp.get("ws2") is not None else None
    need = sorted({int(r["topk_idx"][t, j]) for t in tokens for j in range(wl.k)
                   if d["inv_row"][t, j] >= 0})
    w13 = {e: typed(inp["w13"][e]) for e in need}
    w2 = {e: typed(inp["w2"][e]) for e in need}
    xs = typed(x[list(tokens)]) if len(tokens) else None

    def one(i):
        t = tokens[i]
        sel = [int(e) if d["inv_row"][t, j] >= 0 else None
               for j, e in enumerate(r["topk_idx"][t])]
        return oracle.token_output(xs[i], [w13[e] if e is not None else None for e in sel],
                                   [w2[e] if e is not None else None for e in sel],
                                   r["topk_gate"][t], ws13, ws2, wl.n_shared, wl.I_shared, wl.I)

    n = workers or oracle_workers()
    if n == 1 or len(tokens) < 2:
        return np.stack([one(i) for i in range(len(tokens))])
    with ThreadPoolExecutor(max_workers=n) as ex:
        return np.stack(list(ex.map(one, range(len(tokens)))))


def stratified_tokens(wl, d, min_count=0, max_dropped=64, seed=0):
    """Tokens whose layer outputs reach every part of the grouped GEMM's
    tiling, for full-size parity on a sample:
      * per routed expert segment split into balanced row tiles of at most
        256 rows: the tokens of the first and the last row of every tile
        (so every partial last tile and every tile boundary);
      * per 256-row tile of the shared expert (its rows are the tokens in
        order): the first and the last token;
      * up to max_dropped tokens with a dropped slot;
      * random tokens up to min_count."""
    toks = set()
    off, rt = d["offsets"], d["row_token"]
    for e in range(wl.N):
        a, b = int(off[e]), int(off[e + 1])
        if b <= a:
            continue
        mtc = -(-(b - a) // 256)
        rpt = (-(-(b - a) // mtc) + 15) & ~15
        for m in range(mtc):
            r0 = a + m * rpt
            if r0 < b:
                toks.add(int(rt[r0]))
                toks.add(int(rt[min(r0 + rpt, b) - 1]))
    if wl.n_shared > 0:
        for r0 in range(0, wl.T, 256):
            toks.add(r0)
            toks.add(min(r0 + 255, wl.T - 1))
    dropped = np.nonzero((d["inv_row"] < 0).any(axis=1))[0][:max_dropped]
    toks.update(int(t) for t in dropped)
    if len(toks) < min(min_count, wl.T):
        rng = np.random.default_rng(seed)
        rest = np.setdiff1d(np.arange(wl.T), np.array(sorted(toks), dtype=np.int64))
        toks.update(int(t) for t in rng.choice(rest, size=min(min_count, wl.T) - len(toks),
                                               replace=False))
    return sorted(toks)


def row_rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error of each row; a zero reference row must come back
    exactly zero (error 0) or counts as infinitely wrong."""
    got = np.asarray(got, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return rel


def check_outputs(wl, out, ref_rows, tokens):
    """Normwise over the compared block, then every row on its own."""
    got = f64(out[tokens])
    mr, l2 = normwise(got, ref_rows)
    rows = row_rel_l2(got, ref_rows)
    worst = int(np.argmax(rows)) if len(rows) else 0
    row_bar = BF16_ROW_RELL2 if wl.act_dtype == workloads.BF16 else F32_ROW_RELL2
    if wl.act_dtype == workloads.BF16:
        assert mr <= BF16_MAXREL and l2 <= BF16_RELL2, f"max-rel {mr:.3e} rel-L2 {l2:.3e}"
    else:
        assert mr <= F32_MAXREL, f"max-rel {mr:.3e}"
    if len(rows):
        assert rows[worst] <= row_bar, \
            f"token {list(tokens)[worst]}: row rel-L2 {rows[worst]:.3e} > {row_bar:.0e}"
    return mr, l2


def make_inputs(wl, device="cuda"):
    return synth.make_inputs(wl, device=device)


def route_only(wl, logits, bias=None):
    """moe_route on given fp32 logits: (topk_idx, topk_gate, topk_score, token_lse) tensors."""
    cfg = moe.make_cfg(wl)
    T, k = wl.T, wl.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    score = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lse = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, None, None, logits.clone(), bias, idx, gate, score, lse)
    torch.cuda.synchronize()
    return idx, gate, score, lse


def seq_stats_gpu(wl, cu, idx, lse, logits):
    cfg = moe.make_cfg(wl)
    S = len(cu) - 1
    dev = "cuda"
    f = torch.full((S, wl.N), float("nan"), dtype=torch.float32, device=dev)
    P = torch.full((S, wl.N), float("nan"), dtype=torch.float32, device=dev)
    L = torch.full((S,), float("nan"), dtype=torch.float32, device=dev)
    Lm = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_seq_load_stats_workspace_size(cfg, S), dtype=torch.uint8, device=dev)
    ws.fill_(0xCD)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
    moe.moe_seq_load_stats(cfg, cu_t, idx, lse, logits, f, P, L, Lm, ws)
    torch.cuda.synchronize()
    return f.cpu().numpy(), P.cpu().numpy(), L.cpu().numpy(), float(Lm.cpu().numpy()[0])


def check_seq_stats(wl, cu, idx, lse, logits):
    f, P, L, Lm = seq_stats_gpu(wl, cu, idx, lse, logits)
    ref = oracle.seq_load_stats(logits.cpu().numpy(), idx.cpu().numpy(), cu, wl.k,
                                score_fn_const(wl))
    for name, got, want in (("f", f, ref["f"]), ("P", P, ref["P"]), ("L", L, ref["L"])):
        mr, _ = normwise(got, want)
        assert mr <= F32_MAXREL, f"sequence {name} max-rel {mr}"
    assert abs(Lm - ref["L_mean"]) <= F32_MAXREL * max(1.0, abs(ref["L_mean"]))
    return ref
