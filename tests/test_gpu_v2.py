"""GPU parity of the DeepSeek-v2 routing variants ("DeepSeek MoE：从v1到v3的演进"
§DeepSeek-v2): device-limited routing (top-1 group score, a token reaches at
most topk_groups devices) and device-level token dropping (a device over its
cap drops its lowest-scored assignments), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import workloads
from gpu_common import (F32_MAXREL, check_dispatch, check_outputs, check_routing, check_stats,
                        gpu, layer_forward, make_inputs, normwise, oracle_dispatch, oracle_rows,
                        oracle_route, require_gpu, say)

pytestmark = gpu


def _route_only(wl, logits, bias):
    cfg = moe.make_cfg(wl)
    T, k = wl.T, wl.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    score = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lse = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, None, None, logits.clone(), bias, idx, gate, score, lse)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gate.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("fn", [workloads.SIGMOID, workloads.SOFTMAX])
def test_device_limited_routing_v2_shape_with_ties(fn):
    """160 experts on 8 devices, 3 kept, top-6; integer-valued logits."""
    require_gpu()
    rng = np.random.default_rng(160 + fn)
    T, N = 700, 160
    logits = rng.integers(-3, 4, size=(T, N)).astype(np.float32)
    bias = None
    if fn == workloads.SIGMOID:
        logits = logits * 0.5
        bias = (rng.integers(-2, 3, size=N) * 0.125).astype(np.float32)
    wl = workloads.V2.with_(T=T, score_fn=fn, norm_topk=0)
    say(f"device-limited routing fn={fn}")
    bt = torch.from_numpy(bias).cuda() if bias is not None else None
    idx, gate, _ = _route_only(wl, torch.from_numpy(logits).cuda(), bt)
    r = oracle_route(wl, logits, bias)
    np.testing.assert_array_equal(idx, r["topk_idx"])
    mr, _ = normwise(gate, r["topk_gate"])
    assert mr <= F32_MAXREL
    assert max(len(set(row // 20)) for row in idx) <= 3


@pytest.mark.parametrize("T,N,G,k,cap", [(3000, 32, 4, 6, None), (3000, 32, 4, 6, 2500),
                                         (257, 16, 2, 4, 100), (1, 16, 4, 2, 1), (0, 16, 4, 2, 5),
                                         (5000, 160, 8, 6, None)])
def test_permute_group_drop_matches_oracle_with_ties(T, N, G, k, cap):
    """moe_permute with device-level dropping on routings with tied scores
    (also two experts of one token with equal scores in one group); group
    candidate lists longer than one 1024-thread chunk; cap None = average."""
    require_gpu()
    rng = np.random.default_rng(T + N + k)
    idx = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    score = (rng.integers(0, 8, size=(T, k)) * 0.125).astype(np.float32)
    gc = -1 if cap is None else cap
    wl = workloads.TINY.with_(T=T, N=N, k=k, n_groups=G, topk_groups=G, group_capacity=gc)
    cfg = moe.make_cfg(wl)
    say(f"permute group drop T={T} N={N} G={G} k={k} cap={gc}")
    dev = "cuda"
    counts = torch.empty(N, dtype=torch.int32, device=dev)
    offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
    row_token = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=dev)
    inv_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    nd = torch.empty(2, dtype=torch.int32, device=dev)
    ws = moe.alloc_workspace(cfg)
    ws.fill_(0xAB)
    moe.moe_permute(cfg, torch.from_numpy(idx).to(dev), torch.from_numpy(score).to(dev), None,
                    counts, offsets, row_token[:T * k] if T else row_token[:0], inv_row,
                    n_dropped=nd, ws=ws)
    torch.cuda.synchronize()
    d = oracle_dispatch(wl, idx, score)
    np.testing.assert_array_equal(counts.cpu().numpy(), d["counts"])
    np.testing.assert_array_equal(offsets.cpu().numpy(), d["offsets"])
    M = int(d["offsets"][-1])
    np.testing.assert_array_equal(row_token.cpu().numpy()[:M], d["row_token"])
    np.testing.assert_array_equal(inv_row.cpu().numpy(), d["inv_row"])
    assert list(nd.cpu().numpy()) == [d["n_dropped"], d["n_tok_all_dropped"]]
    if cap is None and T > 100:
        assert d["n_dropped"] > 0


@pytest.mark.parametrize("fn,gc", [(workloads.SIGMOID, -1), (workloads.SIGMOID, 90),
                                   (workloads.SOFTMAX, -1)])
def test_tiny_layer_device_limited_with_group_drop(fn, gc):
    """fp32 tiny layer, 4 devices keep 2, top-1 group score, group dropping:
    every output row against the oracle at 1e-5."""
    require_gpu()
    wl = workloads.TINY.with_(T=300, group_topn=1, group_capacity=gc, score_fn=fn,
                              norm_topk=1 if fn == workloads.SIGMOID else 0,
                              bias_kind="uniform" if fn == workloads.SIGMOID else "none")
    say(f"tiny v2-style layer fn={fn} group_capacity={gc}")
    inp = make_inputs(wl)
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    assert d["n_dropped"] > 0
    check_stats(wl, aux)
    toks = list(range(wl.T))
    ref = oracle_rows(wl, inp, r, d, toks)
    mr, _ = check_outputs(wl, out, ref, toks)
    say(f"  dropped {d['n_dropped']}, max-rel {mr:.2e}")
