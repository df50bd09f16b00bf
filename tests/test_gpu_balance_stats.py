"""GPU parity of the sequence-wise ("DeepSeek MoE：从v1到v3的演进" §DeepSeek-v3)
and device-level (§DeepSeek-v1) balance statistics against the oracle,
through the C ABI: moe_seq_load_stats and moe_group_load_stats."""
import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import workloads
from gpu_common import (F32_MAXREL, check_seq_stats, gpu, layer_forward, make_inputs, normwise,
                        require_gpu, route_only, say, score_fn_const)

pytestmark = gpu


@pytest.mark.parametrize("fn", [workloads.SIGMOID, workloads.SOFTMAX])
@pytest.mark.parametrize("N,G,keep,k", [(256, 8, 4, 8), (160, 8, 3, 6), (16, 4, 2, 4)])
def test_seq_stats_match_oracle(fn, N, G, keep, k):
    """Several sequences: empty ones, one token, a long one over many chunks,
    a ragged tail; logits N(0, 1)."""
    require_gpu()
    T = 1500
    rng = np.random.default_rng(N + k + fn)
    logits = torch.from_numpy(rng.normal(size=(T, N)).astype(np.float32)).cuda()
    wl = workloads.TINY.with_(T=T, N=N, k=k, n_groups=G, topk_groups=keep,
                              group_topn=1 if N == 160 else 2, score_fn=fn,
                              norm_topk=1 if fn == workloads.SIGMOID else 0)
    idx, _, _, lse = route_only(wl, logits)
    cu = [0, 0, 1, 700, 700, 765, 1500]
    say(f"sequence stats N={N} k={k} fn={fn} cu={cu}")
    ref = check_seq_stats(wl, cu, idx, lse, logits)
    say(f"  L per sequence {np.round(ref['L'], 4).tolist()}")


def test_seq_stats_no_sequences_and_single_sequence_equals_batch():
    require_gpu()
    wl = workloads.TINY.with_(T=300)
    inp = make_inputs(wl)
    _, aux = layer_forward(wl, inp)
    # one sequence: the batch statistics
    f, P, L, Lm = __import__("gpu_common").seq_stats_gpu(wl, [0, wl.T], aux["topk_idx"],
                                                         aux["token_lse"], aux["logits"])
    mr, _ = normwise(f[0], aux["f"].cpu().numpy())
    assert mr <= F32_MAXREL
    mr, _ = normwise(P[0], aux["P"].cpu().numpy())
    assert mr <= F32_MAXREL
    assert abs(L[0] - float(aux["scalars"][0])) <= 1e-5 and abs(Lm - L[0]) <= 1e-6
    # no sequences: only the mean is written, as 0
    cfg = moe.make_cfg(wl)
    Lm_t = torch.full((1,), 7.0, device="cuda")
    e = torch.empty((0, wl.N), device="cuda")
    ws = torch.empty(moe.moe_seq_load_stats_workspace_size(cfg, 0), dtype=torch.uint8,
                     device="cuda")
    moe.moe_seq_load_stats(cfg, torch.zeros(1, dtype=torch.int32, device="cuda"),
                           aux["topk_idx"], aux["token_lse"], aux["logits"], e, e,
                           torch.empty(0, device="cuda"), Lm_t, ws)
    torch.cuda.synchronize()
    assert float(Lm_t[0]) == 0.0


@pytest.mark.parametrize("wl_name", ["tiny", "v2"])
def test_group_stats_match_oracle(wl_name):
    require_gpu()
    wl = workloads.get(wl_name)
    if wl_name == "v2":
        wl = wl.with_(T=512)
    inp = make_inputs(wl)
    _, aux = layer_forward(wl, inp)
    cfg = moe.make_cfg(wl)
    G = wl.n_groups
    Fg = torch.empty(G, device="cuda")
    Pg = torch.empty(G, device="cuda")
    Ld = torch.empty(1, device="cuda")
    moe.moe_group_load_stats(cfg, aux["f"], aux["P"], Fg, Pg, Ld)
    torch.cuda.synchronize()
    st = oracle.load_stats(aux["logits"].cpu().numpy(), aux["counts"].cpu().numpy(), wl.k,
                           score_fn_const(wl))
    g = oracle.group_load_stats(st["f"], st["P"], G)
    for name, got, want in (("F", Fg, g["F"]), ("P", Pg, g["P"])):
        mr, _ = normwise(got.cpu().numpy(), want)
        assert mr <= F32_MAXREL, f"{name} max-rel {mr}"
    assert abs(float(Ld[0]) - g["L_dev"]) <= F32_MAXREL * max(1.0, g["L_dev"])
    say(f"{wl.name}: L_dev {float(Ld[0]):.5f} (L_B {st['L_B']:.5f})")
